"""More page layouts on the GPU: K/V kept together inside each block
(FlashInfer-style), separate K and V tensors, the x-split K layout
[num_blocks, num_heads, head_size/x, block_size, x], K-only / V-only calls,
and kernel blocks smaller than the manager's blocks (GPU).

FlashInfer-style pools are compared with the oracle directly.  The others are
compared with the oracle's value of the same tokens in a standard pool: calls
over K and over V add up (linearity over pieces), and kernel-block checksums of
a manager block add up to its checksum (pieces numbered from the request's
first token)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, gpu_blocks, log, req_tensors, to_device_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["simple", "pipelined"])
def schedule(request, monkeypatch):
    monkeypatch.setenv("KVCK_SCHEDULE", request.param)
    return request.param


def _case(name, layout, nh, d, bs, lengths, elem="bf16", layers=(0, 1, 2), start=None, extra=None):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=start, extra_blocks=extra, spare_frac=0.3)
    hp = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), elem) for _ in layers]
    return req, hp, list(layers)


def _oracle(hp, layout, layers, req, bases=None, hb=0, hc=None):
    return oracle.checksum_blocks(hp, layout, layers, bases or [hb] * len(layers), req.block_table, req.num_blocks,
                                  req.start_pos, req.num_tokens, head_begin=hb, head_count=hc)


def _call(pools, layout, layers, req, **kw):
    bt, nb, sp, nt = req_tensors(req)
    return kvck.kvck_checksum_blocks(pools, layout, layers, bt, nb, sp, nt, check=True, **kw)


@pytest.mark.parametrize("layout", ["FI_NHD", "FI_HND"])
def test_flashinfer_style_pools(layout, schedule):
    log(f"[layouts] {layout} {schedule}")
    req, hp, layers = _case(layout, layout, 8, 128, 16, [77, 130, 16, 3], extra=[0, 1, 0, 0])
    got = gpu_blocks([to_device_bits(p) for p in hp], layout, layers, req)
    want = _oracle(hp, layout, layers, req)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])
    # a head shard with global numbering
    got = gpu_blocks([to_device_bits(p) for p in hp], layout, layers, req, bases=[6] * 3, head_begin=6,
                     head_count=2)
    want = _oracle(hp, layout, layers, req, bases=[6] * 3, hb=6, hc=2)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])


@pytest.mark.parametrize("std", ["NHD", "HND"])
def test_separate_k_and_v_tensors(std, schedule):
    log(f"[layouts] separate K/V {std} {schedule}")
    req, hp, layers = _case("kv" + std, std, 4, 64, 16, [50, 17, 90], start=[0, 1, 0])
    want = _oracle(hp, std, layers, req)
    k_pools = [to_device_bits(np.ascontiguousarray(p[0])) for p in hp]
    v_pools = [to_device_bits(np.ascontiguousarray(p[1])) for p in hp]
    out = _call(k_pools, "K_" + std, layers, req)
    out = _call(v_pools, "V_" + std, layers, req, out=out, accumulate=True).cpu().numpy()
    for r, k in req.listed():
        assert int(out[r, k]) == int(want[r, k])
    # K only and V only of the stacked pool, via planes=
    pools = [to_device_bits(p) for p in hp]
    kk = _call(pools, std, layers, req, planes=(0, 1)).cpu().numpy()
    vv = _call(pools, std, layers, req, planes=(1, 1)).cpu().numpy()
    with np.errstate(over="ignore"):
        for r, k in req.listed():
            assert kk[r, k] + vv[r, k] == want[r, k]
            assert kk[r, k] != want[r, k]


@pytest.mark.parametrize("elem,x", [("bf16", 8), ("fp8", 16), ("bf16", 4), ("fp16", 16)])
def test_x_split_k_layout(elem, x, schedule):
    """K in [num_blocks, num_heads, head_size/x, block_size, x] plus V in HND
    equals the oracle on the HND pool holding the same K and V."""
    log(f"[layouts] x-split K {elem} x={x} {schedule}")
    d = 128
    req, hp, layers = _case(f"xsplit{elem}{x}", "HND", 8, d, 16, [100, 31, 2, 64], elem=elem)
    want = _oracle(hp, "HND", layers, req)
    nb = hp[0].shape[1]
    kx = [to_device_bits(np.ascontiguousarray(p[0].reshape(nb, 8, 16, d // x, x).transpose(0, 1, 3, 2, 4)))
          for p in hp]
    v_pools = [to_device_bits(np.ascontiguousarray(p[1])) for p in hp]
    out = _call(kx, "K_XSPLIT", layers, req)
    out = _call(v_pools, "V_HND", layers, req, out=out, accumulate=True).cpu().numpy()
    for r, k in req.listed():
        assert int(out[r, k]) == int(want[r, k]), (r, k)


def test_kernel_blocks_smaller_than_manager_blocks(schedule):
    """A manager block of 32 slots viewed as two kernel blocks of 16: the
    kernel-block checksums of each manager block add up to its checksum."""
    log(f"[layouts] kernel blocks {schedule}")
    req, hp, layers = _case("kblocks", "NHD", 4, 64, 32, [100, 33, 64, 5], start=[0, 1, 0, 0])
    nb = hp[0].shape[1]
    want = _oracle(hp, "NHD", layers, req)
    kernel = [to_device_bits(np.ascontiguousarray(p.reshape(2, nb * 2, 16, 4, 64))) for p in hp]
    R, M = req.num_reqs, req.max_blocks
    kt = np.full((R, 2 * M), -1, np.int32)
    for r in range(R):
        for k in range(int(req.num_blocks[r])):
            kt[r, 2 * k] = 2 * req.block_table[r, k]
            kt[r, 2 * k + 1] = 2 * req.block_table[r, k] + 1
    kreq = wl.Requests(16, req.num_tokens, req.start_pos * 2, req.num_blocks * 2, kt)
    got = gpu_blocks(kernel, "NHD", layers, kreq)
    with np.errstate(over="ignore"):
        for r, k in req.listed():
            assert got[r, 2 * k] + got[r, 2 * k + 1] == want[r, k], (r, k)


def test_copy_with_separate_k_and_x_split():
    """The fused copy on an x-split K plane: staging images hold K rows in
    plain [head][slot][row] order, and the checksums equal the K-only call."""
    log("[layouts] copy x-split")
    req, hp, layers = _case("copyx", "HND", 8, 128, 16, [70, 16], elem="bf16")
    nb = hp[0].shape[1]
    kx = [to_device_bits(np.ascontiguousarray(p[0].reshape(nb, 8, 16, 16, 8).transpose(0, 1, 3, 2, 4)))
          for p in hp]
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(kx[0], "K_XSPLIT", len(layers))
    staging = torch.zeros(int(req.num_blocks.sum()) * per, dtype=torch.uint8, device=DEV)
    got = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, kx, "K_XSPLIT", layers, bt, nbt, sp, nt, staging,
                                         check=True).cpu().numpy()
    ref = _call(kx, "K_XSPLIT", layers, req).cpu().numpy()
    img = staging.cpu().numpy().reshape(-1, len(layers), 1, 8, 16, 256)
    for e, (r, k) in enumerate(req.listed()):
        assert got[r, k] == ref[r, k]
        pos = int(req.start_pos[r]) + k
        v = min(16, max(0, int(req.num_tokens[r]) - pos * 16))
        b = int(req.block_table[r, k])
        for c in range(len(layers)):
            k_rows = hp[c][0, b].view(np.uint8).reshape(8, 16, 256)      # [head][slot][row bytes]
            assert np.array_equal(img[e, c, 0, :, :v], k_rows[:, :v])


TRANS_CASES = [
    # name, elem, heads, head_size, block_size, head_begin, head_count
    ("bf16_d128_bs16", "bf16", 8, 128, 16, 0, None),
    ("fp16_d64_bs32_heads", "fp16", 4, 64, 32, 1, 2),
    ("fp8_d128_bs16", "fp8", 4, 128, 16, 0, None),
    ("fp32_d32_bs8", "fp32", 2, 32, 8, 0, None),
    ("bf16_d72_bs64", "bf16", 2, 72, 64, 0, None),
    ("bf16_d128_bs4", "bf16", 3, 128, 4, 0, None),       # 8-byte chunks
]


@pytest.mark.parametrize("case", TRANS_CASES, ids=[c[0] for c in TRANS_CASES])
def test_element_transposed_planes(case):
    """Planes stored [num_blocks, num_heads, head_size, block_size] (one
    element index of every slot together): K_TRANS + V_TRANS equals the
    oracle on the HND pool holding the same tokens, and so does the pair of
    ROCm's paged-attention cache, x-split K + transposed V."""
    name, elem, nh, d, bs, hb, hc = case
    log(f"[layouts] transposed {name}")
    rng = np.random.default_rng(zlib.crc32(f"trans{name}".encode()))
    req, nb = wl.page_requests(rng, [3 * bs + 5, bs, 7, 2 * bs], bs, start_pos=[0, 1, 0, 0],
                               extra_blocks=[0, 0, 1, 0], spare_frac=0.3)
    layers = [0, 3, 11]
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, nh, d), elem) for _ in layers]
    n = nh - hb if hc is None else hc
    bases = [hb + 5 * i for i in range(len(layers))]
    want = _oracle(hp, "HND", layers, req, bases=bases, hb=hb, hc=n)
    kt = [to_device_bits(np.ascontiguousarray(p[0].transpose(0, 1, 3, 2))) for p in hp]
    vt = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    kw = dict(global_head_base=bases, head_begin=hb, head_count=hc)
    out = _call(kt, "K_TRANS", layers, req, **kw)
    out = _call(vt, "V_TRANS", layers, req, out=out, accumulate=True, **kw).cpu().numpy()
    for r, k in req.listed():
        assert int(out[r, k]) == int(want[r, k]), (r, k)
    es = wl.ELEM_BYTES[elem]
    x = 16 // es
    if d % x == 0:
        kx = [to_device_bits(np.ascontiguousarray(p[0].reshape(nb, nh, bs, d // x, x).transpose(0, 1, 3, 2, 4)))
              for p in hp]
        out = _call(kx, "K_XSPLIT", layers, req, **kw)
        out = _call(vt, "V_TRANS", layers, req, out=out, accumulate=True, **kw).cpu().numpy()
        for r, k in req.listed():
            assert int(out[r, k]) == int(want[r, k]), (r, k)


def test_element_transposed_limits():
    """What the element-transposed path rejects before any launch: blocks whose
    element rows are shorter than one 8-byte load, and, for the fused copy,
    blocks of more than 1024 slots (a tile row of the in-register transpose
    must fit one lane table)."""
    log("[layouts] transposed limits")
    rng = np.random.default_rng(77)
    req, nb = wl.page_requests(rng, [20], 2, spare_frac=0.5)
    hp = wl.host_random_bits(rng, wl.pool_shape("HND", nb, 2, 2, 64), "bf16")
    vt = [to_device_bits(np.ascontiguousarray(hp[1].transpose(0, 1, 3, 2)))]
    with pytest.raises(kvck.KvckError) as ei:
        _call(vt, "V_TRANS", [0], req)                  # 2 slots x 2 bytes: no 8-byte load fits
    assert ei.value.status == -2
    req, nb = wl.page_requests(rng, [3000], 2048, spare_frac=0.5)
    hp = wl.host_random_bits(rng, wl.pool_shape("HND", nb, 2048, 1, 16), "bf16")
    vt = [to_device_bits(np.ascontiguousarray(hp[1].transpose(0, 1, 3, 2)))]
    bt, nbt, sp, nt = req_tensors(req)
    staging = torch.zeros(int(req.num_blocks.sum()) * kvck.kvck_staging_bytes(vt[0], "V_TRANS", 1), dtype=torch.uint8,
                          device=DEV)
    with pytest.raises(kvck.KvckError) as ei:
        kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vt, "V_TRANS", [0], bt, nbt, sp, nt, staging)
    assert ei.value.status == -2
    # the checksum of the same blocks is supported
    got = _call(vt, "V_TRANS", [0], req).cpu().numpy()
    ref = [np.concatenate([np.zeros_like(hp[:1]), hp[1:]])]
    want = oracle.checksum_blocks(ref, "HND", [0], [0], req.block_table, req.num_blocks, req.start_pos, req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])

"""Fused copy + checksum (connector save / load) on the GPU.

Save: the checksums equal the oracle's and the staging buffer holds exactly
the specified block images (valid slots only, request order, cache order,
[plane][head][slot][row]); load: a pool paged on other block ids receives the
same valid rows, and the checksums are the same (GPU)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, log, req_tensors, to_device_bits, to_host_bits

pytestmark = pytest.mark.gpu

CASES = [
    # name, layout, elem, layers, heads, head_size, block_size, lengths, start, extra, head_begin, head_count
    ("nhd_bf16", "NHD", "bf16", [0, 1, 2], 2, 64, 16, [50, 17, 33, 1], None, [0, 1, 0, 2], 0, None),
    ("hnd_d128", "HND", "bf16", [3, 9], 8, 128, 16, [77, 130, 16], [1, 0, 0], None, 0, None),
    ("hnd_shard", "HND", "bf16", [0, 1, 2, 3, 4], 8, 128, 16, [90, 40], None, None, 2, 2),
    ("nhd_fp8_12h", "NHD", "fp8", [5], 12, 64, 16, [100, 31, 2], None, None, 0, None),
    ("mla_bs64", "MLA", "bf16", [0, 1, 60], 1, 576, 64, [130, 64, 3], None, None, 0, None),
    ("nhd_8byte_rows", "NHD", "bf16", [0, 3], 3, 4, 4, [13, 6], None, None, 0, None),
    ("nhd_bs64_fp16", "NHD", "fp16", [0, 1], 12, 64, 64, [300, 65], None, None, 0, None),
    ("nhd_fp8_shard", "NHD", "fp8", [2, 7], 6, 32, 16, [60, 21], None, [0, 1], 1, 3),
]


def _row(pool, layout, plane, b, i, h):
    if layout == "NHD":
        return pool[plane, b, i, h]
    if layout == "HND":
        return pool[plane, b, h, i]
    return pool[b, i]


def _expected_images(pools, layout, req, head_begin, head_count, bs, row_bytes):
    """uint8 [entries, caches, planes, heads, bs, row_bytes]: valid slots only, the rest 0."""
    planes = 1 if layout == "MLA" else 2
    listed = req.listed()
    img = np.zeros((len(listed), len(pools), planes, head_count, bs, row_bytes), np.uint8)
    for e, (r, k) in enumerate(listed):
        pos = int(req.start_pos[r]) + k
        v = min(bs, max(0, int(req.num_tokens[r]) - pos * bs))
        b = int(req.block_table[r, k])
        for c, p in enumerate(pools):
            for pl in range(planes):
                for hh in range(head_count):
                    for i in range(v):
                        img[e, c, pl, hh, i] = np.frombuffer(
                            np.ascontiguousarray(_row(p, layout, pl, b, i, head_begin + hh)).tobytes(), np.uint8)
    return img


@pytest.fixture(params=["1", "2", "1-merge0", "2-merge1", "1-grouped", "2-grouped"])
def copy_buffers(request, monkeypatch):
    """Run the test with one unit buffer per wave and with two
    (KVCK_COPY_BUFFERS), under the library's choice of reading a slot's heads as
    one row, with that choice forced off or on (KVCK_MERGE_HEADS), and with
    positions visited grouped by block id instead of in listing order (forced
    with KVCK_COPY_ORDER: these small pools take listing order by default)."""
    buffers, *flags = request.param.split("-")
    monkeypatch.setenv("KVCK_COPY_BUFFERS", buffers)
    for f in flags:
        if f.startswith("merge"):
            monkeypatch.setenv("KVCK_MERGE_HEADS", f[len("merge"):])
        elif f == "grouped":
            monkeypatch.setenv("KVCK_COPY_ORDER", "grouped")
    return request.param


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_copy_save_and_load(case, copy_buffers):
    name, layout, elem, layers, nh, d, bs, lengths, start, extra, hb, hc = case
    log(f"[copy] {name} buffers={copy_buffers}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=start, extra_blocks=extra, spare_frac=0.3)
    shape = wl.pool_shape(layout, nb, bs, nh, d)
    hp = [wl.host_random_bits(rng, shape, elem) for _ in layers]
    pools = [to_device_bits(p) for p in hp]
    n_heads = (nh - hb) if hc is None else hc
    bases = [hb + 3] * len(layers)
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(pools[0], layout, len(layers), n_heads)
    n_entries = int(req.num_blocks.sum())
    staging = torch.zeros(n_entries * per, dtype=torch.uint8, device=DEV)
    got = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, layout, layers, bt, nbt, sp, nt, staging,
                                         global_head_base=bases, head_begin=hb, head_count=hc, check=True)
    got = got.cpu().numpy()
    want = oracle.checksum_blocks(hp, layout, layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=hb, head_count=n_heads)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    row_bytes = d * wl.ELEM_BYTES[elem]
    exp = _expected_images(hp, layout, req, hb, n_heads, bs, row_bytes)
    assert np.array_equal(staging.cpu().numpy().reshape(exp.shape), exp)

    # load into a pool paged on a different permutation of block ids
    req2, _ = wl.page_requests(np.random.default_rng(99), lengths, bs, pool_blocks=nb, start_pos=start,
                               extra_blocks=extra)
    dst_h = [np.zeros(shape, wl.HOST_BITS[elem]) for _ in layers]
    dst = [to_device_bits(p) for p in dst_h]
    bt2, nbt2, sp2, nt2 = req_tensors(req2)
    got2 = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, dst, layout, layers, bt2, nbt2, sp2, nt2, staging,
                                          global_head_base=bases, head_begin=hb, head_count=hc, check=True)
    got2 = got2.cpu().numpy()
    for r, k in req.listed():
        assert got2[r, k] == got[r, k], (r, k)
    # the destination holds the source rows at the valid slots, zeros elsewhere
    dst_back = [to_host_bits(t) for t in dst]
    assert np.array_equal(_expected_images(dst_back, layout, req2, hb, n_heads, bs, row_bytes), exp)
    again = kvck.kvck_checksum_blocks(dst, layout, layers, bt2, nbt2, sp2, nt2, global_head_base=bases,
                                      head_begin=hb, head_count=hc, check=True).cpu().numpy()
    for r, k in req.listed():
        assert again[r, k] == got[r, k]


def test_copy_staging_full_is_flagged():
    log("[copy] staging full")
    rng = np.random.default_rng(5)
    req, nb = wl.page_requests(rng, [40, 40], 16, spare_frac=0.5)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16"))]
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(pools[0], "NHD", 1)
    staging = torch.zeros(3 * per, dtype=torch.uint8, device=DEV)     # 6 listed positions, room for 3
    with pytest.raises(kvck.KvckDeviceError) as ei:
        kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, "NHD", [0], bt, nbt, sp, nt, staging, check=True)
    assert ei.value.flags & kvck.KVCK_FLAG_STAGING_FULL


def test_copy_many_caches(copy_buffers):
    """More caches than one argument block: several launches, image offsets by global cache index."""
    log("[copy] 70 caches")
    rng = np.random.default_rng(6)
    req, nb = wl.page_requests(rng, [40, 9], 16, spare_frac=0.5)
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 2, 16), "bf16") for _ in range(70)]
    pools = [to_device_bits(p) for p in hp]
    layers = list(range(70))
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(pools[0], "HND", 70)
    staging = torch.zeros(int(req.num_blocks.sum()) * per, dtype=torch.uint8, device=DEV)
    got = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, "HND", layers, bt, nbt, sp, nt, staging,
                                         check=True).cpu().numpy()
    want = oracle.checksum_blocks(hp, "HND", layers, [0] * 70, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])
    exp = _expected_images(hp, "HND", req, 0, 2, 16, 32)
    assert np.array_equal(staging.cpu().numpy().reshape(exp.shape), exp)


TRANS_CASES = [
    # name, elem, heads, head_size, block_size, lengths, start, head_begin, head_count
    ("bf16_d128_bs16", "bf16", 4, 128, 16, [50, 17, 33, 16], [0, 1, 0, 0], 0, None),
    ("fp8_d64_bs32", "fp8", 3, 64, 32, [70, 5, 64], None, 1, 2),
    ("fp32_d32_bs8", "fp32", 2, 32, 8, [21, 9, 8], [0, 2, 0], 0, None),
    ("bf16_d256_bs64", "bf16", 2, 256, 64, [130, 64, 3], None, 0, None),   # two element-row groups
    ("bf16_d64_bs4", "bf16", 3, 64, 4, [13, 6, 4], None, 1, None),         # 8-byte chunks
    ("fp8_d32_bs8", "fp8", 2, 32, 8, [20, 3, 9], [1, 0, 0], 0, None),       # 8-byte chunks of 8 slots
    ("fp32_d8_bs2", "fp32", 5, 8, 2, [7, 2, 1], None, 2, 3),                 # 8-byte chunks of 2 slots
    ("bf16_d576_bs128", "bf16", 1, 576, 128, [300, 128, 5], None, 0, None),  # several groups either way
    ("fp8_d128_bs256", "fp8", 2, 128, 256, [600, 17], None, 1, 1),
]


@pytest.mark.parametrize("transpose", ["auto", "regs", "lds"])
@pytest.mark.parametrize("case", TRANS_CASES, ids=[c[0] for c in TRANS_CASES])
def test_copy_element_transposed_planes(case, transpose, monkeypatch):
    """Fused save / load of planes stored [num_blocks, num_heads, head_size,
    block_size] (ROCm's V layout): the staging image and checksums equal those
    of the same tokens saved from an HND V plane (and the oracle's), and a load
    writes exactly the valid elements of a pool paged on other ids."""
    name, elem, nh, d, bs, lengths, start, hb, hc = case
    if transpose != "auto":
        monkeypatch.setenv("KVCK_TCOPY", transpose)   # the transpose in registers or through LDS
    log(f"[copy] transposed {name} {transpose}")
    rng = np.random.default_rng(zlib.crc32(f"tcopy{name}".encode()))
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=start, extra_blocks=[1] * len(lengths), spare_frac=0.3)
    layers = [0, 5, 9]
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, nh, d), elem) for _ in layers]
    n_heads = (nh - hb) if hc is None else hc
    bases = [hb + 2 * i for i in range(len(layers))]
    kw = dict(global_head_base=bases, head_begin=hb, head_count=hc, check=True)
    vt = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    vh = [to_device_bits(np.ascontiguousarray(p[1])) for p in hp]
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(vt[0], "V_TRANS", len(layers), n_heads)
    assert per == kvck.kvck_staging_bytes(vh[0], "V_HND", len(layers), n_heads)
    n_entries = int(req.num_blocks.sum())
    st_t = torch.zeros(n_entries * per, dtype=torch.uint8, device=DEV)
    st_h = torch.zeros(n_entries * per, dtype=torch.uint8, device=DEV)
    got_t = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vt, "V_TRANS", layers, bt, nbt, sp, nt, st_t,
                                           **kw).cpu().numpy()
    got_h = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vh, "V_HND", layers, bt, nbt, sp, nt, st_h,
                                           **kw).cpu().numpy()
    # a V-only partial is the checksum of the pool with its K plane zeroed
    ref = [np.concatenate([np.zeros_like(p[:1]), p[1:]]) for p in hp]
    want = oracle.checksum_blocks(ref, "HND", layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=hb, head_count=n_heads)
    for r, k in req.listed():
        assert int(got_t[r, k]) == int(want[r, k]) == int(got_h[r, k]), (r, k)
    row_bytes = d * wl.ELEM_BYTES[elem]
    exp = _expected_images(hp, "HND", req, hb, n_heads, bs, row_bytes)[:, :, 1:2]   # the V plane's images
    assert np.array_equal(st_t.cpu().numpy().reshape(exp.shape), exp)
    assert np.array_equal(st_h.cpu().numpy(), st_t.cpu().numpy())

    # load into an empty transposed pool paged on other ids
    req2, _ = wl.page_requests(np.random.default_rng(7), lengths, bs, pool_blocks=nb, start_pos=start,
                               extra_blocks=[1] * len(lengths))
    dst = [torch.zeros_like(t) for t in vt]
    bt2, nbt2, sp2, nt2 = req_tensors(req2)
    got2 = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, dst, "V_TRANS", layers, bt2, nbt2, sp2, nt2, st_t,
                                          **kw).cpu().numpy()
    for r, k in req.listed():
        assert got2[r, k] == got_t[r, k], (r, k)
    # back in HND form: the valid rows of every listed position, and nothing else written
    back = [to_host_bits(t).transpose(0, 1, 3, 2) for t in dst]
    back_hnd = [np.stack([np.zeros_like(b), b]) for b in back]
    assert np.array_equal(_expected_images(back_hnd, "HND", req2, hb, n_heads, bs, row_bytes)[:, :, 1:2], exp)
    assert sum(int(np.count_nonzero(np.ascontiguousarray(b).view(np.uint8))) for b in back) == int(np.count_nonzero(
        _expected_images(back_hnd, "HND", req2, hb, n_heads, bs, row_bytes)))   # bytes on both sides


def test_copy_element_transposed_many_caches():
    """Transposed V planes over more caches than one argument block (several launches):
    the staging bytes and checksums equal those of the HND V planes holding the same tokens."""
    log("[copy] transposed, 70 caches")
    rng = np.random.default_rng(8)
    req, nb = wl.page_requests(rng, [40, 9, 23], 16, spare_frac=0.5)
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 2, 64), "bf16") for _ in range(70)]
    vt = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    vh = [to_device_bits(np.ascontiguousarray(p[1])) for p in hp]
    layers = list(range(70))
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(vt[0], "V_TRANS", 70)
    st_t = torch.zeros(int(req.num_blocks.sum()) * per, dtype=torch.uint8, device=DEV)
    st_h = torch.zeros_like(st_t)
    got_t = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vt, "V_TRANS", layers, bt, nbt, sp, nt, st_t,
                                           check=True).cpu().numpy()
    got_h = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vh, "V_HND", layers, bt, nbt, sp, nt, st_h,
                                           check=True).cpu().numpy()
    assert np.array_equal(st_t.cpu().numpy(), st_h.cpu().numpy())
    ref = [np.concatenate([np.zeros_like(p[:1]), p[1:]]) for p in hp]
    want = oracle.checksum_blocks(ref, "HND", layers, [0] * 70, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got_t[r, k]) == int(got_h[r, k]) == int(want[r, k]), (r, k)


def test_copy_order_over_a_large_pool(monkeypatch):
    """Visiting positions grouped by block id over a pool of more than 32768
    blocks (several ids per bucket), with ids at both ends of the pool and an
    id past the pool at a position with valid slots:
    save and load give the same staging bytes, destination pool, checksums
    and error bits as listing order, and the checksums equal the oracle's
    (the bad id's position contributes nothing and is flagged)."""
    log("[copy] visiting order, large pool")
    rng = np.random.default_rng(61)
    nb_pool = 70001
    lengths = rng.integers(1, 65, size=300)
    req, nb = wl.page_requests(rng, lengths, 16, pool_blocks=nb_pool)
    tab = req.block_table
    tab[0, 0] = 0
    tab[1, 0] = nb_pool - 1
    tab[4, 0] = nb_pool                             # past the pool, valid slots: flagged, contributes 0
    layers = [1, 2]
    hp = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 16), "bf16") for _ in layers]
    pools = [to_device_bits(p) for p in hp]
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(pools[0], "NHD", len(layers))
    n_entries = int(req.num_blocks.sum())
    res = {}
    for order in ("grouped", "listing"):
        monkeypatch.setenv("KVCK_COPY_ORDER", order)
        staging = torch.zeros(n_entries * per, dtype=torch.uint8, device=DEV)
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        saved = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, "NHD", layers, bt, nbt, sp, nt, staging,
                                               error_flags=flags)
        dst = [torch.zeros_like(p) for p in pools]
        loaded = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, dst, "NHD", layers, bt, nbt, sp, nt, staging,
                                                error_flags=flags)
        torch.cuda.synchronize()
        res[order] = (saved.cpu().numpy().copy(), loaded.cpu().numpy().copy(), staging.cpu(), [d.cpu() for d in dst],
                      int(flags.item()))
    a, b = res["grouped"], res["listing"]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert torch.equal(a[2], b[2]) and all(torch.equal(x, y) for x, y in zip(a[3], b[3]))
    assert a[4] == b[4] == kvck.KVCK_FLAG_BAD_BLOCK_ID
    good = tab.copy()
    good[4, 0] = 0
    want = oracle.checksum_blocks(hp, "NHD", layers, [0, 0], good, req.num_blocks, req.start_pos, req.num_tokens)
    for r, k in req.listed():
        expect = 0 if (r, k) == (4, 0) else int(want[r, k])
        assert int(a[0][r, k]) == expect == int(a[1][r, k]), (r, k)

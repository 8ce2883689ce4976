"""Seeded sweep of the fused copy + checksum (connector save / load) over small
random configurations (GPU).

Save: checksums equal the oracle's and the staging buffer holds exactly the
valid rows of each listed position ([plane][head][slot][row] per cache, in
request and cache order).  Load into a pool paged on other block ids: the
valid rows land there, everything else stays zero, and the checksums repeat.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, log, req_tensors, to_device_bits, to_host_bits

pytestmark = pytest.mark.gpu

LAYOUTS = ["NHD", "HND", "FI_NHD", "FI_HND", "MLA"]


def _case(i):
    rng = np.random.default_rng(zlib.crc32(f"copysweep{i}".encode()))
    layout = LAYOUTS[i % len(LAYOUTS)]
    elem = ["fp8", "bf16", "fp32"][int(rng.integers(0, 3))]
    es = wl.ELEM_BYTES[elem]
    heads = 1 if layout == "MLA" else int(rng.integers(1, 9))
    unit = 8 // es
    d = unit * int(rng.integers(1, 40))
    bs = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    layers = sorted(int(x) << (int(x) % 17) for x in rng.choice(100, size=int(rng.integers(1, 4)), replace=False))
    n_req = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(0, 3 * bs + 20, size=n_req)]
    start = [int(x) for x in rng.integers(0, 2, size=n_req)]
    extra = [int(x) for x in rng.integers(0, 2, size=n_req)]
    hb = int(rng.integers(0, heads))
    hc = int(rng.integers(1, heads - hb + 1))
    buffers = ["1", "2"][int(rng.integers(0, 2))]
    merge = [None, "0", "1"][int(rng.integers(0, 3))]   # a slot's heads read as one row: auto, off, on
    order = ["listing", "grouped"][i % 2]               # positions in listing order or grouped by block id
    return dict(i=i, layout=layout, elem=elem, heads=heads, d=d, bs=bs, layers=layers, lengths=lengths,
                start=start, extra=extra, hb=hb, hc=hc, buffers=buffers, merge=merge, order=order)


CASES = [_case(i) for i in range(120)]


def _ids(c):
    return (f"{c['i']}-{c['layout']}-{c['elem']}-h{c['heads']}-d{c['d']}-bs{c['bs']}-b{c['buffers']}"
            f"-m{c['merge'] or 'auto'}-{c['order']}")


def _rows(pool, layout, pl, b, v, hb, n):
    """(n heads, v slots, row) of block b, plane pl."""
    if layout == "NHD":
        return np.swapaxes(pool[pl, b, :v, hb:hb + n], 0, 1)
    if layout == "HND":
        return pool[pl, b, hb:hb + n, :v]
    if layout == "FI_NHD":
        return np.swapaxes(pool[b, pl, :v, hb:hb + n], 0, 1)
    if layout == "FI_HND":
        return pool[b, pl, hb:hb + n, :v]
    return pool[b, :v][None]


def _images(pools, layout, req, hb, n, bs, row_bytes):
    planes = 1 if layout == "MLA" else 2
    listed = req.listed()
    img = np.zeros((len(listed), len(pools), planes, n, bs, row_bytes), np.uint8)
    for e, (r, k) in enumerate(listed):
        v = min(bs, max(0, int(req.num_tokens[r]) - (int(req.start_pos[r]) + k) * bs))
        if v == 0:
            continue
        b = int(req.block_table[r, k])
        for c, p in enumerate(pools):
            for pl in range(planes):
                rows = np.ascontiguousarray(_rows(p, layout, pl, b, v, hb, n))
                img[e, c, pl, :, :v] = rows.view(np.uint8).reshape(n, v, row_bytes)
    return img


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_copy_sweep_case(case, monkeypatch):
    monkeypatch.setenv("KVCK_COPY_BUFFERS", case["buffers"])
    monkeypatch.setenv("KVCK_COPY_ORDER", case["order"])
    if case["merge"] is not None:
        monkeypatch.setenv("KVCK_MERGE_HEADS", case["merge"])
    log(f"[copy sweep] {_ids(case)} heads {case['hb']}+{case['hc']}")
    rng = np.random.default_rng(2000 + case["i"])
    layout, bs, nh, d, layers = case["layout"], case["bs"], case["heads"], case["d"], case["layers"]
    hb, hc = case["hb"], case["hc"]
    req, nb = wl.page_requests(rng, case["lengths"], bs, start_pos=case["start"], extra_blocks=case["extra"],
                               spare_frac=0.3)
    shape = wl.pool_shape(layout, nb, bs, nh, d)
    hp = [wl.host_random_bits(rng, shape, case["elem"]) for _ in layers]
    pools = [to_device_bits(p) for p in hp]
    bases = [hb + 7] * len(layers)
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(pools[0], layout, len(layers), hc)
    staging = torch.zeros(max(1, int(req.num_blocks.sum())) * per, dtype=torch.uint8, device=DEV)
    got = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, layout, layers, bt, nbt, sp, nt, staging,
                                         global_head_base=bases, head_begin=hb, head_count=hc,
                                         check=True).cpu().numpy()
    want = oracle.checksum_blocks(hp, layout, layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=hb, head_count=hc)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), ("save", r, k)
    row_bytes = d * wl.ELEM_BYTES[case["elem"]]
    exp = _images(hp, layout, req, hb, hc, bs, row_bytes)
    n_img = exp.size
    assert np.array_equal(staging.cpu().numpy()[:n_img].reshape(exp.shape), exp)

    req2, _ = wl.page_requests(np.random.default_rng(3000 + case["i"]), case["lengths"], bs, pool_blocks=nb,
                               start_pos=case["start"], extra_blocks=case["extra"])
    dst = [to_device_bits(np.zeros(shape, wl.HOST_BITS[case["elem"]])) for _ in layers]
    bt2, nbt2, sp2, nt2 = req_tensors(req2)
    got2 = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, dst, layout, layers, bt2, nbt2, sp2, nt2, staging,
                                          global_head_base=bases, head_begin=hb, head_count=hc,
                                          check=True).cpu().numpy()
    for r, k in req.listed():
        assert got2[r, k] == got[r, k], ("load", r, k)
    back = [to_host_bits(t) for t in dst]
    assert np.array_equal(_images(back, layout, req2, hb, hc, bs, row_bytes), exp)
    # nothing but the loaded rows was written
    total = sum(int(np.count_nonzero(b.view(np.uint8))) for b in back)
    assert total == int(np.count_nonzero(exp))


def _tcase(i):
    rng = np.random.default_rng(zlib.crc32(f"tcopysweep{i}".encode()))
    elem = ["fp8", "bf16", "fp32"][int(rng.integers(0, 3))]
    es = wl.ELEM_BYTES[elem]
    heads = int(rng.integers(1, 6))
    d = (8 // es) * int(rng.integers(1, 33))                     # rows of whole 8-byte pieces
    bs = int(rng.choice([b for b in (1, 2, 4, 8, 16, 32, 64) if (b * es) % 8 == 0]))
    layers = sorted(int(x) << (int(x) % 17) for x in rng.choice(100, size=int(rng.integers(1, 4)), replace=False))
    n_req = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(0, 3 * bs + 20, size=n_req)]
    start = [int(x) for x in rng.integers(0, 2, size=n_req)]
    hb = int(rng.integers(0, heads))
    hc = int(rng.integers(1, heads - hb + 1))
    transpose = ["regs", "lds"][int(rng.integers(0, 2))]
    return dict(i=i, elem=elem, heads=heads, d=d, bs=bs, layers=layers, lengths=lengths, start=start, hb=hb, hc=hc,
                transpose=transpose)


TCASES = [_tcase(i) for i in range(72)]


@pytest.mark.parametrize("case", TCASES,
                         ids=lambda c: f"{c['i']}-{c['elem']}-h{c['heads']}-d{c['d']}-bs{c['bs']}-{c['transpose']}")
def test_copy_sweep_element_transposed(case, monkeypatch):
    """Element-transposed V planes: save gives the V_HND save's staging bytes and checksums,
    a load into a pool paged on other ids repeats them and writes only the valid elements
    (transpose in registers or through LDS)."""
    monkeypatch.setenv("KVCK_TCOPY", case["transpose"])
    log(f"[copy sweep] transposed {case}")
    rng = np.random.default_rng(5000 + case["i"])
    bs, nh, d, hb, hc = case["bs"], case["heads"], case["d"], case["hb"], case["hc"]
    req, nb = wl.page_requests(rng, case["lengths"], bs, start_pos=case["start"], spare_frac=0.3)
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, nh, d), case["elem"]) for _ in case["layers"]]
    vt = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    vh = [to_device_bits(np.ascontiguousarray(p[1])) for p in hp]
    bases = [hb + 1] * len(hp)
    kw = dict(global_head_base=bases, head_begin=hb, head_count=hc, check=True)
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(vt[0], "V_TRANS", len(hp), hc)
    n = max(1, int(req.num_blocks.sum()))
    st_t = torch.zeros(n * per, dtype=torch.uint8, device=DEV)
    st_h = torch.zeros(n * per, dtype=torch.uint8, device=DEV)
    got_t = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vt, "V_TRANS", case["layers"], bt, nbt, sp, nt,
                                           st_t, **kw).cpu().numpy()
    got_h = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, vh, "V_HND", case["layers"], bt, nbt, sp, nt,
                                           st_h, **kw).cpu().numpy()
    ref = [np.concatenate([np.zeros_like(p[:1]), p[1:]]) for p in hp]
    want = oracle.checksum_blocks(ref, "HND", case["layers"], bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=hb, head_count=hc)
    for r, k in req.listed():
        assert int(got_t[r, k]) == int(want[r, k]) == int(got_h[r, k]), (r, k)
    assert np.array_equal(st_t.cpu().numpy(), st_h.cpu().numpy())
    req2, _ = wl.page_requests(np.random.default_rng(6000 + case["i"]), case["lengths"], bs, pool_blocks=nb,
                               start_pos=case["start"])
    dst = [torch.zeros_like(t) for t in vt]
    dsth = [torch.zeros_like(t) for t in vh]
    bt2, nbt2, sp2, nt2 = req_tensors(req2)
    got2 = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, dst, "V_TRANS", case["layers"], bt2, nbt2, sp2, nt2,
                                          st_t, **kw).cpu().numpy()
    kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, dsth, "V_HND", case["layers"], bt2, nbt2, sp2, nt2, st_h,
                                   **kw)
    for r, k in req.listed():
        assert got2[r, k] == got_t[r, k], (r, k)
    # the transposed pool holds exactly what the HND load wrote, element for element
    for a, b in zip(dst, dsth):
        assert np.array_equal(to_host_bits(a).transpose(0, 1, 3, 2), to_host_bits(b))

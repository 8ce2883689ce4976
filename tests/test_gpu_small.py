"""HIP path == oracle, element by element, on small seeded inputs (GPU).

Sizes the oracle finishes in seconds that still span several lane tables,
several head batches and ragged tails; plus edge cases: empty batches,
positions past the last token, bad block ids and requests, accumulate,
several launches of caches, the 8-byte load path, streams, determinism.
"""

import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import (DEV, SENTINEL, assert_match, assert_unlisted_untouched, gpu_blocks, log, oracle_at,
                         req_tensors, sample_positions, to_device_bits, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["auto", "simple", "pipelined", "auto-compact"])
def schedule(request, monkeypatch):
    """Run the test under the library's own choices, under each main-pass
    schedule forced (KVCK_SCHEDULE), and with every call's positions listed by
    the plan launch first (KVCK_PLAN=compact) instead of small calls planning in
    place."""
    sched, _, plan = request.param.partition("-")
    if sched != "auto":
        monkeypatch.setenv("KVCK_SCHEDULE", sched)
    if plan:
        monkeypatch.setenv("KVCK_PLAN", plan)
    return request.param


CASES = [
    # name, layout, elem, layers, heads, head_size, block_size, lengths, extra
    ("nhd_bf16", "NHD", "bf16", [0, 1, 2], 2, 64, 16, [50, 17, 33, 1, 64], None),
    ("hnd_bf16_d128", "HND", "bf16", [0, 5, 31], 8, 128, 16, [77, 130, 16, 5], None),
    ("nhd_fp16_12h", "NHD", "fp16", [3, 4], 12, 64, 16, [100, 31, 2], [0, 2, 1]),
    ("hnd_fp16_12h", "HND", "fp16", [7], 12, 64, 16, [100, 31, 2], None),
    ("nhd_bs64", "NHD", "fp16", [0, 1], 12, 64, 64, [300, 65, 63], None),
    ("nhd_fp8", "NHD", "fp8", [0, 11], 12, 64, 16, [90, 7], None),
    ("nhd_fp8_bs64", "NHD", "fp8", [2], 12, 64, 64, [200, 64], None),
    ("mla_bs64", "MLA", "bf16", [0, 1, 60], 1, 576, 64, [130, 64, 3], None),
    ("mla_bs16", "MLA", "bf16", [9, 10], 1, 576, 16, [70, 16], None),
    ("hnd_bs1", "HND", "bf16", [1, 2], 3, 16, 1, [5, 2], None),
    ("nhd_bs3_odd", "NHD", "fp32", [4], 5, 12, 3, [10, 4, 9], None),
    ("nhd_8byte_rows", "NHD", "bf16", [0, 3], 3, 4, 4, [13, 6], None),
    ("hnd_big_heads", "HND", "bf16", [2], 32, 128, 16, [40], None),
]


def _host_case(seed, layout, elem, layers, nh, d, bs, lengths, extra, start=None):
    rng = np.random.default_rng(seed)
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=start, extra_blocks=extra, spare_frac=0.3)
    shape = wl.pool_shape(layout, nb, bs, nh, d)
    pools = [wl.host_random_bits(rng, shape, elem) for _ in layers]
    return req, pools


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parity_small(case, schedule):
    name, layout, elem, layers, nh, d, bs, lengths, extra = case
    log(f"[parity_small] {name} {schedule}")
    req, hpools = _host_case(zlib.crc32(name.encode()) % 1000, layout, elem, layers, nh, d, bs, lengths, extra)
    dpools = [to_device_bits(p) for p in hpools]
    got = gpu_blocks(dpools, layout, layers, req)
    want = oracle.checksum_blocks(hpools, layout, layers, [0] * len(layers), req.block_table, req.num_blocks,
                                  req.start_pos, req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (name, r, k)
    assert_unlisted_untouched(got, req)


_GRID_CASE = {}


def _grid_case():
    """About 2,200 listed positions over 4 layers: with the listed plan, more
    tasks than resident waves at any launch shape, so each wave runs several."""
    if not _GRID_CASE:
        rng = np.random.default_rng(77)
        lengths = rng.integers(100, 601, size=100)
        layers = [0, 3, 4, 9]
        req, nb = wl.page_requests(rng, lengths, 16, spare_frac=0.1)
        hpools = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 12, 64), "fp16") for _ in layers]
        want = oracle.checksum_blocks(hpools, "NHD", layers, [0] * len(layers), req.block_table, req.num_blocks,
                                      req.start_pos, req.num_tokens)
        _GRID_CASE.update(req=req, hpools=hpools, layers=layers, want=want)
    return _GRID_CASE


@pytest.mark.parametrize("grid", ["1", "2", "64"])
@pytest.mark.parametrize("sched", ["simple", "pipelined"])
def test_launch_shapes_match_oracle(grid, sched, monkeypatch):
    """Results do not depend on the launch shape: one, two or as many
    workgroups per CU as fit (KVCK_GRID_PER_CU), under either schedule, with
    every wave striding over several tasks."""
    monkeypatch.setenv("KVCK_GRID_PER_CU", grid)
    monkeypatch.setenv("KVCK_SCHEDULE", sched)
    monkeypatch.setenv("KVCK_PLAN", "compact")
    log(f"[launch_shapes] grid {grid} {sched}")
    c = _grid_case()
    req = c["req"]
    got = gpu_blocks([to_device_bits(p) for p in c["hpools"]], "NHD", c["layers"], req)
    for r, k in req.listed():
        assert int(got[r, k]) == int(c["want"][r, k]), (grid, sched, r, k)
    assert_unlisted_untouched(got, req)


@pytest.mark.parametrize("plan", ["in place", "compact"])
def test_block_table_view_of_wider_rows(plan, monkeypatch):
    """A block table that is a column slice of a wider table (row stride >
    max_blocks, the extra columns holding out-of-range ids) gives the oracle's
    checksums, whether the call plans in place (the main pass reads the table
    itself) or lists its positions first."""
    if plan == "compact":
        monkeypatch.setenv("KVCK_PLAN", "compact")
    log(f"[block_table_view] {plan}")
    req, hpools = _host_case(91, "HND", "bf16", [0, 2], 4, 64, 16, [70, 33, 1, 48], None)
    wide = np.full((req.num_reqs, req.max_blocks + 5), 2**31 - 1, dtype=np.int32)
    wide[:, :req.max_blocks] = req.block_table
    bt = torch.from_numpy(wide).to(DEV)[:, :req.max_blocks]
    assert bt.stride(0) == req.max_blocks + 5
    _, nb, sp, nt = req_tensors(req)
    dpools = [to_device_bits(p) for p in hpools]
    out = torch.full((req.num_reqs, req.max_blocks), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64)
    kvck.kvck_checksum_blocks(dpools, "HND", [0, 2], bt, nb, sp, nt, out=out, check=True)
    got = out.cpu().numpy().view(np.uint64).reshape(req.num_reqs, req.max_blocks)
    want = oracle.checksum_blocks(hpools, "HND", [0, 2], [0, 0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (plan, r, k)
    assert_unlisted_untouched(got, req)


def test_tiny_config_golden():
    """The tiny workload on the GPU equals the oracle's committed values."""
    import json
    import os
    w = wl.tiny()
    log("[tiny] config 1")
    pools = [to_device_bits(p) for p in w.host_pools()]
    got = gpu_blocks(pools, w.layout, w.layer_numbers, w.req)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")) as f:
        gold = json.load(f)
    assert [str(int(x)) for x in got[0, :4]] == gold["checksums"]


def test_start_pos_heads_subset_and_global_base(schedule):
    log("[heads subset]")
    rng = np.random.default_rng(5)
    req, nb = wl.page_requests(rng, [90, 40, 200], 16, start_pos=[2, 0, 5], extra_blocks=[1, 0, 2], spare_frac=0.2)
    pools_h = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16") for _ in range(3)]
    pools = [to_device_bits(p) for p in pools_h]
    layers = [4, 9, 30000]
    bases = [16, 18, 65534 - 2]
    got = gpu_blocks(pools, "HND", layers, req, bases=bases, head_begin=3, head_count=2)
    want = oracle.checksum_blocks(pools_h, "HND", layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=3, head_count=2)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])


def test_tp_shards_sum_and_pp_split_sum(schedule):
    log("[tp/pp partial sums]")
    rng = np.random.default_rng(6)
    req, nb = wl.page_requests(rng, [300, 77, 16], 16, spare_frac=0.1)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16"))
             for _ in range(4)]
    layers = [0, 1, 2, 3]
    full = gpu_blocks(pools, "HND", layers, req)
    with np.errstate(over="ignore"):
        tot = np.zeros_like(full)
        for h in range(0, 8, 2):
            tot += gpu_blocks(pools, "HND", layers, req, bases=[h] * 4, head_begin=h, head_count=2)
        pp = gpu_blocks(pools[:1], "HND", layers[:1], req) + gpu_blocks(pools[1:], "HND", layers[1:], req)
    for r, k in req.listed():
        assert tot[r, k] == full[r, k] and pp[r, k] == full[r, k]


def test_accumulate_adds_mod_2_64(schedule):
    log("[accumulate]")
    rng = np.random.default_rng(7)
    req, nb = wl.page_requests(rng, [64, 100], 16, spare_frac=0.1)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16"))
             for _ in range(2)]
    base = gpu_blocks(pools, "NHD", [0, 1], req)
    init = rng.integers(0, 2**63, size=base.shape, dtype=np.int64).view(np.uint64) * np.uint64(2) + np.uint64(1)
    out = torch.from_numpy(init.view(np.int64).copy()).to(DEV).view(torch.uint64)
    got = gpu_blocks(pools, "NHD", [0, 1], req, out=out, accumulate=True)
    with np.errstate(over="ignore"):
        for r, k in req.listed():
            assert got[r, k] == init[r, k] + base[r, k]
    # a single cache takes the direct-write path
    one = gpu_blocks(pools[:1], "NHD", [0], req)
    out = torch.from_numpy(init.view(np.int64).copy()).to(DEV).view(torch.uint64)
    got = gpu_blocks(pools[:1], "NHD", [0], req, out=out, accumulate=True)
    with np.errstate(over="ignore"):
        for r, k in req.listed():
            assert got[r, k] == init[r, k] + one[r, k]


def test_many_caches_several_launches(schedule):
    """More caches than one argument block carries (several main launches)."""
    log("[70 caches]")
    rng = np.random.default_rng(8)
    req, nb = wl.page_requests(rng, [40, 9], 16, spare_frac=0.5)
    hp = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 16), "bf16") for _ in range(70)]
    layers = list(range(100, 170))
    got = gpu_blocks([to_device_bits(p) for p in hp], "NHD", layers, req)
    want = oracle.checksum_blocks(hp, "NHD", layers, [0] * 70, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])


def test_the_most_caches_one_call_takes(schedule):
    """KVCK_MAX_CACHES (4096) caches in one call: 64 launches of the argument
    block, thousands of partial groups summed by the second pass; layer numbers
    spread over the whole int32 range and global heads over all 65536."""
    log("[4096 caches]")
    assert kvck.KVCK_MAX_CACHES == 4096
    rng = np.random.default_rng(32)
    req, nb = wl.page_requests(rng, [9, 4, 0, 7], 2, start_pos=[0, 3, 0, 1], extra_blocks=[1, 0, 0, 0],
                               spare_frac=0.5)
    hp = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 2, 1, 8), "bf16") for _ in range(4096)]
    layers = [int(x) for x in rng.choice(1 << 31, size=4096, replace=False)]
    bases = [int(x) for x in rng.integers(0, 65536, size=4096)]
    got = gpu_blocks([to_device_bits(p) for p in hp], "NHD", layers, req, bases=bases)
    want = oracle.checksum_blocks(hp, "NHD", layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    assert_unlisted_untouched(got, req)


def test_empty_and_past_end_positions(schedule):
    log("[empty]")
    rng = np.random.default_rng(9)
    # a request with no listed positions, one with only positions past its tokens
    req, nb = wl.page_requests(rng, [0, 5, 40], 16, start_pos=[0, 1, 0], extra_blocks=[0, 2, 1], spare_frac=0.5)
    hp = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16")]
    got = gpu_blocks([to_device_bits(hp[0])], "NHD", [0], req)
    want = oracle.checksum_blocks(hp, "NHD", [0], [0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k])
    assert_unlisted_untouched(got, req)
    # zero requests: nothing launched, nothing written
    bt = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    e32 = torch.zeros(0, dtype=torch.int32, device=DEV)
    e64 = torch.zeros(0, dtype=torch.int64, device=DEV)
    out = kvck.kvck_checksum_blocks([to_device_bits(hp[0])], "NHD", [0], bt, e32, e64, e64)
    assert out.numel() == 0


def test_bad_block_id_and_bad_request_flagged():
    log("[flags]")
    rng = np.random.default_rng(10)
    req, nb = wl.page_requests(rng, [40, 40], 16, spare_frac=0.5)
    pool = to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16"))
    bad = wl.Requests(16, req.num_tokens, req.start_pos, req.num_blocks, req.block_table.copy())
    bad.block_table[0, 1] = nb + 5
    with pytest.raises(kvck.KvckDeviceError) as ei:
        gpu_blocks([pool], "NHD", [0], bad)
    assert ei.value.flags & kvck.KVCK_FLAG_BAD_BLOCK_ID
    bad2 = wl.Requests(16, req.num_tokens, req.start_pos.copy(), req.num_blocks, req.block_table)
    bad2.start_pos[1] = -3
    with pytest.raises(kvck.KvckDeviceError) as ei:
        gpu_blocks([pool], "NHD", [0], bad2)
    assert ei.value.flags & kvck.KVCK_FLAG_BAD_REQUEST
    # an invalid id where no slot is valid is never read and not an error
    past = wl.Requests(16, np.array([10, 40]), req.start_pos, np.array([2, 3], np.int32), req.block_table.copy())
    past.block_table[0, 1] = -1
    got = gpu_blocks([pool], "NHD", [0], past)
    assert got[0, 1] == 0
    # a caller's flag word holding a stale bit is cleared by check=True
    bt, nbt, sp, nt = req_tensors(req)
    stale = torch.full((1,), kvck.KVCK_FLAG_BAD_BLOCK_ID, dtype=torch.int32, device=DEV)
    kvck.kvck_checksum_blocks([pool], "NHD", [0], bt, nbt, sp, nt, error_flags=stale, check=True)
    assert int(stale.item()) == 0


@pytest.mark.parametrize("layout,ncaches", [("NHD", 1), ("NHD", 3), ("HND", 2), ("MLA", 4), ("HND", 70),
                                            ("V_TRANS", 2)])
def test_plan_in_place_matches_listed_plan(layout, ncaches, monkeypatch):
    """Small calls read the request arrays in the main pass (no plan launch);
    the result, the entries left untouched and the error bits must be those of
    the listed plan, with bad requests, bad ids and past-end ids mixed in."""
    log(f"[plan in place] {layout} caches {ncaches}")
    rng = np.random.default_rng(zlib.crc32(f"inplace{layout}{ncaches}".encode()))
    bs, nh, d = 16, 3, 64
    req, nb = wl.page_requests(rng, [40, 0, 70, 33, 16, 90], bs, start_pos=[0, 0, 1, 0, 2, 0],
                               extra_blocks=[1, 0, 0, 2, 0, 1], spare_frac=0.4)
    pool_layout = "HND" if layout == "V_TRANS" else layout
    heads = 1 if layout == "MLA" else nh
    hp = [wl.host_random_bits(rng, wl.pool_shape(pool_layout, nb, bs, heads, 576 if layout == "MLA" else d), "bf16")
          for _ in range(ncaches)]
    if layout == "V_TRANS":
        dev_pools = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    else:
        dev_pools = [to_device_bits(p) for p in hp]
    layers = [3 * i + 1 for i in range(ncaches)]
    bt = req.block_table.copy()
    nbpr = req.num_blocks.copy()
    sp = req.start_pos.copy()
    bt[0, 1] = nb + 3                      # a listed block with valid slots: flagged, contributes 0
    bt[3, int(nbpr[3]) - 1] = -7           # past the last token: never read, not an error
    nbpr[4] = req.max_blocks + 1           # bad request: lists nothing
    sp[5] = -1                             # bad request: lists nothing
    results = {}
    for plan in ("auto", "compact"):
        if plan == "compact":
            monkeypatch.setenv("KVCK_PLAN", "compact")
        else:
            monkeypatch.delenv("KVCK_PLAN", raising=False)
        out = torch.full((req.num_reqs, req.max_blocks), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64)
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        kvck.kvck_checksum_blocks(dev_pools, layout, layers, torch.from_numpy(bt).to(DEV),
                                  torch.from_numpy(nbpr).to(DEV), torch.from_numpy(sp).to(DEV),
                                  torch.from_numpy(req.num_tokens).to(DEV), out=out, error_flags=flags)
        torch.cuda.synchronize()
        results[plan] = (out.cpu().numpy().view(np.uint64).reshape(req.num_reqs, req.max_blocks).copy(),
                         int(flags.item()))
    assert np.array_equal(results["auto"][0], results["compact"][0])
    assert results["auto"][1] == results["compact"][1] == kvck.KVCK_FLAG_BAD_BLOCK_ID | kvck.KVCK_FLAG_BAD_REQUEST
    got = results["auto"][0]
    # the oracle on the same requests with the bad ones listing nothing and the bad id's block zeroed
    ok = wl.Requests(bs, req.num_tokens, np.where(sp < 0, 0, sp), np.where(np.arange(req.num_reqs) >= 4, 0, nbpr)
                     .astype(np.int32), np.where(bt < 0, 0, np.where(bt >= nb, 0, bt)).astype(np.int32))
    # a V-only call is the checksum of the pool with its K plane zeroed
    ref = [np.concatenate([np.zeros_like(p[:1]), p[1:]]) for p in hp] if layout == "V_TRANS" else hp
    want = oracle.checksum_blocks(ref, pool_layout, layers, [0] * ncaches, ok.block_table, ok.num_blocks,
                                  ok.start_pos, ok.num_tokens)
    for r, k in ok.listed():
        exp = 0 if (r, k) == (0, 1) else int(want[r, k])
        assert int(got[r, k]) == exp, (r, k)
    for r in (4, 5):
        assert np.all(got[r] == np.uint64(SENTINEL))
    assert_unlisted_untouched(got, ok)


def test_host_rejects_before_launch():
    log("[host errors]")
    rng = np.random.default_rng(11)
    req, nb = wl.page_requests(rng, [20], 16, spare_frac=0.5)
    pool = to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16"))
    with pytest.raises(kvck.KvckError) as ei:
        gpu_blocks([pool], "NHD", [0], req, bases=[65535])
    assert ei.value.status == -2
    with pytest.raises(kvck.KvckError) as ei:
        gpu_blocks([pool], "NHD", [-1], req)
    assert ei.value.status == -1
    # a layer number past 16 bits is valid (the page bounds heads, not layers)
    got = gpu_blocks([pool], "NHD", [40000], req)
    want = oracle.checksum_blocks([to_host_bits(pool)], "NHD", [40000], [0], req.block_table, req.num_blocks,
                                  req.start_pos, req.num_tokens)
    assert np.array_equal(got[0, :int(req.num_blocks[0])], want[0, :int(req.num_blocks[0])])
    with pytest.raises(kvck.KvckError) as ei:
        gpu_blocks([pool], "NHD", [0], req, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert ei.value.status == -4


def test_determinism_and_streams():
    log("[determinism]")
    rng = np.random.default_rng(12)
    req, nb = wl.page_requests(rng, list(rng.integers(1, 600, 40)), 16, spare_frac=0.1)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16"))
             for _ in range(5)]
    a = gpu_blocks(pools, "HND", list(range(5)), req)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_blocks(pools, "HND", list(range(5)), req, stream=s)
    ws = torch.empty(kvck.kvck_blocks_workspace_bytes(5, req.num_reqs, req.max_blocks), dtype=torch.uint8,
                     device=DEV)
    c = gpu_blocks(pools, "HND", list(range(5)), req, workspace=ws)
    d = gpu_blocks(pools, "HND", list(range(5)), req, workspace=ws)
    assert np.array_equal(a, b) and np.array_equal(a, c) and np.array_equal(a, d)
    for sched in ("simple", "pipelined"):
        os.environ["KVCK_SCHEDULE"] = sched
        try:
            e = gpu_blocks(pools, "HND", list(range(5)), req, workspace=ws)
        finally:
            del os.environ["KVCK_SCHEDULE"]
        assert np.array_equal(a, e), sched


def test_calls_on_another_stream_wait_for_the_current_one():
    """A call given stream=s without entering torch.cuda.stream(s): the pool
    is rewritten on the current stream just before (behind a long kernel),
    and out, workspace and flag word are allocated and cleared there by the
    binding; the call on s must still see all of it (s waits for the current
    stream) and its buffers must not be handed out again while s uses them."""
    log("[side stream]")
    rng = np.random.default_rng(19)
    req, nb = wl.page_requests(rng, list(rng.integers(1, 900, 30)), 16, spare_frac=0.1)
    host = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16") for _ in range(4)]
    pools = [to_device_bits(p) for p in host]
    layers = [0, 1, 2, 3]
    want = gpu_blocks(pools, "HND", layers, req)
    bt, nbt, sp, nt = req_tensors(req)
    saved = pools[0].clone()
    busy = torch.zeros(64 << 20, dtype=torch.float32, device=DEV)
    hs = [[wl.host_random_bits(rng, (5, 4, 16), "fp32")] for _ in range(2)]
    states = [[to_device_bits(a) for a in l] for l in hs]
    sids = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    want_states = oracle.checksum_states(hs, [1, 3], [0, 0], sids.cpu().numpy())
    s = torch.cuda.Stream()
    for i in range(3):
        pools[0].zero_()
        for _ in range(20):
            busy.add_(1.0)             # keeps the current stream busy
        pools[0].copy_(saved)          # the final cache bytes, written on the current stream
        got = kvck.kvck_checksum_blocks(pools, "HND", layers, bt, nbt, sp, nt, stream=s, check=(i == 2))
        gs = kvck.kvck_checksum_states(states, [1, 3], sids, stream=s)
        torch.cuda.synchronize()
        got = got.cpu().numpy().view(np.uint64)
        for r, k in req.listed():
            assert got[r, k] == want[r, k], (i, r, k)
        assert np.array_equal(gs.cpu().numpy().view(np.uint64), want_states), i


def test_states_small_parity():
    log("[states small]")
    rng = np.random.default_rng(13)
    layers = [1, 3, 5]
    shapes = [(6, 8, 4), (6, 2, 16)]     # rows x (...) : fp32 row 128 B, fp16 row 64 B
    elems = ["fp32", "fp16"]
    hs = [[wl.host_random_bits(rng, (9,) + s, e) for s, e in zip(shapes, elems)] for _ in layers]
    slots = np.array([4, 0, 8, 2], np.int32)
    ds = [[to_device_bits(a) for a in l] for l in hs]
    sid = torch.from_numpy(slots).to(DEV)
    for rb, rc, base in [(0, None, 0), (1, 3, 10), (5, 1, 7)]:
        got = kvck.kvck_checksum_states(ds, layers, sid, global_row_base=base, row_begin=rb, row_count=rc,
                                        check=True)
        want = oracle.checksum_states(hs, layers, [base] * 3, slots, row_begin=rb, row_count=rc)
        assert np.array_equal(got.cpu().numpy(), want), (rb, rc)
    bad = torch.tensor([0, 9], dtype=torch.int32, device=DEV)
    with pytest.raises(kvck.KvckDeviceError):
        kvck.kvck_checksum_states(ds, layers, bad, check=True)


@pytest.mark.parametrize("nlayers", [33, 70, 4096])
def test_states_many_layers(nlayers):
    """More Mamba layers than one argument block carries (32): several launches
    whose partials the second pass sums, up to the most layers a call takes
    (KVCK_MAX_CACHES); layer numbers and row bases spread over their ranges."""
    log(f"[states] {nlayers} layers")
    rng = np.random.default_rng(1000 + nlayers)
    layers = [int(x) for x in rng.choice(1 << 31, size=nlayers, replace=False)]
    bases = [int(x) for x in rng.integers(0, 65536 - 3, size=nlayers)]
    hs = [[wl.host_random_bits(rng, (3, 3, 8), "fp16"), wl.host_random_bits(rng, (3, 3, 4), "fp32")]
          for _ in layers]
    slots = np.array([2, 0, 2, 1, 0], np.int32)
    ds = [[to_device_bits(a) for a in l] for l in hs]
    sid = torch.from_numpy(slots).to(DEV)
    for rb, rc in [(0, None), (1, 2)]:
        got = kvck.kvck_checksum_states(ds, layers, sid, global_row_base=bases, row_begin=rb, row_count=rc,
                                        check=True)
        want = oracle.checksum_states(hs, layers, bases, slots, row_begin=rb, row_count=rc)
        assert np.array_equal(got.cpu().numpy(), want), (rb, rc)


def test_more_than_1024_requests(schedule):
    """Batches above 1024 requests take the two-kernel plan (scan, then fill)."""
    log("[1500 requests]")
    rng = np.random.default_rng(14)
    lengths = rng.integers(0, 41, size=1500)
    req, nb = wl.page_requests(rng, lengths, 16, start_pos=None, extra_blocks=rng.integers(0, 2, size=1500),
                               spare_frac=0.2)
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 2, 32), "bf16") for _ in range(3)]
    got = gpu_blocks([to_device_bits(p) for p in hp], "HND", [0, 1, 2], req)
    want = oracle.checksum_blocks(hp, "HND", [0, 1, 2], [0] * 3, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    assert_unlisted_untouched(got, req)


_MANY = {}


def _seventy_thousand_requests():
    """70,000 requests of 0-12 tokens at block size 4, start positions 0-2 and
    up to one listed position past the last token: 69 chunks of the plan's
    1024-request scan, about 107k listed positions among 280k slots; the
    oracle's values, computed once."""
    if not _MANY:
        rng = np.random.default_rng(31)
        n = 70000
        lengths = rng.integers(0, 13, size=n)
        start = rng.integers(0, 3, size=n)
        req, nb = wl.page_requests(rng, lengths, 4, start_pos=start, extra_blocks=rng.integers(0, 2, size=n),
                                   spare_frac=0.1)
        hp = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 4, 2, 16), "bf16") for _ in range(3)]
        want = oracle.checksum_blocks(hp, "NHD", [0, 1, 2], [0] * 3, req.block_table, req.num_blocks,
                                      req.start_pos, req.num_tokens)
        _MANY.update(req=req, hp=hp, want=want)
    return _MANY["req"], _MANY["hp"], _MANY["want"]


@pytest.mark.parametrize("sched", ["auto", "simple", "pipelined"])
def test_seventy_thousand_requests(sched, monkeypatch):
    """A batch far past one scan chunk: the plan carries its prefix across 69
    chunks of 1024 requests; every listed position equals the oracle and no
    other entry is written."""
    log(f"[70000 requests] {sched}")
    if sched != "auto":
        monkeypatch.setenv("KVCK_SCHEDULE", sched)
    req, hp, want = _seventy_thousand_requests()
    got = gpu_blocks([to_device_bits(p) for p in hp], "NHD", [0, 1, 2], req)
    listed = np.arange(req.max_blocks)[None, :] < req.num_blocks[:, None]
    assert int(listed.sum()) > 100000
    bad = np.argwhere(listed & (got != want))
    assert bad.size == 0, f"{len(bad)} mismatches, first at (request, position) {tuple(bad[0])}"
    assert np.all(got[~listed] == np.uint64(SENTINEL)), "unlisted entries were written"


@pytest.mark.parametrize("ncaches", [3, 70])
def test_second_pass_beyond_one_grid(ncaches, monkeypatch):
    """1.1M listed positions, one cache per partial group (the simple
    schedule): more positions than one grid of the second pass covers, so it
    strides (the partials sum for 3 groups, its wave-per-output variant for
    70).  Every position equals the sum, mod 2^64, of one-cache calls, which
    write their values directly; 3000 sampled positions equal the oracle."""
    log(f"[1.1M positions] {ncaches} caches")
    monkeypatch.setenv("KVCK_SCHEDULE", "simple")
    rng = np.random.default_rng(40 + ncaches)
    req, nb = wl.page_requests(rng, np.full(275_000, 8), 2, spare_frac=0.02)
    assert int(req.num_blocks.sum()) > 1 << 20
    g = torch.Generator(device=DEV)
    g.manual_seed(41 + ncaches)
    pools = [wl.device_fill(wl.pool_shape("NHD", nb, 2, 1, 8), "bf16", "bits", g, DEV) for _ in range(ncaches)]
    layers = [int(x) for x in rng.choice(1 << 20, size=ncaches, replace=False)]
    got = gpu_blocks(pools, "NHD", layers, req)
    total = np.zeros_like(got)
    with np.errstate(over="ignore"):
        for p, layer in zip(pools, layers):
            total += gpu_blocks([p], "NHD", [layer], req)
    listed = np.arange(req.max_blocks)[None, :] < req.num_blocks[:, None]
    assert np.array_equal(got[listed], total[listed])
    pos = sample_positions(req, 3000, seed=ncaches, include_tails=False)
    assert_match(got, oracle_at(pools, "NHD", layers, req, pos), "sampled positions")


def test_largest_numbering(schedule):
    """The largest numbering the method allows: layer 32767 with 65536 heads
    per layer, so the slice factor m = 2(layer*65536 + head) + 1 reaches
    2^32 - 1 (8-byte rows, block size 2)."""
    log("[largest numbering]")
    rng = np.random.default_rng(15)
    req, nb = wl.page_requests(rng, [3, 4, 1], 2, extra_blocks=[0, 1, 0], spare_frac=0.5)
    hp = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 2, 65536, 4), "bf16") for _ in range(2)]
    layers = [32767, 1]
    got = gpu_blocks([to_device_bits(p) for p in hp], "NHD", layers, req)
    want = oracle.checksum_blocks(hp, "NHD", layers, [0, 0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    # the last two global heads of the largest layer alone, by head subset
    got = gpu_blocks([to_device_bits(hp[0])], "NHD", [32767], req, bases=[65534], head_begin=65534, head_count=2)
    want = oracle.checksum_blocks(hp[:1], "NHD", [32767], [65534], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=65534, head_count=2)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)


BIG_LAYERS = [(1 << 31) - 1, 1 << 20, 40000, 3]


@pytest.mark.parametrize("layout,elem,nh,d", [("HND", "bf16", 8, 128), ("NHD", "fp8", 12, 64), ("NHD", "fp16", 4, 64),
                                              ("MLA", "bf16", 1, 576)])
def test_layer_numbers_beyond_16_bits(layout, elem, nh, d, schedule):
    """Layer numbers are not bounded by the page (the number in the layer's
    name): at layer 2^31 - 1 the factor m = 2(layer*65536 + head) + 1 nears
    2^48.  Separate heads (HND), merged heads (fp8 NHD, 64-byte rows) and a
    single latent head (MLA), and the fused save of the same pools."""
    log(f"[large layer numbers] {layout} {elem}")
    rng = np.random.default_rng(zlib.crc32(f"layers{layout}{elem}".encode()))
    req, nb = wl.page_requests(rng, list(rng.integers(1, 300, 9)), 16, extra_blocks=[1] + [0] * 8, spare_frac=0.3)
    hp = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, 16, nh, d), elem) for _ in BIG_LAYERS]
    pools = [to_device_bits(p) for p in hp]
    bases = [nh * 7] * len(BIG_LAYERS)
    got = gpu_blocks(pools, layout, BIG_LAYERS, req, bases=bases)
    want = oracle.checksum_blocks(hp, layout, BIG_LAYERS, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    bt, nbt, sp, nt = req_tensors(req)
    staging = torch.empty(int(req.num_blocks.sum()) * kvck.kvck_staging_bytes(pools[0], layout, len(pools)),
                          dtype=torch.uint8, device=DEV)
    saved = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, layout, BIG_LAYERS, bt, nbt, sp, nt, staging,
                                           global_head_base=bases, check=True).cpu().numpy().view(np.uint64)
    for r, k in req.listed():
        assert int(saved[r, k]) == int(want[r, k]), (r, k)


def test_states_layer_numbers_beyond_16_bits():
    """Mamba states on layers up to 2^31 - 1."""
    log("[large layer numbers] states")
    rng = np.random.default_rng(17)
    layers = [(1 << 31) - 1, 1 << 20, 1]
    hs = [[wl.host_random_bits(rng, (6, 4, 8, 4), "fp32"), wl.host_random_bits(rng, (6, 4, 16), "fp16")]
          for _ in layers]
    slots = np.array([5, 0, 3], dtype=np.int32)
    got = kvck.kvck_checksum_states([[to_device_bits(a) for a in l] for l in hs], layers,
                                    torch.from_numpy(slots).to(DEV), global_row_base=9, check=True)
    want = oracle.checksum_states(hs, layers, [9] * 3, slots)
    assert np.array_equal(got.cpu().numpy().view(np.uint64), want)


@pytest.mark.parametrize("layout,elem,nh,d", [("HND", "bf16", 8, 128), ("NHD", "fp8", 12, 64), ("MLA", "bf16", 1, 576)])
def test_piece_indices_beyond_32_bits(layout, elem, nh, d, schedule):
    """Requests whose first listed block starts past token 2^31: piece indices
    j = t*P + p exceed 2^32 (and 2^36 for MLA's P = 144)."""
    log(f"[large piece indices] {layout} {elem}")
    rng = np.random.default_rng(zlib.crc32(f"big{layout}{elem}".encode()))
    bs = 16
    start = [(1 << 27) + 1, (1 << 28) + 5, 7]
    lengths = [(s + 2) * bs + 9 for s in start]        # three listed blocks each, the last partly valid
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=start, extra_blocks=[1, 0, 0], spare_frac=0.3)
    hp = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), elem) for _ in range(2)]
    layers = [0, 9]
    got = gpu_blocks([to_device_bits(p) for p in hp], layout, layers, req)
    want = oracle.checksum_blocks(hp, layout, layers, [0, 0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    if layout == "HND":
        # the fused save path numbers pieces the same way
        bt, nbt, sp, nt = (torch.from_numpy(x).to(DEV) for x in (req.block_table, req.num_blocks, req.start_pos,
                                                                    req.num_tokens))
        pools = [to_device_bits(p) for p in hp]
        per = kvck.kvck_staging_bytes(pools[0], layout, len(layers))
        staging = torch.zeros(int(req.num_blocks.sum()) * per, dtype=torch.uint8, device=DEV)
        cs = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, layout, layers, bt, nbt, sp, nt, staging,
                                            check=True).cpu().numpy()
        for r, k in req.listed():
            assert int(cs[r, k]) == int(want[r, k]), (r, k)


MERGE_CASES = [
    # name, layout, elem, heads, head_size, block_size, lengths, head_begin, head_count
    ("nhd_fp8_d64", "NHD", "fp8", 12, 64, 16, [90, 7, 33], 0, None),
    ("nhd_fp8_bs64", "NHD", "fp8", 12, 64, 64, [200, 64, 5], 0, None),
    ("nhd_fp8_heads_3_8", "NHD", "fp8", 12, 64, 16, [50, 17], 3, 5),
    ("nhd_bf16_d32", "NHD", "bf16", 4, 32, 16, [40, 16, 9], 1, 2),
    ("nhd_fp16_d64", "NHD", "fp16", 12, 64, 16, [100, 31], 0, None),
    ("nhd_bf16_d384_bs64", "NHD", "bf16", 2, 384, 64, [130, 64], 0, None),
    ("fi_nhd_fp8", "FI_NHD", "fp8", 8, 64, 16, [77, 16], 2, 4),
    ("nhd_fp32_d2_bs1", "NHD", "fp32", 6, 2, 1, [5, 2], 0, None),         # 8-byte rows, 8-byte chunks
]


@pytest.mark.parametrize("merge", ["0", "1"])
@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_merged_heads_parity(case, merge, monkeypatch):
    """Heads side by side in a slot read as one row per slot (KVCK_MERGE_HEADS=1)
    or head by head (=0): both equal the oracle."""
    name, layout, elem, nh, d, bs, lengths, hb, hc = case
    monkeypatch.setenv("KVCK_MERGE_HEADS", merge)
    log(f"[merged heads] {name} merge={merge}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=[1] + [0] * (len(lengths) - 1),
                               extra_blocks=[0] * (len(lengths) - 1) + [1], spare_frac=0.3)
    layers = [2, 5, 9]
    hp = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), elem) for _ in layers]
    n = nh - hb if hc is None else hc
    bases = [hb + 7 * i for i in range(len(layers))]
    got = gpu_blocks([to_device_bits(p) for p in hp], layout, layers, req, bases=bases, head_begin=hb, head_count=hc)
    want = oracle.checksum_blocks(hp, layout, layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens, head_begin=hb, head_count=n)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    assert_unlisted_untouched(got, req)


@pytest.mark.parametrize("layout,elem,nh,d", [("HND", "bf16", 2, 384), ("NHD", "bf16", 2, 384), ("MLA", "fp8", 1, 1536)])
def test_row_groups_fit_one_lane_table(layout, elem, nh, d, schedule, monkeypatch):
    """Rows whose size does not divide a lane table's 16 KiB (768- and
    1536-byte rows in 64-slot blocks) are split into row groups that fit."""
    monkeypatch.setenv("KVCK_MERGE_HEADS", "0")
    log(f"[row groups] {layout} {elem} d={d}")
    rng = np.random.default_rng(zlib.crc32(f"rg{layout}{d}".encode()))
    req, nb = wl.page_requests(rng, [150, 64, 3], 64, spare_frac=0.3)
    layers = [0, 1]
    hp = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, 64, nh, d), elem) for _ in layers]
    got = gpu_blocks([to_device_bits(p) for p in hp], layout, layers, req)
    want = oracle.checksum_blocks(hp, layout, layers, [0, 0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)


def test_calls_from_several_host_threads():
    """The library is thread-safe: host threads, each with its own stream,
    workspace and output, calling at once on two layouts all get the
    single-thread result."""
    import threading
    log("[threads]")
    rng = np.random.default_rng(16)
    req, nb = wl.page_requests(rng, list(rng.integers(1, 400, 24)), 16, spare_frac=0.1)
    layouts = {"HND": [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16"))
                       for _ in range(6)],
               "NHD": [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 12, 64), "fp8"))
                       for _ in range(6)]}
    want = {k: gpu_blocks(p, k, list(range(6)), req) for k, p in layouts.items()}
    bt, nbt, sp, nt = req_tensors(req)
    errors, results = [], {}

    def worker(i):
        try:
            layout = "HND" if i % 2 == 0 else "NHD"
            s = torch.cuda.Stream()
            ws = torch.empty(kvck.kvck_blocks_workspace_bytes(6, req.num_reqs, req.max_blocks), dtype=torch.uint8,
                             device=DEV)
            out = torch.zeros((req.num_reqs, req.max_blocks), dtype=torch.uint64, device=DEV)
            s.wait_stream(torch.cuda.current_stream())  # the zero fill above runs on this thread's current stream
            with torch.cuda.stream(s):
                for _ in range(5):
                    kvck.kvck_checksum_blocks(layouts[layout], layout, list(range(6)), bt, nbt, sp, nt, out=out,
                                              workspace=ws, stream=s)
            s.synchronize()
            results[i] = (layout, out.cpu().numpy().view(np.uint64))
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(6)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert len(results) == 6
    for i, (layout, got) in results.items():
        for r, k in req.listed():
            assert got[r, k] == want[layout][r, k], (i, r, k)


@pytest.mark.parametrize("layout,elem,nh,d,bs", [("NHD", "fp8", 12, 64, 16), ("NHD", "bf16", 8, 32, 16),
                                                 ("MLA", "bf16", 1, 576, 16), ("MLA", "bf16", 1, 576, 64),
                                                 ("NHD", "fp8", 3, 64, 8)])
@pytest.mark.parametrize("ncaches", [1, 5])
def test_merged_rows_stream_across_tasks(layout, elem, nh, d, bs, ncaches, monkeypatch):
    """Merged rows stream their units across task boundaries in planned calls:
    a wave's tasks follow one another with both load buffers in flight.  Many
    tasks per wave (the plan forced, one or five caches), positions with no
    valid slot and bad block ids in the middle of the stream, start offsets,
    and (one cache: a direct write) accumulate onto the previous values -- every
    position equal to the oracle, unlisted entries untouched."""
    log(f"[merged stream] {layout} {elem} {nh}x{d} bs{bs} caches {ncaches}")
    monkeypatch.setenv("KVCK_PLAN", "compact")
    rng = np.random.default_rng(zlib.crc32(f"stream{layout}{elem}{nh}{d}{bs}{ncaches}".encode()))
    R = 300
    lengths = list(rng.integers(1, 12 * bs, R))
    start = [int(x) if i % 7 == 3 else 0 for i, x in enumerate(rng.integers(0, 3, R))]
    extra = [1 if i % 5 == 0 else 0 for i in range(R)]          # positions past the last token: no valid slot
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=start, extra_blocks=extra, spare_frac=0.2)
    layers = [int(x) for x in rng.choice(1000, ncaches, replace=False)]
    hp = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), elem) for _ in layers]
    pools = [to_device_bits(p) for p in hp]
    want = oracle.checksum_blocks(hp, layout, layers, [0] * ncaches, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    got = gpu_blocks(pools, layout, layers, req)
    for r, k in req.listed():
        assert int(got[r, k]) == int(want[r, k]), (r, k)
    assert_unlisted_untouched(got, req)
    # accumulate onto the previous output: every listed entry doubles (mod 2^64)
    prev = torch.from_numpy(got.view(np.int64).copy()).to(DEV).view(torch.uint64)
    got2 = gpu_blocks(pools, layout, layers, req, out=prev, accumulate=True)
    with np.errstate(over="ignore"):
        for r, k in req.listed():
            assert got2[r, k] == np.uint64(want[r, k]) * np.uint64(2), (r, k)
    # bad ids scattered through the stream: those positions contribute 0 and are flagged
    bad = req.block_table.copy()
    listed = req.listed()
    hit = [listed[i] for i in rng.choice(len(listed), 9, replace=False)]
    for r, k in hit:
        bad[r, k] = nb + 3 + r
    breq = wl.Requests(req.block_size, req.num_tokens, req.start_pos, req.num_blocks, bad)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    got3 = gpu_blocks(pools, layout, layers, breq, check=False,
                      out=torch.full((R, req.max_blocks), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64))
    bt, nbt, sp, nt = req_tensors(breq)
    kvck.kvck_checksum_blocks(pools, layout, layers, bt, nbt, sp, nt, error_flags=flags)
    torch.cuda.synchronize()
    valid_hit = [(r, k) for r, k in hit
                 if oracle.num_valid_tokens(int(req.start_pos[r]) + k, bs, int(req.num_tokens[r])) > 0]
    assert (int(flags.item()) & kvck.KVCK_FLAG_BAD_BLOCK_ID) == (kvck.KVCK_FLAG_BAD_BLOCK_ID if valid_hit else 0)
    for r, k in listed:
        assert int(got3[r, k]) == (0 if (r, k) in hit else int(want[r, k])), (r, k)


def test_prepared_call_equals_the_wrapper():
    """A PreparedCall gives the wrapper's results, also into one replica column
    and with accumulate, and can be called repeatedly."""
    log("[small] prepared call")
    rng = np.random.default_rng(77)
    req, nb = wl.page_requests(rng, [50, 17, 33], 16, start_pos=[0, 1, 0], spare_frac=0.3)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16")) for _ in range(3)]
    pc = kvck.prepare_caches(pools, "NHD", [0, 4, 9])
    bt, nbt, sp, nt = req_tensors(req)
    ws = torch.empty(kvck.kvck_blocks_workspace_bytes(3, req.num_reqs, req.max_blocks), dtype=torch.uint8,
                     device=DEV)
    want = kvck.kvck_checksum_blocks(pc, None, None, bt, nbt, sp, nt, check=True).cpu().view(torch.int64).numpy()
    want = want.view(np.uint64)
    values = torch.zeros((req.num_reqs, req.max_blocks, 2), dtype=torch.uint64, device=DEV)
    call = kvck.prepare_call(pc, bt, nbt, sp, nt, values[..., 1], ws)
    for _ in range(3):
        call()
    acc = kvck.prepare_call(pc, bt, nbt, sp, nt, values[..., 0], ws, accumulate=True)
    acc()
    acc()
    torch.cuda.synchronize()
    got = values.cpu().view(torch.int64).numpy().view(np.uint64)
    for r, k in req.listed():
        assert got[r, k, 1] == want[r, k]
        with np.errstate(over="ignore"):
            assert got[r, k, 0] == want[r, k] * np.uint64(2)
    with pytest.raises(ValueError):
        kvck.prepare_call(pc, bt, nbt, sp, nt, values[..., 1], ws[:8])      # workspace too small

"""The allocation-free checksum entry point (kvck_checksum_blocks_noalloc)
against kvck_checksum_blocks on the same inputs, bit for bit, through the C
ABI: two calls in a row, the second on a smaller batch (the scratch array then
holds the first call's records and partials), then a larger one again with
accumulate, bad ids and requests, and a call that does not fit the scratch."""

import numpy as np
import pytest
import torch

import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, SENTINEL, assert_match, gpu_blocks, log, oracle_at, req_tensors, sample_positions

pytestmark = pytest.mark.gpu


def _sentinel_out(req):
    return torch.full((req.num_reqs, req.max_blocks), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64)


def _noalloc(pools, layout, layers, req, out, **kw):
    bt, nb, sp, nt = req_tensors(req)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    kvck.kvck_checksum_blocks_noalloc(pools, layout, layers, bt, nb, sp, nt, out, **kw)
    assert torch.cuda.memory_allocated(DEV) == before  # the wrapper allocates nothing either
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint64).reshape(req.num_reqs, req.max_blocks)


def test_noalloc_equals_workspace_call():
    rng = np.random.default_rng(31)
    # 1: a planned call whose 32 layers form several task groups (records and partials in the scratch)
    log("[noalloc] 32 layers HND, 40 requests")
    req1, nb1 = wl.page_requests(rng, list(rng.integers(100, 3000, 40)), 16, spare_frac=0.05)
    pools1 = [torch.randint(-2**15, 2**15, wl.pool_shape("HND", nb1, 16, 8, 128), dtype=torch.int16, device=DEV)
              for _ in range(32)]
    layers1 = list(range(32))
    want1 = gpu_blocks(pools1, "HND", layers1, req1)
    got1 = _noalloc(pools1, "HND", layers1, req1, _sentinel_out(req1))
    assert np.array_equal(got1, want1)
    assert_match(got1, oracle_at(pools1, "HND", layers1, req1, sample_positions(req1, 24, seed=2)), "noalloc 1")
    # 2: right after, a smaller call planned in place (fp8 NHD, merged rows), on top of call 1's scratch
    log("[noalloc] 5 layers fp8 NHD, 3 requests")
    req2, nb2 = wl.page_requests(rng, [70, 5, 33], 16, start_pos=[0, 0, 1], extra_blocks=[1, 0, 0], spare_frac=0.3)
    pools2 = [torch.randint(0, 256, wl.pool_shape("NHD", nb2, 16, 12, 64), dtype=torch.uint8, device=DEV)
              for _ in range(5)]
    layers2 = [3, 9, 100, 40000, (1 << 31) - 1]
    want2 = gpu_blocks(pools2, "NHD", layers2, req2, bases=[4] * 5)
    got2 = _noalloc(pools2, "NHD", layers2, req2, _sentinel_out(req2), global_head_base=[4] * 5)
    assert np.array_equal(got2, want2)
    assert_match(got2, oracle_at(pools2, "NHD", layers2, req2, req2.listed(), bases=[4] * 5), "noalloc 2")
    # 3: the first batch again, a TP-shard subset accumulated onto its output
    log("[noalloc] accumulate, head subset")
    base = torch.from_numpy(got1.view(np.int64).copy()).to(DEV).view(torch.uint64)
    want3 = gpu_blocks(pools1, "HND", layers1, req1, bases=[2] * 32, head_begin=2, head_count=2,
                       out=torch.from_numpy(got1.view(np.int64).copy()).to(DEV).view(torch.uint64), accumulate=True)
    got3 = _noalloc(pools1, "HND", layers1, req1, base, global_head_base=[2] * 32, head_begin=2, head_count=2,
                    accumulate=True)
    assert np.array_equal(got3, want3)


def test_noalloc_flags_and_limits():
    rng = np.random.default_rng(32)
    log("[noalloc] bad ids and requests")
    req, nb = wl.page_requests(rng, [40, 50, 60], 16, spare_frac=0.3)
    pools = [torch.randint(-2**15, 2**15, wl.pool_shape("HND", nb, 16, 2, 64), dtype=torch.int16, device=DEV)
             for _ in range(3)]
    req.block_table[0, 1] = nb + 5          # outside the pool
    req.num_blocks[2] = req.max_blocks + 1  # a bad request
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = _noalloc(pools, "HND", [0, 1, 2], req, _sentinel_out(req), error_flags=flags)
    assert int(flags.item()) == kvck.KVCK_FLAG_BAD_BLOCK_ID | kvck.KVCK_FLAG_BAD_REQUEST
    want = gpu_blocks(pools, "HND", [0, 1, 2], req, check=False)
    assert np.array_equal(got, want)
    assert got[0, 1] == 0 and np.all(got[2] == np.uint64(SENTINEL))
    # a batch whose position records alone exceed the scratch: refused, nothing launched or written
    log("[noalloc] over the scratch limit")
    R, M = 1100, 1024
    bt = torch.zeros((R, M), dtype=torch.int32, device=DEV)
    zeros32 = torch.zeros(R, dtype=torch.int32, device=DEV)
    zeros64 = torch.zeros(R, dtype=torch.int64, device=DEV)
    out = torch.zeros((R, M), dtype=torch.uint64, device=DEV)
    with pytest.raises(kvck.KvckError) as e:
        kvck.kvck_checksum_blocks_noalloc(pools, "HND", [0, 1, 2], bt, zeros32, zeros64, zeros64, out)
    assert e.value.status == -7

"""kvck calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, after eager changes to the cache between replays, equals an
eager call (GPU)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, log, req_tensors, to_device_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule", ["simple", "pipelined"])
def test_graph_replays_match_eager(schedule, monkeypatch):
    monkeypatch.setenv("KVCK_SCHEDULE", schedule)
    log(f"[graphs] {schedule}")
    rng = np.random.default_rng(40)
    req, nb = wl.page_requests(rng, [100, 37, 300, 5], 16, spare_frac=0.2)
    layers = [0, 1, 2, 3, 4]
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16"))
             for _ in layers]
    pc = kvck.prepare_caches(pools, "HND", layers)
    bt, nbt, sp, nt = req_tensors(req)
    out = torch.zeros((req.num_reqs, req.max_blocks), dtype=torch.uint64, device=DEV)
    ws = torch.empty(kvck.kvck_blocks_workspace_bytes(len(layers), req.num_reqs, req.max_blocks),
                     dtype=torch.uint8, device=DEV)

    def eager():
        return kvck.kvck_checksum_blocks(pc, None, None, bt, nbt, sp, nt, workspace=torch.empty_like(ws)).cpu()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvck.kvck_checksum_blocks(pc, None, None, bt, nbt, sp, nt, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvck.kvck_checksum_blocks(pc, None, None, bt, nbt, sp, nt, out=out, workspace=ws)
    listed = req.listed()
    for rep in range(4):
        # eager work between replays: clear the output, flip one bit of one listed block
        out.view(torch.int64).zero_()
        r, k = listed[(7 * rep) % len(listed)]
        b = int(req.block_table[r, k])
        pools[rep % len(pools)].view(torch.int16)[rep % 2, b, rep, 0, 3] ^= 1 << rep
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = eager().numpy()
        for rr, kk in listed:
            assert got[rr, kk] == want[rr, kk], (rep, rr, kk)

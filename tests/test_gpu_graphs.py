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


@pytest.mark.parametrize("layout", ["HND", "V_TRANS"])
def test_graph_replays_fused_copy(layout):
    """A save then a load captured in one graph (row layout, and an element-
    transposed V plane through the LDS transpose): each replay, after eager
    changes to the source pool and a cleared destination, gives the eager
    calls' staging bytes, destination pool and checksums."""
    log(f"[graphs] fused copy {layout}")
    rng = np.random.default_rng(41)
    req, nb = wl.page_requests(rng, [100, 37, 300, 5], 16, spare_frac=0.2)
    layers = [0, 3, 4]
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 4, 128), "bf16") for _ in layers]
    if layout == "V_TRANS":
        src = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    else:
        src = [to_device_bits(p) for p in hp]
    dst = [torch.zeros_like(t) for t in src]
    bt, nbt, sp, nt = req_tensors(req)
    per = kvck.kvck_staging_bytes(src[0], layout, len(layers))
    staging = torch.zeros(int(req.num_blocks.sum()) * per, dtype=torch.uint8, device=DEV)
    out_s = torch.zeros((req.num_reqs, req.max_blocks), dtype=torch.uint64, device=DEV)
    out_l = torch.zeros_like(out_s)
    ws_s = torch.empty(kvck.kvck_blocks_workspace_bytes(len(layers), req.num_reqs, req.max_blocks),
                       dtype=torch.uint8, device=DEV)
    ws_l = torch.empty_like(ws_s)

    def calls(st, ds, os_, ol, wss, wsl):
        kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, src, layout, layers, bt, nbt, sp, nt, st, out=os_,
                                       workspace=wss)
        kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, ds, layout, layers, bt, nbt, sp, nt, st, out=ol,
                                       workspace=wsl)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(staging, dst, out_s, out_l, ws_s, ws_l)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(staging, dst, out_s, out_l, ws_s, ws_l)
    listed = req.listed()
    for rep in range(4):
        r, k = listed[(5 * rep) % len(listed)]
        b = int(req.block_table[r, k])
        # one element of slot 0 (valid at every listed position) of the V plane
        if layout == "V_TRANS":
            src[rep % len(src)].view(torch.int16)[b, rep % 4, 3, 0] ^= 1 << rep
        else:
            src[rep % len(src)].view(torch.int16)[1, b, rep % 4, 0, 3] ^= 1 << rep
        for t in dst:
            t.zero_()
        staging.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (staging.cpu().clone(), [t.cpu().clone() for t in dst], out_s.cpu().numpy().copy(),
               out_l.cpu().numpy().copy())
        st2 = torch.zeros_like(staging)
        ds2 = [torch.zeros_like(t) for t in dst]
        o2s, o2l = torch.zeros_like(out_s), torch.zeros_like(out_l)
        calls(st2, ds2, o2s, o2l, torch.empty_like(ws_s), torch.empty_like(ws_l))
        torch.cuda.synchronize()
        assert torch.equal(got[0], st2.cpu()), rep
        assert all(torch.equal(a, b.cpu()) for a, b in zip(got[1], ds2)), rep
        for rr, kk in listed:
            assert got[2][rr, kk] == o2s.cpu().numpy()[rr, kk] == got[3][rr, kk], (rep, rr, kk)


@pytest.mark.parametrize("schedule,ncaches", [("default", 3), ("simple", 20)])
def test_graph_replays_noalloc(schedule, ncaches, monkeypatch):
    """The allocation-free call captured into a graph, writing one replica
    column: each replay, after eager changes to the cache, equals an eager
    kvck_checksum_blocks with its own workspace.  Twenty caches under the
    simple schedule keep per-group partials in the library's scratch array
    and reduce them in a second launch; three caches form one group.  A first
    call outside the capture looks up the scratch array's address."""
    if schedule != "default":
        monkeypatch.setenv("KVCK_SCHEDULE", schedule)
    log(f"[graphs] allocation-free {schedule} caches={ncaches}")
    rng = np.random.default_rng(42)
    req, nb = wl.page_requests(rng, [100, 37, 300, 5], 16, start_pos=[0, 1, 0, 0], spare_frac=0.2)
    layers = list(range(0, 2 * ncaches, 2))
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 4, 64), "bf16"))
             for _ in layers]
    pc = kvck.prepare_caches(pools, "NHD", layers)
    bt, nbt, sp, nt = req_tensors(req)
    values = torch.zeros((req.num_reqs, req.max_blocks, 2), dtype=torch.uint64, device=DEV)
    col = values[..., 1]
    kvck.kvck_checksum_blocks_noalloc(pc, None, None, bt, nbt, sp, nt, col)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvck.kvck_checksum_blocks_noalloc(pc, None, None, bt, nbt, sp, nt, col)
    listed = req.listed()
    for rep in range(4):
        values.view(torch.int64).zero_()
        r, k = listed[(3 * rep) % len(listed)]
        b = int(req.block_table[r, k])
        pools[rep % len(pools)].view(torch.int16)[rep % 2, b, 0, rep % 4, 5] ^= 1 << (rep + 2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = values.cpu().view(torch.int64).numpy()
        want = kvck.kvck_checksum_blocks(pc, None, None, bt, nbt, sp, nt).cpu().view(torch.int64).numpy()
        for rr, kk in listed:
            assert got[rr, kk, 1] == want[rr, kk], (rep, rr, kk)
        assert not got[..., 0].any()

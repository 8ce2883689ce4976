"""Helpers of the GPU parity tests: move seeded inputs to the device, call the
HIP path through the C ABI binding, and compute oracle values of sampled
positions from the bytes the device holds."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl

DEV = "cuda"
SENTINEL = 0x5A5A5A5A5A5A5A5A


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a device tensor as an unsigned numpy array of the same shape."""
    es = t.element_size()
    dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[es]
    npdt = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[es]
    return t.contiguous().view(dt).cpu().numpy().view(npdt)


def to_device_bits(a: np.ndarray) -> torch.Tensor:
    dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[a.dtype.itemsize]
    npdt = {1: np.uint8, 2: np.int16, 4: np.int32}[a.dtype.itemsize]
    return torch.from_numpy(np.ascontiguousarray(a).view(npdt)).to(DEV).view(dt)


def req_tensors(req: wl.Requests):
    return (torch.from_numpy(req.block_table).to(DEV), torch.from_numpy(req.num_blocks).to(DEV),
            torch.from_numpy(req.start_pos).to(DEV), torch.from_numpy(req.num_tokens).to(DEV))


def gpu_blocks(pools, layout, layer_numbers, req: wl.Requests, bases=None, head_begin=0, head_count=None,
               out=None, accumulate=False, check=True, stream=None, workspace=None):
    bt, nb, sp, nt = req_tensors(req)
    if out is None:
        out = torch.full((req.num_reqs, req.max_blocks), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64)
    res = kvck.kvck_checksum_blocks(pools, layout, layer_numbers, bt, nb, sp, nt, global_head_base=bases,
                                    head_begin=head_begin, head_count=head_count, out=out, accumulate=accumulate,
                                    check=check, stream=stream, workspace=workspace)
    torch.cuda.synchronize()
    return res.cpu().numpy().view(np.uint64).reshape(req.num_reqs, req.max_blocks)


def oracle_at(pools, layout, layer_numbers, req: wl.Requests, positions, bases=None, head_begin=0,
              head_count=None):
    """Oracle checksums of the listed positions ``[(r, k), ..]`` computed from
    host copies of just the blocks those positions name."""
    ids = sorted({int(req.block_table[r, k]) for r, k in positions})
    remap = {b: i for i, b in enumerate(ids)}
    idx = torch.tensor(ids, dtype=torch.int64, device=pools[0].device)
    mini = []
    for p in pools:
        sub = p.index_select(0 if layout == "MLA" else 1, idx)
        mini.append(to_host_bits(sub))
    n = len(pools)
    bases = [head_begin] * n if bases is None else list(bases)
    out = {}
    for r, k in positions:
        out[(r, k)] = oracle.kv_checksum.checksum_position(
            mini, layout, layer_numbers, bases, remap[int(req.block_table[r, k])], int(req.start_pos[r]) + k,
            int(req.num_tokens[r]), head_begin, head_count)
    return out


def sample_positions(req: wl.Requests, n, seed=0, include_tails=True):
    """``n`` random listed positions plus (optionally) every request's last one."""
    rng = np.random.default_rng(seed)
    allpos = req.listed()
    pick = [allpos[i] for i in rng.choice(len(allpos), min(n, len(allpos)), replace=False)]
    if include_tails:
        pick += [(r, int(req.num_blocks[r]) - 1) for r in range(req.num_reqs) if req.num_blocks[r] > 0]
    return sorted(set(pick))


def assert_match(got: np.ndarray, want: dict, what=""):
    bad = [(rk, int(got[rk]), v) for rk, v in want.items() if int(got[rk]) != v]
    assert not bad, f"{what}: {len(bad)} of {len(want)} positions differ, first {bad[:3]}"


def assert_unlisted_untouched(got: np.ndarray, req: wl.Requests):
    for r in range(req.num_reqs):
        tail = got[r, int(req.num_blocks[r]):]
        assert np.all(tail == np.uint64(SENTINEL)), f"request {r}: unlisted entries were written"

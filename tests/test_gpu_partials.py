"""Partials the checksum page describes, on one GPU (GPU).

* Several caches of one layer (an attention KV cache and its indexer cache)
  number their heads consecutively: calls over each, with the heads' global
  bases, add up to the checksum of both.
* Replicated KV (GQA with more TP ranks than KV heads): every replica of a head
  computes the same partial, so partials are kept per replica; one replica of
  each head summed gives the full checksum.
* A Mamba layer whose TP split is unknown has one slice per TP shard: the
  shard's whole state is one slice, numbered by the shard's rank.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, gpu_blocks, log, to_device_bits

pytestmark = pytest.mark.gpu


def test_kv_and_indexer_caches_of_one_layer():
    log("[partials] KV + indexer caches")
    rng = np.random.default_rng(30)
    req, nb = wl.page_requests(rng, [120, 33, 7], 16, spare_frac=0.2)
    layers = [0, 1, 2, 3]
    kv = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16") for _ in layers]
    idx = [wl.host_random_bits(rng, wl.pool_shape("MLA", nb, 16, 1, 128), "fp8") for _ in layers]   # 1 head
    got = gpu_blocks([to_device_bits(p) for p in kv], "HND", layers, req, bases=[0] * 4)
    out = torch.from_numpy(got.view(np.int64).copy()).to(DEV).view(torch.uint64)
    both = gpu_blocks([to_device_bits(p) for p in idx], "MLA", layers, req, bases=[8] * 4, out=out, accumulate=True)
    with np.errstate(over="ignore"):
        want = (oracle.checksum_blocks(kv, "HND", layers, [0] * 4, req.block_table, req.num_blocks, req.start_pos,
                                       req.num_tokens)
                + oracle.checksum_blocks(idx, "MLA", layers, [8] * 4, req.block_table, req.num_blocks,
                                         req.start_pos, req.num_tokens))
    for r, k in req.listed():
        assert both[r, k] == want[r, k]


def test_replicated_kv_heads():
    """8 KV heads on 16 TP ranks: 2 replicas per head, rank r holds head r // 2
    with replica index r % 2 (each rank's pool holds only its head)."""
    log("[partials] replicated KV")
    rng = np.random.default_rng(31)
    req, nb = wl.page_requests(rng, [90, 40], 16, spare_frac=0.2)
    layers = [0, 1, 2]
    full = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 64), "bf16") for _ in layers]
    want = oracle.checksum_blocks(full, "HND", layers, [0] * 3, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    by_key = {}
    for rank in range(16):
        head, replica = rank // 2, rank % 2
        shard = [to_device_bits(np.ascontiguousarray(p[:, :, head:head + 1])) for p in full]
        part = gpu_blocks(shard, "HND", layers, req, bases=[head] * 3)
        by_key.setdefault((2, replica), []).append(part)
    # replicas agree head by head; one replica of every head sums to the full checksum
    for a, b in zip(by_key[(2, 0)], by_key[(2, 1)]):
        assert np.array_equal(a, b)
    for key in by_key:
        with np.errstate(over="ignore"):
            tot = sum(by_key[key][1:], by_key[key][0].copy())
        for r, k in req.listed():
            assert tot[r, k] == want[r, k]


def test_mamba_layer_with_unknown_split_is_one_slice_per_shard():
    log("[partials] Mamba unknown split")
    rng = np.random.default_rng(32)
    layers = [1, 3]
    shapes = [(6, 8, 4), (6, 2, 16)]
    elems = ["fp32", "fp16"]
    tp_rank = 3
    hs = [[wl.host_random_bits(rng, (5,) + s, e) for s, e in zip(shapes, elems)] for _ in layers]
    # the shard's whole state of a slot is one slice: view every state as one row
    one_row = [[a.reshape(a.shape[0], 1, -1) for a in l] for l in hs]
    slots = np.array([4, 0, 2], np.int32)
    got = kvck.kvck_checksum_states([[to_device_bits(a) for a in l] for l in one_row], layers,
                                    torch.from_numpy(slots).to(DEV), global_row_base=tp_rank, check=True)
    want = oracle.checksum_states(one_row, layers, [tp_rank] * 2, slots)
    assert np.array_equal(got.cpu().numpy(), want)
    # it differs from the known-split checksum of the same bytes (rows as slices)
    rows = oracle.checksum_states(hs, layers, [0, 0], slots)
    assert not np.array_equal(rows, want)

"""Faults forced from the host, detected by the HIP path (GPU).

The checksum exists to catch a KV transfer that went wrong (vLLM API page
"vllm.distributed.kv_transfer.kv_checksum.checksum", the paragraphs on what a
checksum detects and on TP/PP partials).  Each fault is made on the device
with torch indexing, the GPU recomputes, and the test checks

* a flipped bit in a valid slot changes exactly its own position (a piece's
  weight m(2j+1) is odd, hence invertible mod 2^64, so this always holds), and
  the new value equals the oracle's on the changed bytes;
* a flipped bit in an excluded slot, or in a block no request lists, changes
  nothing;
* swapped block-table entries, swapped layer numbers, two heads' data
  exchanged, and a missing TP-shard partial all change the affected
  positions (and the swapped table equals the oracle's on it).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_kvck_amd as kvck  # noqa: F401  (the extension must load)
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import gpu_blocks, log, oracle_at, to_device_bits

pytestmark = pytest.mark.gpu

BS, NH, D = 16, 8, 128
LAYERS = [0, 1, 2, 3]


def _case(seed=50):
    rng = np.random.default_rng(seed)
    lengths = [200, 37, 130, 16, 75, 300]
    req, nb = wl.page_requests(rng, lengths, BS, start_pos=[0, 1, 0, 0, 2, 0], extra_blocks=[0, 0, 1, 0, 0, 1],
                               spare_frac=0.3)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("HND", nb, BS, NH, D), "bf16")) for _ in LAYERS]
    return rng, req, nb, pools


def _valid(req, r, k):
    pos = int(req.start_pos[r]) + k
    return min(BS, max(0, int(req.num_tokens[r]) - pos * BS))


def test_bit_flips_change_exactly_their_position():
    log("[faults] bit flips")
    rng, req, nb, pools = _case()
    base = gpu_blocks(pools, "HND", LAYERS, req)
    valid_pos = [(r, k) for r, k in req.listed() if _valid(req, r, k) > 0]
    for trial in range(6):
        r, k = valid_pos[int(rng.integers(0, len(valid_pos)))]
        b = int(req.block_table[r, k])
        li, plane, h = int(rng.integers(0, len(LAYERS))), int(rng.integers(0, 2)), int(rng.integers(0, NH))
        slot = int(rng.integers(0, _valid(req, r, k)))
        elem, bit = int(rng.integers(0, D)), int(rng.integers(0, 16))
        view = pools[li].view(torch.int16)
        view[plane, b, h, slot, elem] ^= (1 << bit) if bit < 15 else -(1 << 15)
        got = gpu_blocks(pools, "HND", LAYERS, req)
        changed = [(rr, kk) for rr, kk in req.listed() if got[rr, kk] != base[rr, kk]]
        assert changed == [(r, k)], (trial, changed)
        want = oracle_at(pools, "HND", LAYERS, req, [(r, k)])
        assert int(got[r, k]) == want[(r, k)], trial
        view[plane, b, h, slot, elem] ^= (1 << bit) if bit < 15 else -(1 << 15)   # undo
    assert np.array_equal(gpu_blocks(pools, "HND", LAYERS, req), base)


def test_flips_outside_the_checksummed_bytes_change_nothing():
    log("[faults] excluded slots and unlisted blocks")
    rng, req, nb, pools = _case(51)
    base = gpu_blocks(pools, "HND", LAYERS, req)
    listed_blocks = {int(req.block_table[r, k]) for r, k in req.listed()}
    spare = [b for b in range(nb) if b not in listed_blocks]
    # a slot at or past num_tokens of a partly valid position
    part = [(r, k) for r, k in req.listed() if 0 < _valid(req, r, k) < BS]
    assert part and spare
    r, k = part[0]
    b = int(req.block_table[r, k])
    for p in pools:
        p.view(torch.int16)[:, b, :, _valid(req, r, k):, :] ^= 0x1234
        p.view(torch.int16)[:, spare[0], :, :, :] ^= 0x0F0F
    assert np.array_equal(gpu_blocks(pools, "HND", LAYERS, req), base)


def test_swapped_table_entries_layers_and_heads_are_detected():
    log("[faults] swaps")
    rng, req, nb, pools = _case(52)
    base = gpu_blocks(pools, "HND", LAYERS, req)
    # two block-table entries of one request exchanged
    r = 0
    k1, k2 = 1, 5
    sw = wl.Requests(BS, req.num_tokens, req.start_pos, req.num_blocks, req.block_table.copy())
    sw.block_table[r, [k1, k2]] = sw.block_table[r, [k2, k1]]
    got = gpu_blocks(pools, "HND", LAYERS, sw)
    assert got[r, k1] != base[r, k1] and got[r, k2] != base[r, k2]
    want = oracle_at(pools, "HND", LAYERS, sw, [(r, k1), (r, k2)])
    assert int(got[r, k1]) == want[(r, k1)] and int(got[r, k2]) == want[(r, k2)]
    valid_pos = [(rr, kk) for rr, kk in req.listed() if _valid(req, rr, kk) > 0]
    # two layers' numbers exchanged (pools handed over in the wrong order)
    got = gpu_blocks([pools[1], pools[0]] + pools[2:], "HND", LAYERS, req)
    assert all(got[rk] != base[rk] for rk in valid_pos)
    # two heads' data exchanged in one layer
    p = pools[2].view(torch.int16)
    saved = p.clone()
    p[:, :, [3, 6]] = saved[:, :, [6, 3]]
    got = gpu_blocks(pools, "HND", LAYERS, req)
    assert all(got[rk] != base[rk] for rk in valid_pos)
    p.copy_(saved)
    assert np.array_equal(gpu_blocks(pools, "HND", LAYERS, req), base)


def test_missing_shard_partial_is_detected():
    log("[faults] missing shard")
    rng, req, nb, pools = _case(53)
    full = gpu_blocks(pools, "HND", LAYERS, req)
    parts = [gpu_blocks(pools, "HND", LAYERS, req, bases=[h] * len(LAYERS), head_begin=h, head_count=2)
             for h in range(0, NH, 2)]
    valid_pos = [(r, k) for r, k in req.listed() if _valid(req, r, k) > 0]
    with np.errstate(over="ignore"):
        allsum = parts[0] + parts[1] + parts[2] + parts[3]
        for drop in range(4):
            three = sum((parts[i] for i in range(4) if i != drop), np.zeros_like(full))
            assert all(three[rk] != full[rk] for rk in valid_pos), drop
    assert all(allsum[rk] == full[rk] for rk in req.listed())

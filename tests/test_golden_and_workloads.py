"""Page-printed constants, the oracle's regression values, and the shapes of
the seeded workloads (CPU only)."""

import hashlib
import json
import os

import numpy as np

import oracle
from oracle import brute
from paged_kv_cache_kvck_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_page_constants():
    g = _load("page_constants.json")
    assert oracle.MAX_KV_HEADS_PER_LAYER == g["MAX_KV_HEADS_PER_LAYER"]["value"]
    assert oracle.BLOCK_CHECKSUM_BYTES == g["BLOCK_CHECKSUM_BYTES"]["value"]
    w = wl.gpt2()
    assert list(w.shape) == g["gpt2_pool_shape"]["value"]
    assert int(np.prod(w.shape)) * wl.ELEM_BYTES[w.elem] == g["gpt2_pool_tensor_bytes"]["value"]


def test_tiny_regression_and_brute():
    g = _load("tiny_oracle.json")
    w = wl.tiny()
    pools = w.host_pools()
    assert hashlib.sha256(b"".join(p.tobytes() for p in pools)).hexdigest() == g["pool_sha256"]
    assert w.req.block_table[0].tolist() == g["block_table"]
    out = oracle.checksum_blocks(pools, w.layout, w.layer_numbers, w.bases, w.req.block_table,
                                 w.req.num_blocks, w.req.start_pos, w.req.num_tokens)
    assert [str(int(x)) for x in out[0, :4]] == g["checksums"]
    b = brute.blocks(pools, w.layout, w.layer_numbers, w.bases, w.req.block_table,
                     w.req.num_blocks, w.req.start_pos, w.req.num_tokens)
    assert [str(b[(0, k)]) for k in range(4)] == g["checksums"]


def test_tiny_structure():
    w = wl.tiny()
    assert w.shape == (2, 16, 16, 2, 64)
    assert int(w.req.num_tokens[0]) == 50 and int(w.req.num_blocks[0]) == 4
    ids = w.req.block_table[0, :4]
    assert len(set(ids.tolist())) == 4 and ids.min() >= 0 and ids.max() < 16
    assert w.valid_bytes() == 51200


def test_request_paging():
    rng = np.random.default_rng(0)
    lengths = wl.uniform_lengths(rng, 64, 128, 2048)
    assert lengths.min() >= 128 and lengths.max() <= 2048
    req, nb = wl.page_requests(rng, lengths, 16, pool_blocks=18545)
    ids = np.concatenate([req.block_table[r, :req.num_blocks[r]] for r in range(64)])
    assert len(np.unique(ids)) == ids.size and ids.max() < nb
    for r in range(64):
        assert req.num_blocks[r] * 16 >= lengths[r] > (req.num_blocks[r] - 1) * 16


def test_repage_roundtrip():
    rng = np.random.default_rng(1)
    lengths = [37, 5, 64]
    r16, n16 = wl.page_requests(rng, lengths, 16, spare_frac=0.3)
    r64, n64 = wl.page_requests(rng, lengths, 64, spare_frac=0.3)
    a = wl.host_random_bits(rng, wl.pool_shape("NHD", n16, 16, 3, 8), "bf16")
    b = np.zeros(wl.pool_shape("HND", n64, 64, 3, 8), np.uint16)
    wl.repage_numpy(a, "NHD", r16, b, "HND", r64)
    for r, n in enumerate(lengths):
        for t in range(n):
            assert np.array_equal(a[:, r16.block_table[r, t // 16], t % 16],
                                  b[:, r64.block_table[r, t // 64], :, t % 64])


def test_workload_sizes():
    assert abs(wl.gpt2().valid_bytes() / 2.57e9 - 1) < 0.1
    w3 = wl.llama3_8b()
    assert abs(w3.valid_bytes() / 146e9 - 1) < 0.05
    assert w3.layout == "HND" and w3.shape[1:] == (w3.pool_blocks, 8, 16, 128)
    shard = wl.llama3_8b(head_begin=2, head_count=2, global_base=2)
    assert shard.valid_bytes() * 4 == w3.valid_bytes()
    attn, mamba = wl.hybrid()
    assert abs(attn.valid_bytes() / 54.8e9 - 1) < 0.1
    assert mamba.valid_bytes() == 128 * 24 * 64 * (128 * 16 * 4 + 4 * 256 * 2)

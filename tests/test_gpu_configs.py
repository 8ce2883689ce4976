"""Full-size workloads on the GPU, in the launch configuration the benchmark
times: sampled positions against the oracle (computed one by one from host
copies of the blocks they name) and properties that hold at any size
(additivity over block sizes, layout independence, TP-shard and layer-split
partial sums)."""

import gc

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import (DEV, assert_match, assert_unlisted_untouched, gpu_blocks, log, oracle_at, sample_positions,
                         to_host_bits)

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _req_sums(vals, req):
    with np.errstate(over="ignore"):
        return np.array([vals[r, :int(req.num_blocks[r])].sum(dtype=np.uint64) for r in range(req.num_reqs)])


def test_gpt2_shaped_full():
    w = wl.gpt2()
    log(f"[gpt2] pools {w.shape} x {w.num_layers}")
    pools = w.device_pools()
    got = gpu_blocks(pools, w.layout, w.layer_numbers, w.req)
    pos = sample_positions(w.req, 160, seed=1)
    assert_match(got, oracle_at(pools, w.layout, w.layer_numbers, w.req, pos), "gpt2")
    assert_unlisted_untouched(got, w.req)
    del pools
    _free()


def test_llama3_8b_shaped_full_and_tp_shard():
    w = wl.llama3_8b()
    log(f"[llama3] pools {w.shape} x {w.num_layers}")
    pools = w.device_pools()
    got = gpu_blocks(pools, w.layout, w.layer_numbers, w.req)
    pos = sample_positions(w.req, 64, seed=3)
    assert_match(got, oracle_at(pools, w.layout, w.layer_numbers, w.req, pos), "llama3 full")
    assert_unlisted_untouched(got, w.req)
    # TP = 4 shard over heads {2, 3}, global numbering from 2
    log("[llama3] shard heads 2..3")
    shard = gpu_blocks(pools, w.layout, w.layer_numbers, w.req, bases=[2] * 32, head_begin=2, head_count=2)
    spos = sample_positions(w.req, 48, seed=4, include_tails=False)
    assert_match(shard, oracle_at(pools, w.layout, w.layer_numbers, w.req, spos, bases=[2] * 32, head_begin=2,
                                  head_count=2), "llama3 shard")
    # every position: the four shards sum to the full checksum
    with np.errstate(over="ignore"):
        tot = shard.copy()
        for h in (0, 4, 6):
            tot = tot + gpu_blocks(pools, w.layout, w.layer_numbers, w.req, bases=[h] * 32, head_begin=h,
                                   head_count=2)
    for r, k in w.req.listed():
        assert tot[r, k] == got[r, k], (r, k)
    del pools
    _free()



def test_llama3_8b_fused_copy_full():
    """The fused save and load in the benchmark's configuration: the llama3-shaped
    pools (32 layers), the first 128 requests, positions visited grouped by block
    id.  The save's checksums equal the checksum call's at every position and the
    oracle's at sampled ones; sampled staging entries hold the pool rows of their
    valid slots; a load into the zeroed pools restores the sampled blocks' valid
    slots and gives the same checksums."""
    w = wl.llama3_8b()
    log(f"[llama3 copy] pools {w.shape} x {w.num_layers}")
    pools = w.device_pools()
    r0 = w.req
    half = r0.num_reqs // 2
    req = wl.Requests(r0.block_size, r0.num_tokens[:half].copy(), r0.start_pos[:half].copy(),
                      r0.num_blocks[:half].copy(), np.ascontiguousarray(r0.block_table[:half]))
    bt, nbt, sp, nt = (torch.from_numpy(x).to(DEV) for x in (req.block_table, req.num_blocks, req.start_pos,
                                                             req.num_tokens))
    per = kvck.kvck_staging_bytes(pools[0], w.layout, w.num_layers)
    entries = int(req.num_blocks.sum())
    staging = torch.empty(entries * per, dtype=torch.uint8, device=DEV)
    saved = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, w.layout, w.layer_numbers, bt, nbt, sp, nt,
                                           staging, check=True).cpu().numpy()
    ref = gpu_blocks(pools, w.layout, w.layer_numbers, req)
    for r, k in req.listed():
        assert saved[r, k] == ref[r, k], (r, k)
    pos = sample_positions(req, 32, seed=12)
    assert_match(saved, oracle_at(pools, w.layout, w.layer_numbers, req, pos), "llama3 save")
    # staging images of sampled positions: [plane][head][slot][row] per cache, valid slots only
    first = np.concatenate([[0], np.cumsum(req.num_blocks.astype(np.int64))])
    img = per // w.num_layers
    bs, nh, rb = req.block_size, w.num_heads, w.head_size * 2
    kept = {}
    for r, k in pos:
        e = int(first[r]) + k
        b = int(req.block_table[r, k])
        v = oracle.num_valid_tokens(int(req.start_pos[r]) + k, bs, int(req.num_tokens[r]))
        blocks = [to_host_bits(p[:, b]).view(np.uint8).reshape(2, nh, bs, rb) for p in pools]
        kept[(r, k)] = (b, v, blocks)
        ent = staging[e * per:(e + 1) * per].cpu().numpy().reshape(w.num_layers, 2, nh, bs, rb)
        for c in range(w.num_layers):
            assert np.array_equal(ent[c][:, :, :v], blocks[c][:, :, :v]), (r, k, c)
    # load into the zeroed pools
    for p in pools:
        p.zero_()
    loaded = kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_LOAD, pools, w.layout, w.layer_numbers, bt, nbt, sp, nt,
                                            staging, check=True).cpu().numpy()
    for r, k in req.listed():
        assert loaded[r, k] == saved[r, k], (r, k)
    for (r, k), (b, v, blocks) in kept.items():
        for c, p in enumerate(pools):
            back = to_host_bits(p[:, b]).view(np.uint8).reshape(2, nh, bs, rb)
            assert np.array_equal(back[:, :, :v], blocks[c][:, :, :v]), (r, k, c)
            assert not back[:, :, v:].any(), (r, k, c)
    del pools, staging
    _free()

def test_invariance_set():
    """Config-2 tokens re-paged at block size 64, in HND, as fp8 bits, and an
    MLA 61 x 576 latent cache: per-request sums agree across block sizes and
    layouts, and sampled positions of each variant match the oracle."""
    base = wl.gpt2()
    log("[invariance] gpt2 bs16 NHD")
    p16 = base.device_pools()
    c16 = gpu_blocks(p16, "NHD", base.layer_numbers, base.req)
    ref = _req_sums(c16, base.req)
    lengths = base.req.num_tokens
    # (i) block size 64, NHD
    r64, n64 = wl.page_requests(np.random.default_rng(40), lengths, 64, spare_frac=0.05)
    log("[invariance] bs64 NHD")
    p64 = [torch.zeros(wl.pool_shape("NHD", n64, 64, 12, 64), dtype=p16[0].dtype, device=DEV) for _ in p16]
    for s, d in zip(p16, p64):
        wl.repage_torch(s, "NHD", base.req, d, "NHD", r64)
    c64 = gpu_blocks(p64, "NHD", base.layer_numbers, r64)
    assert np.array_equal(_req_sums(c64, r64), ref)
    assert_match(c64, oracle_at(p64, "NHD", base.layer_numbers, r64, sample_positions(r64, 40, seed=5)), "bs64")
    del p64
    # (ii) HND at block size 16, same block ids
    log("[invariance] bs16 HND")
    ph = [p.permute(0, 1, 3, 2, 4).contiguous() for p in p16]
    ch = gpu_blocks(ph, "HND", base.layer_numbers, base.req)
    assert np.array_equal(ch, c16)
    del ph, p16
    _free()
    # (iii) fp8 bits, P = head/4, block sizes 16 and 64
    log("[invariance] fp8")
    f = wl.gpt2(seed=41, elem="fp8")
    f16 = f.device_pools()
    cf16 = gpu_blocks(f16, "NHD", f.layer_numbers, f.req)
    rf64, nf64 = wl.page_requests(np.random.default_rng(42), f.req.num_tokens, 64, spare_frac=0.05)
    f64 = [torch.zeros(wl.pool_shape("NHD", nf64, 64, 12, 64), dtype=torch.uint8, device=DEV) for _ in f16]
    for s, d in zip(f16, f64):
        wl.repage_torch(s, "NHD", f.req, d, "NHD", rf64)
    cf64 = gpu_blocks(f64, "NHD", f.layer_numbers, rf64)
    assert np.array_equal(_req_sums(cf16, f.req), _req_sums(cf64, rf64))
    assert_match(cf16, oracle_at(f16, "NHD", f.layer_numbers, f.req, sample_positions(f.req, 40, seed=6)), "fp8")
    # block size 64 position by position too (the sums above cannot place an error)
    assert_match(cf64, oracle_at(f64, "NHD", f.layer_numbers, rf64, sample_positions(rf64, 40, seed=9)), "fp8 bs64")
    assert_unlisted_untouched(cf64, rf64)
    del f16, f64
    _free()
    # (iv) MLA: 61 layers x one latent head of 576 bf16, block sizes 64 and 16
    log("[invariance] MLA")
    m = wl.mla()
    m64 = m.device_pools()
    cm64 = gpu_blocks(m64, "MLA", m.layer_numbers, m.req)
    assert_match(cm64, oracle_at(m64, "MLA", m.layer_numbers, m.req, sample_positions(m.req, 24, seed=7)), "mla64")
    rm16, nm16 = wl.page_requests(np.random.default_rng(43), m.req.num_tokens, 16, spare_frac=0.05)
    m16 = [torch.zeros((nm16, 16, 576), dtype=m64[0].dtype, device=DEV) for _ in m64]
    for s, d in zip(m64, m16):
        wl.repage_torch(s, "MLA", m.req, d, "MLA", rm16)
    cm16 = gpu_blocks(m16, "MLA", m.layer_numbers, rm16)
    assert np.array_equal(_req_sums(cm64, m.req), _req_sums(cm16, rm16))
    assert_match(cm16, oracle_at(m16, "MLA", m.layer_numbers, rm16, sample_positions(rm16, 40, seed=10)), "mla16")
    assert_unlisted_untouched(cm16, rm16)
    del m64, m16
    _free()


def test_hybrid_attention_and_mamba():
    attn, mamba = wl.hybrid()
    log("[hybrid] attention group")
    pools = attn.device_pools()
    got = gpu_blocks(pools, attn.layout, attn.layer_numbers, attn.req)
    pos = sample_positions(attn.req, 48, seed=8)
    assert_match(got, oracle_at(pools, attn.layout, attn.layer_numbers, attn.req, pos), "hybrid attention")
    del pools
    _free()
    log("[hybrid] mamba group")
    states = mamba.device_states()
    sid = torch.from_numpy(mamba.slot_ids).to(DEV)
    g = kvck.kvck_checksum_states(states, mamba.layer_numbers, sid, check=True).cpu().numpy()
    # oracle on 16 requests, from host copies of their slots
    pick = list(range(0, 128, 8))
    slots = mamba.slot_ids[pick]
    host = [[to_host_bits(s.index_select(0, torch.from_numpy(slots.astype(np.int64)).to(DEV))) for s in l]
            for l in states]
    want = oracle.checksum_states(host, mamba.layer_numbers, mamba.bases, np.arange(len(pick)))
    assert np.array_equal(g[pick], want)
    # row shards and layer splits sum to the whole, for every request
    with np.errstate(over="ignore"):
        rows = (kvck.kvck_checksum_states(states, mamba.layer_numbers, sid, row_begin=0, row_count=16,
                                          global_row_base=0).cpu().numpy()
                + kvck.kvck_checksum_states(states, mamba.layer_numbers, sid, row_begin=16, row_count=48,
                                            global_row_base=16).cpu().numpy())
        layers = (kvck.kvck_checksum_states(states[:10], mamba.layer_numbers[:10], sid).cpu().numpy()
                  + kvck.kvck_checksum_states(states[10:], mamba.layer_numbers[10:], sid).cpu().numpy())
    assert np.array_equal(rows, g) and np.array_equal(layers, g)
    del states
    _free()

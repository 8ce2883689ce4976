"""Replica-keyed output columns (GPU).

The checksum page keys a worker's partial checksums by the replica key
(replicas, replica_index) of the layers they cover: a group's values are
(num_positions, len(replica_keys)), one column per key, and what is offloaded
with a block is its row summed (class KVChecksumGroup, attribute ReplicaKey).
Every checksum entry point writes its results ``out_stride`` elements apart,
so a call given ``values[..., c]`` fills column c.  Each case fills one
column of a sentinel-filled array and checks that column against the oracle
and every other entry for the sentinel, through each way the library writes
results: calls planned in place or from a position list, written directly or
summed over task groups by each second-pass kernel, merged rows streamed
across tasks, element-transposed planes, the fused copy, the allocation-free
call, and Mamba states.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, SENTINEL, log, req_tensors, to_device_bits

pytestmark = pytest.mark.gpu

COLUMNS = 3


def _values(shape):
    return torch.full(shape + (COLUMNS,), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64)


def _check_column(values, col, req, want):
    """Column ``col`` holds ``want`` at every listed position; every other
    entry of the array still holds the sentinel."""
    v = values.cpu().view(torch.int64).numpy().view(np.uint64)
    listed = np.zeros(v.shape[:2], bool)
    for r, k in req.listed():
        listed[r, k] = True
        assert int(v[r, k, col]) == int(want[r, k]), (r, k)
    keep = np.ones(v.shape, bool)
    keep[..., col] = ~listed
    assert np.all(v[keep] == np.uint64(SENTINEL)), "entries outside the listed column positions were written"


# name, layout, caches, heads, head_size, block_size, request lengths, switches
BLOCK_CASES = [
    ("dense_direct", "NHD", 2, 4, 64, 16, [70, 33, 16, 5], {}),
    ("dense_groups", "NHD", 70, 2, 32, 16, [40, 17, 9], {"KVCK_SCHEDULE": "simple"}),
    ("planned_direct", "HND", 2, 4, 64, 16, [70, 33, 16, 5], {"KVCK_PLAN": "compact"}),
    ("planned_groups", "HND", 8, 2, 64, 16, [90, 20, 3], {"KVCK_PLAN": "compact", "KVCK_SCHEDULE": "simple"}),
    ("planned_many_groups", "HND", 70, 2, 32, 16, [40, 17, 9],
     {"KVCK_PLAN": "compact", "KVCK_SCHEDULE": "simple"}),
    ("merged_stream_direct", "MLA", 1, 1, 576, 16, [150, 64, 31], {"KVCK_PLAN": "compact",
                                                                   "KVCK_SCHEDULE": "pipelined"}),
    ("merged_stream_groups", "MLA", 4, 1, 576, 16, [150, 64, 31], {"KVCK_PLAN": "compact",
                                                                   "KVCK_SCHEDULE": "pipelined"}),
    ("pipelined_planes", "HND", 6, 2, 128, 16, [200, 45, 16], {"KVCK_PLAN": "compact",
                                                               "KVCK_SCHEDULE": "pipelined"}),
    ("plan_many_requests", "NHD", 1, 2, 64, 16, "many", {"KVCK_PLAN": "compact"}),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
@pytest.mark.parametrize("col", [0, 2])
def test_blocks_fill_one_replica_column(case, col, monkeypatch):
    name, layout, ncaches, nh, d, bs, lengths, env = case
    log(f"[replicas] blocks {name} column {col}")
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    rng = np.random.default_rng(zlib.crc32(f"replica{name}".encode()))
    if lengths == "many":
        lengths = rng.integers(1, 2 * bs + 1, size=1100)   # more than 1024 requests: the two-launch plan
    req, nb = wl.page_requests(rng, lengths, bs, start_pos=[1] + [0] * (len(lengths) - 1),
                               extra_blocks=[0, 1] + [0] * (len(lengths) - 2), spare_frac=0.2)
    layers = [3 * i + 1 for i in range(ncaches)]
    bases = [0 if layout == "MLA" else nh * (i % 3) for i in range(ncaches)]
    host = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), "bf16") for _ in layers]
    want = oracle.checksum_blocks(host, layout, layers, bases, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    values = _values((req.num_reqs, req.max_blocks))
    bt, nbt, sp, nt = req_tensors(req)
    dev_pools = [to_device_bits(p) for p in host]
    got = kvck.kvck_checksum_blocks(dev_pools, layout, layers, bt, nbt, sp, nt, global_head_base=bases,
                                    out=values[..., col], check=True)
    assert got.data_ptr() == values[..., col].data_ptr()
    torch.cuda.synchronize()
    _check_column(values, col, req, want)
    # accumulate into the same column: every listed entry doubles, nothing else moves
    kvck.kvck_checksum_blocks(dev_pools, layout, layers, bt, nbt, sp, nt, global_head_base=bases,
                              out=values[..., col], accumulate=True, check=True)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):
        _check_column(values, col, req, want * np.uint64(2))


def test_transposed_planes_fill_one_replica_column(monkeypatch):
    """K_TRANS then V_TRANS accumulated into column 1 equal the oracle on the
    HND pools holding the same tokens (planned and in place)."""
    log("[replicas] element-transposed planes")
    rng = np.random.default_rng(71)
    bs, nh, d = 16, 4, 64
    req, nb = wl.page_requests(rng, [60, 16, 9], bs, extra_blocks=[1, 0, 0], spare_frac=0.3)
    layers = [0, 5]
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, nh, d), "bf16") for _ in layers]
    want = oracle.checksum_blocks(hp, "HND", layers, [0, 0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    kt = [to_device_bits(np.ascontiguousarray(p[0].transpose(0, 1, 3, 2))) for p in hp]
    vt = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    bt, nbt, sp, nt = req_tensors(req)
    for plan in ("dense", "compact"):
        monkeypatch.setenv("KVCK_PLAN", plan)
        values = _values((req.num_reqs, req.max_blocks))
        col = values[..., 1]
        kvck.kvck_checksum_blocks(kt, "K_TRANS", layers, bt, nbt, sp, nt, out=col, check=True)
        kvck.kvck_checksum_blocks(vt, "V_TRANS", layers, bt, nbt, sp, nt, out=col, accumulate=True, check=True)
        torch.cuda.synchronize()
        v = values.cpu().view(torch.int64).numpy().view(np.uint64)
        for r, k in req.listed():
            assert int(v[r, k, 1]) == int(want[r, k]), (plan, r, k)
        assert np.all(v[..., 0] == np.uint64(SENTINEL)) and np.all(v[..., 2] == np.uint64(SENTINEL))


@pytest.mark.parametrize("layout,nh,d", [("HND", 4, 64), ("MLA", 1, 576)])
def test_fused_copy_fills_one_replica_column(layout, nh, d):
    log(f"[replicas] fused copy {layout}")
    rng = np.random.default_rng(zlib.crc32(f"replicacopy{layout}".encode()))
    bs = 16
    req, nb = wl.page_requests(rng, [100, 40, 7], bs, extra_blocks=[0, 1, 0], spare_frac=0.2)
    layers = [2, 6, 7]
    host = [wl.host_random_bits(rng, wl.pool_shape(layout, nb, bs, nh, d), "bf16") for _ in layers]
    want = oracle.checksum_blocks(host, layout, layers, [0] * 3, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    pools = [to_device_bits(p) for p in host]
    per = kvck.kvck_staging_bytes(pools[0], layout, len(layers))
    staging = torch.zeros(int(req.num_blocks.sum()) * per, dtype=torch.uint8, device=DEV)
    values = _values((req.num_reqs, req.max_blocks))
    bt, nbt, sp, nt = req_tensors(req)
    kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, pools, layout, layers, bt, nbt, sp, nt, staging,
                                   out=values[..., 2], check=True)
    torch.cuda.synchronize()
    _check_column(values, 2, req, want)


def test_noalloc_fills_one_replica_column():
    log("[replicas] allocation-free call")
    rng = np.random.default_rng(73)
    bs, nh, d = 16, 2, 128
    req, nb = wl.page_requests(rng, [90, 31, 16, 2], bs, start_pos=[0, 1, 0, 0], spare_frac=0.2)
    layers = [0, 1, 2, 3, 4]
    host = [wl.host_random_bits(rng, wl.pool_shape("NHD", nb, bs, nh, d), "fp16") for _ in layers]
    want = oracle.checksum_blocks(host, "NHD", layers, [0] * 5, req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    values = _values((req.num_reqs, req.max_blocks))
    bt, nbt, sp, nt = req_tensors(req)
    kvck.kvck_checksum_blocks_noalloc([to_device_bits(p) for p in host], "NHD", layers, bt, nbt, sp, nt,
                                      out=values[..., 1])
    torch.cuda.synchronize()
    _check_column(values, 1, req, want)


@pytest.mark.parametrize("nlayers,rows", [(1, 8), (3, 20)])
def test_states_fill_one_replica_column(nlayers, rows):
    """One task group writes the column directly; several go through the
    second pass."""
    log(f"[replicas] Mamba states layers={nlayers} rows={rows}")
    rng = np.random.default_rng(74 + nlayers)
    slots = 9
    shapes = [(slots, rows, 4, 8), (slots, rows, 32)]
    elems = ["fp32", "bf16"]
    layers = [2 * i + 1 for i in range(nlayers)]
    hs = [[wl.host_random_bits(rng, s, e) for s, e in zip(shapes, elems)] for _ in layers]
    slot_ids = np.array([4, 0, 8, 2], np.int32)
    want = oracle.checksum_states(hs, layers, [0] * nlayers, slot_ids)
    values = torch.full((len(slot_ids), COLUMNS), SENTINEL, dtype=torch.int64, device=DEV).view(torch.uint64)
    kvck.kvck_checksum_states([[to_device_bits(a) for a in l] for l in hs], layers,
                              torch.from_numpy(slot_ids).to(DEV), out=values[:, 1], check=True)
    torch.cuda.synchronize()
    v = values.cpu().view(torch.int64).numpy().view(np.uint64)
    assert np.array_equal(v[:, 1], want)
    assert np.all(v[:, [0, 2]] == np.uint64(SENTINEL))


def test_worker_group_values_and_offloaded_tags():
    """One worker (TP rank 3 of 4) of a model whose layers carry two replica
    keys: layers 0-1 have 8 KV heads (2 per rank, key (1, 0)), layers 2-3
    have 2 KV heads replicated twice (this rank holds head 1, key (2, 1)).
    Its group values are (positions, 2); each column equals the oracle over
    that key's layers, and the tags of the offloaded value use each row
    summed."""
    log("[replicas] worker values and tags")
    rng = np.random.default_rng(75)
    bs, d, rank = 16, 64, 3
    req, nb = wl.page_requests(rng, [120, 47, 16], bs, start_pos=[0, 2, 0], spare_frac=0.2)
    full_a = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, 8, d), "bf16") for _ in range(2)]
    full_b = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, 2, d), "bf16") for _ in range(2)]
    shard_a = [np.ascontiguousarray(p[:, :, 2 * rank:2 * rank + 2]) for p in full_a]
    shard_b = [np.ascontiguousarray(p[:, :, 1:2]) for p in full_b]
    keys = [(1, 0), (2, 1)]
    values = torch.zeros((req.num_reqs, req.max_blocks, len(keys)), dtype=torch.uint64, device=DEV)
    bt, nbt, sp, nt = req_tensors(req)
    kvck.kvck_checksum_blocks([to_device_bits(p) for p in shard_a], "HND", [0, 1], bt, nbt, sp, nt,
                              global_head_base=[2 * rank] * 2, out=values[..., 0], check=True)
    kvck.kvck_checksum_blocks([to_device_bits(p) for p in shard_b], "HND", [2, 3], bt, nbt, sp, nt,
                              global_head_base=[1] * 2, out=values[..., 1], check=True)
    torch.cuda.synchronize()
    v = values.cpu().view(torch.int64).numpy().view(np.uint64)
    want_a = oracle.checksum_blocks(shard_a, "HND", [0, 1], [2 * rank] * 2, req.block_table, req.num_blocks,
                                    req.start_pos, req.num_tokens)
    want_b = oracle.checksum_blocks(shard_b, "HND", [2, 3], [1] * 2, req.block_table, req.num_blocks,
                                    req.start_pos, req.num_tokens)
    for r, k in req.listed():
        assert (int(v[r, k, 0]), int(v[r, k, 1])) == (int(want_a[r, k]), int(want_b[r, k])), (r, k)
    # tags of the offloaded value: each listed row's columns summed
    hashes = rng.integers(0, 256, size=(req.num_reqs * req.max_blocks, 32), dtype=np.uint8)
    fp = 0x0DDBA11CAFEF00D5
    tagged, _ = kvck.kvck_tag_checksums(values.view(-1), torch.from_numpy(hashes).to(DEV), fp,
                                        num_blocks_per_req=nbt, columns=len(keys))
    torch.cuda.synchronize()
    t = tagged.cpu().view(torch.int64).numpy().view(np.uint64).reshape(req.num_reqs, req.max_blocks)
    offl = oracle.tags.offloaded_value(v)
    for r, k in req.listed():
        i = r * req.max_blocks + k
        assert int(t[r, k]) == int(oracle.tags.tag_checksums([offl[r, k]], [hashes[i].tobytes()], fp)[0]), (r, k)
    # the load-time check compares against the row sums: a consistent load has no mismatch, a changed
    # replica column is caught at its position
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, mm = kvck.kvck_tag_checksums(values.view(-1), torch.from_numpy(hashes).to(DEV), fp, num_blocks_per_req=nbt,
                                    columns=len(keys), tagged=False, stored=tagged, mismatch_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0
    values.view(torch.int64)[0, 1, 1] += 1
    _, mm = kvck.kvck_tag_checksums(values.view(-1), torch.from_numpy(hashes).to(DEV), fp, num_blocks_per_req=nbt,
                                    columns=len(keys), tagged=False, stored=tagged)
    torch.cuda.synchronize()
    m = mm.cpu().numpy().reshape(req.num_reqs, req.max_blocks)
    assert [(r, k) for r, k in req.listed() if m[r, k]] == [(0, 1)]


def test_binding_rejects_unevenly_spaced_outputs():
    log("[replicas] binding checks")
    rng = np.random.default_rng(76)
    req, nb = wl.page_requests(rng, [40, 20], 16)
    pools = [to_device_bits(wl.host_random_bits(rng, wl.pool_shape("NHD", nb, 16, 2, 64), "bf16"))]
    bt, nbt, sp, nt = req_tensors(req)
    values = _values((req.num_reqs, req.max_blocks))
    with pytest.raises(ValueError):   # a transposed column: entries not evenly spaced in row-major order
        kvck.kvck_checksum_blocks(pools, "NHD", [0], bt, nbt, sp, nt, out=values[..., 0].t())
    with pytest.raises(ValueError):   # too few entries
        kvck.kvck_checksum_blocks(pools, "NHD", [0], bt, nbt, sp, nt, out=values[:1, :, 0])


def test_transposed_fused_copy_fills_one_replica_column():
    """The fused save of element-transposed K and V planes (K_TRANS, then
    V_TRANS accumulated) into column 0 equals the oracle on the HND pools
    holding the same tokens; no other entry moves."""
    log("[replicas] transposed fused copy")
    rng = np.random.default_rng(78)
    bs, nh, d = 16, 2, 64
    req, nb = wl.page_requests(rng, [70, 20, 5], bs, extra_blocks=[0, 1, 0], spare_frac=0.3)
    layers = [1, 2]
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, bs, nh, d), "bf16") for _ in layers]
    want = oracle.checksum_blocks(hp, "HND", layers, [0, 0], req.block_table, req.num_blocks, req.start_pos,
                                  req.num_tokens)
    kt = [to_device_bits(np.ascontiguousarray(p[0].transpose(0, 1, 3, 2))) for p in hp]
    vt = [to_device_bits(np.ascontiguousarray(p[1].transpose(0, 1, 3, 2))) for p in hp]
    bt, nbt, sp, nt = req_tensors(req)
    entries = int(req.num_blocks.sum())
    values = _values((req.num_reqs, req.max_blocks))
    for i, (planes, layout) in enumerate(((kt, "K_TRANS"), (vt, "V_TRANS"))):
        staging = torch.zeros(entries * kvck.kvck_staging_bytes(planes[0], layout, len(layers)), dtype=torch.uint8,
                              device=DEV)
        kvck.kvck_copy_checksum_blocks(kvck.KVCK_COPY_SAVE, planes, layout, layers, bt, nbt, sp, nt, staging,
                                       out=values[..., 0], accumulate=i > 0, check=True)
    torch.cuda.synchronize()
    _check_column(values, 0, req, want)

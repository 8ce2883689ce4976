"""Offloaded-checksum tags on the GPU == the tag oracle, and the offload
round trip detects a corrupted block, a wrong block hash and a wrong
fingerprint (GPU)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import DEV, gpu_blocks, log, to_device_bits

pytestmark = pytest.mark.gpu


def _hashes(rng, n, nbytes=32):
    return rng.integers(0, 256, size=(n, nbytes), dtype=np.uint8)


def test_tags_match_oracle():
    log("[tags] oracle parity")
    rng = np.random.default_rng(20)
    n = 5000
    c = rng.integers(0, 2**63, size=n, dtype=np.int64).view(np.uint64) * np.uint64(3)
    h = _hashes(rng, n)
    fp = 0xC0FFEE0123456789
    want = oracle.tags.tag_checksums(c, [bytes(r) for r in h], fp)
    ct = torch.from_numpy(c.view(np.int64)).to(DEV).view(torch.uint64)
    ht = torch.from_numpy(h).to(DEV)
    tagged, mm = kvck.kvck_tag_checksums(ct, ht, fp)
    assert mm is None
    assert np.array_equal(tagged.cpu().numpy(), want)
    # compare mode: flip some stored values
    stored = want.copy()
    bad = rng.choice(n, 17, replace=False)
    stored[bad] ^= np.uint64(1 << 13)
    count = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, mm = kvck.kvck_tag_checksums(ct, ht, fp, tagged=False,
                                    stored=torch.from_numpy(stored.view(np.int64)).to(DEV).view(torch.uint64),
                                    mismatch_count=count)
    torch.cuda.synchronize()
    want_mm = oracle.tags.offload_mismatches(c, [bytes(r) for r in h], fp, stored)
    assert np.array_equal(mm.cpu().numpy().astype(bool), want_mm)
    assert int(count.item()) == 17


def test_tags_beyond_one_grid():
    """2.5M entries of two replica columns: more than one grid covers (8192
    workgroups of 256 threads), so the kernel strides.  Tags equal the oracle
    on 20k sampled entries (the first and last 1000 among them); in compare
    mode exactly the 33 planted mismatches are flagged and counted."""
    log("[tags] 2.5M entries")
    rng = np.random.default_rng(23)
    n, cols = 2_500_000, 2
    c = rng.integers(0, 2**63, size=(n, cols), dtype=np.int64).view(np.uint64)
    h = _hashes(rng, n)
    fp = 0x0123456789ABCDEF
    ct = torch.from_numpy(c.reshape(-1).view(np.int64)).to(DEV).view(torch.uint64)
    ht = torch.from_numpy(h).to(DEV)
    tagged, _ = kvck.kvck_tag_checksums(ct, ht, fp, columns=cols)
    got = tagged.cpu().numpy()
    sample = np.unique(np.concatenate([np.arange(1000), np.arange(n - 1000, n), rng.choice(n, 18000, replace=False)]))
    row_sum = oracle.tags.offloaded_value(c[sample])
    want = oracle.tags.tag_checksums(row_sum, [bytes(r) for r in h[sample]], fp)
    assert np.array_equal(got[sample], want)
    stored = got.copy()
    planted = rng.choice(n, 33, replace=False)
    stored[planted] ^= np.uint64(1) << np.uint64(40)
    count = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, mm = kvck.kvck_tag_checksums(ct, ht, fp, columns=cols, tagged=False,
                                    stored=torch.from_numpy(stored.view(np.int64)).to(DEV).view(torch.uint64),
                                    mismatch_count=count)
    torch.cuda.synchronize()
    assert np.array_equal(np.flatnonzero(mm.cpu().numpy()), np.sort(planted))
    assert int(count.item()) == 33


def test_offload_round_trip():
    log("[tags] offload round trip")
    rng = np.random.default_rng(21)
    req, nb = wl.page_requests(rng, [100, 37, 300], 16, spare_frac=0.2)
    hp = [wl.host_random_bits(rng, wl.pool_shape("HND", nb, 16, 8, 128), "bf16") for _ in range(3)]
    pools = [to_device_bits(p) for p in hp]
    layers = [0, 1, 2]
    R, M = req.num_reqs, req.max_blocks
    hashes = _hashes(rng, R * M)
    ht = torch.from_numpy(hashes).to(DEV)
    nbt = torch.from_numpy(req.num_blocks).to(DEV)
    fp = 0x1234
    c = gpu_blocks(pools, "HND", layers, req)
    ct = torch.from_numpy(c.view(np.int64).copy()).to(DEV).view(torch.uint64)
    stored, _ = kvck.kvck_tag_checksums(ct.view(-1), ht, fp, num_blocks_per_req=nbt)
    # unlisted entries are not written
    s = stored.cpu().numpy().reshape(R, M)
    for r in range(R):
        assert not s[r, int(req.num_blocks[r]):].any()

    def check(checks, hashes_t=ht, fingerprint=fp):
        cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
        _, mm = kvck.kvck_tag_checksums(checks.view(-1), hashes_t, fingerprint, num_blocks_per_req=nbt,
                                        tagged=False, stored=stored, mismatch_count=cnt)
        torch.cuda.synchronize()
        return int(cnt.item()), mm.cpu().numpy().reshape(R, M)

    assert check(ct)[0] == 0
    # corrupt one element of one listed block of layer 1 and checksum again
    r, k = 2, 5
    b = int(req.block_table[r, k])
    pools[1].view(torch.int16)[1, b, 3, 7, 11] ^= 1
    c2 = gpu_blocks(pools, "HND", layers, req)
    n_bad, mm = check(torch.from_numpy(c2.view(np.int64).copy()).to(DEV).view(torch.uint64))
    assert n_bad == 1 and mm[r, k] == 1
    pools[1].view(torch.int16)[1, b, 3, 7, 11] ^= 1
    # a load that presents another block's hash, or another group's fingerprint
    wrong = ht.clone()
    wrong[0] = ht[1]
    assert check(ct, hashes_t=wrong)[0] == 1
    n_listed = int(req.num_blocks.sum())
    assert check(ct, fingerprint=fp + 1)[0] == n_listed


def test_rejected_requests_are_not_tagged():
    """A request the checksum call rejects (count outside [0, max_blocks],
    negative start position) leaves its entries unwritten there, so the tags
    call lists nothing for it either: no tag written, no comparison made, no
    mismatch counted -- whatever stale values its entries hold."""
    log("[tags] rejected requests")
    rng = np.random.default_rng(22)
    req, nb = wl.page_requests(rng, [60, 40, 90, 20], 16, spare_frac=0.2)
    R, M = req.num_reqs, req.max_blocks
    counts = req.num_blocks.copy()
    counts[1] = M + 1          # too many listed blocks
    counts[3] = -2             # negative count
    start = req.start_pos.copy()
    start[2] = -1              # negative start position
    nbt = torch.from_numpy(counts).to(DEV)
    spt = torch.from_numpy(start).to(DEV)
    stale = rng.integers(0, 2**63, size=R * M, dtype=np.int64)
    ct = torch.from_numpy(stale).to(DEV).view(torch.uint64)
    ht = torch.from_numpy(_hashes(rng, R * M)).to(DEV)
    sentinel = np.uint64(0x5A5A5A5A5A5A5A5A)
    tagged = torch.full((R * M,), int(sentinel.view(np.int64)), dtype=torch.int64, device=DEV).view(torch.uint64)
    kvck.kvck_tag_checksums(ct, ht, 77, num_blocks_per_req=nbt, start_pos=spt, block_size=16, tagged=tagged)
    # stored values that match nothing: every listed entry of a good request mismatches
    stored = torch.zeros(R * M, dtype=torch.int64, device=DEV).view(torch.uint64)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, mm = kvck.kvck_tag_checksums(ct, ht, 77, num_blocks_per_req=nbt, start_pos=spt, block_size=16, tagged=False,
                                    stored=stored, mismatch_count=cnt)
    torch.cuda.synchronize()
    t = tagged.cpu().numpy().reshape(R, M)
    want = oracle.tags.tag_checksums(stale.view(np.uint64), [bytes(r) for r in ht.cpu().numpy()], 77).reshape(R, M)
    good = [0]
    assert int(cnt.item()) == sum(int(counts[r]) for r in good)
    for r in range(R):
        listed = int(counts[r]) if r in good else 0
        assert np.array_equal(t[r, :listed], want[r, :listed]), r
        assert np.all(t[r, listed:] == sentinel), r
    # without start positions only the count rule applies: request 2 is listed again
    cnt.zero_()
    kvck.kvck_tag_checksums(ct, ht, 77, num_blocks_per_req=nbt, tagged=False, stored=stored, mismatch_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == int(counts[0]) + int(counts[2])

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

"""The C example program on the GPU: the checksums it prints through the C ABI
alone (no Python, no torch in that process) equal the oracle's on the same
splitmix64 pools (GPU)."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from paged_kv_cache_kvck_amd import workloads as wl
from gpu_helpers import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "paged_kv_cache_kvck_amd", "kvck_demo")

# the program's configuration (examples/kvck_demo.c)
LAYERS, NB, BS, NH, D = [0, 7, 31], 24, 16, 4, 64
TABLE = np.array([[5, 17, 2, 9], [11, 0, -1, -1], [21, 3, 14, -1]], np.int32)
NUM_BLOCKS = np.array([4, 2, 3], np.int32)
START = np.array([0, 1, 0], np.int64)
TOKENS = np.array([50, 40, 33], np.int64)


def test_c_program_matches_oracle():
    log("[c abi] kvck_demo")
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in r.stdout.split("\n"):
        if line.strip():
            tag, rr, kk, val = line.split()
            got[(tag, int(rr), int(kk))] = int(val)
    shape = (2, NB, BS, NH, D)
    nbytes = int(np.prod(shape)) * 2
    pools = [wl.splitmix64_bytes(1000 + i, nbytes).view(np.uint16).reshape(shape) for i in range(len(LAYERS))]
    full = oracle.checksum_blocks(pools, "NHD", LAYERS, [0] * 3, TABLE, NUM_BLOCKS, START, TOKENS)
    shard = oracle.checksum_blocks(pools, "NHD", LAYERS, [1] * 3, TABLE, NUM_BLOCKS, START, TOKENS, head_begin=1,
                                   head_count=2)
    listed = [(r_, k) for r_ in range(3) for k in range(int(NUM_BLOCKS[r_]))]
    assert len(got) == 2 * len(listed)
    for r_, k in listed:
        assert got[("full", r_, k)] == int(full[r_, k]), (r_, k)
        assert got[("shard", r_, k)] == int(shard[r_, k]), (r_, k)

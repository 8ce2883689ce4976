"""Host-side logic of bench.py (CPU): the one-GPU rule, the code-only source
hash that decides whether committed HBM counters still apply, and the
committed traffic figure itself."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_cache_kvck_amd import sources  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 1
    assert "one GPU" in capsys.readouterr().err


def test_code_only_ignores_comments_and_whitespace():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no overflow check */\n}\n"
    b = "int f(int x){\n\treturn 2*x;\n}"
    assert sources.code_only(a) == sources.code_only(b)
    assert sources.code_only(a) != sources.code_only(a.replace("2 * x", "3 * x"))


def test_committed_traffic_is_null_or_close_to_the_valid_bytes():
    """Either the main pass changed since the counters were taken (null), or
    the HBM bytes per launch they give are within 2 % above the valid bytes:
    nothing read twice."""
    t = bench.committed_traffic("llama3_8b")
    with open(os.path.join(ROOT, "profiles", "traffic_llama3_8b.json")) as f:
        j = json.load(f)
    if t is None:
        assert j["kernel_sources_sha256"] != sources.kernel_sources_sha()
        return
    valid = j["valid_bytes_per_launch"]
    assert valid <= t <= 1.02 * valid, (t, valid)


def test_cpu_baseline_legs_agree_on_a_small_workload():
    """The benchmark's CPU-baseline leg on a small workload held in CPU
    tensors: the one-process oracle values equal the reference checksums
    given as the "GPU" output, and the parallel leg's layer-subset partials
    (two processes) add up to them mod 2^64."""
    import numpy as np
    import torch
    import oracle
    from paged_kv_cache_kvck_amd import workloads as wl

    w = wl.llama3_8b(num_reqs=6, lo=20, hi=200, layers=5)
    host = [wl.host_random_bits(np.random.default_rng(i), w.shape, "bf16") for i in range(w.num_layers)]
    pools = [torch.from_numpy(h.view(np.int16)) for h in host]
    ref = oracle.checksum_blocks(host, w.layout, w.layer_numbers, w.bases, w.req.block_table, w.req.num_blocks,
                                 w.req.start_pos, w.req.num_tokens)
    res = bench.cpu_baseline(pools, w, 0.5, ref, 2, chunk=8)
    assert res["gpu_checked_positions"] > 0 and res["gpu_mismatches"] == 0
    par = res["parallel"]
    assert par["cores"] == 2 and par["positions_compared"] == res["gpu_checked_positions"]
    assert par["partial_sum_mismatches"] == 0
    # a wrong reference is noticed
    bad = ref.copy()
    bad[0, 0] ^= np.uint64(1)
    res = bench.cpu_baseline(pools, w, 100.0, bad, 2, chunk=64)
    assert res["gpu_mismatches"] == 1 and res["gpu_checked_positions"] == len(w.req.listed())

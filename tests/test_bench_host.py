"""Host-side logic of bench.py (CPU): the one-GPU rule, the code-only source
hash that decides whether committed HBM counters still apply, and the
committed traffic figure itself."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 1
    assert "one GPU" in capsys.readouterr().err


def test_code_only_ignores_comments_and_whitespace():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no overflow check */\n}\n"
    b = "int f(int x){\n\treturn 2*x;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("2 * x", "3 * x"))


def test_committed_traffic_is_null_or_close_to_the_valid_bytes():
    """Either the main pass changed since the counters were taken (null), or
    the HBM bytes per launch they give are within 2 % above the valid bytes:
    nothing read twice."""
    t = bench.committed_traffic("llama3_8b")
    with open(os.path.join(ROOT, "profiles", "traffic_llama3_8b.json")) as f:
        j = json.load(f)
    if t is None:
        assert j["kernel_sources_sha256"] != bench.kernel_sources_sha()
        return
    valid = j["valid_bytes_per_launch"]
    assert valid <= t <= 1.02 * valid, (t, valid)

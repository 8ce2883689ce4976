"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds libkvck's sources with the sanitizers on the host code only (device
code is compiled as usual and never run here), links them into the C driver
``tests/host_sanitize/abi_checks.cpp``, and runs it: every entry point is
called with arguments it must reject, including integers at the edges of
their types, and with valid arguments that must report the missing device.
Any out-of-bounds host access, signed overflow or other undefined behaviour
aborts the program.
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_kvck_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_checks.cpp")

# sanitizers apply to host code only (-Xarch_host before each one)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_abi_checks_under_asan_and_ubsan(tmp_path):
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        if src.endswith(".hip"):
            cmd = ["hipcc", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
        else:
            cmd = ["hipcc", "--offload-host-only"]
        cmd += COMMON + SAN + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources + [DRIVER]))
    exe = str(tmp_path / "abi_checks")
    r = subprocess.run(["hipcc"] + SAN + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "all checks passed" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]

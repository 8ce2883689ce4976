"""The library from plain C (CPU): the public header is strict C99, and the C
example program (examples/kvck_demo.c, built with the library) draws the same
splitmix64 stream as the seeded input module and fails cleanly without a
gfx950 device.  Its checksums are compared with the oracle on the GPU
(tests/test_gpu_c_abi.py)."""

import os
import shutil
import struct
import subprocess

import pytest
import torch

from paged_kv_cache_kvck_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "paged_kv_cache_kvck_amd", "kvck_demo")

# splitmix64 seeded 0: its first outputs as published with the generator
PUBLISHED_SEED0 = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def _stream(seed, n):
    r = subprocess.run([DEMO, "--stream", str(seed), str(n)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    return [int(x, 16) for x in r.stdout.split()]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_strict_c99(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "kvck.h"\nint main(void) { return kvck_abi_version() == KVCK_ABI_VERSION ? 0 : 1; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_demo_stream_is_splitmix64():
    assert _stream(0, 3) == PUBLISHED_SEED0
    for seed in (0, 1000, 1002):
        got = _stream(seed, 64)
        want = list(struct.unpack("<64Q", bytes(wl.splitmix64_bytes(seed, 64 * 8))))
        assert got == want, seed


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device answer")
def test_demo_without_device_exits_cleanly():
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "KVCK_ERR_NO_DEVICE" in r.stderr

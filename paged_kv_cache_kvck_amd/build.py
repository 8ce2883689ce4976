"""Build libkvck.so in-tree for gfx950 with hipcc.

    python -m paged_kv_cache_kvck_amd.build [--save-temps DIR]

The library is a plain C-ABI shared object (include/kvck.h); the Python
binding loads it with ctypes, so no torch C++ extension is involved.  The
build also makes ``kvck_demo``, a plain C program that uses the library
through include/kvck.h alone (examples/kvck_demo.c).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkvck.so")
DEMO = os.path.join(PKG, "kvck_demo")
ARCH = "gfx950"

# Packed-FP32 instructions are kept out of every kernel (no FP32 math is used
# anyway; the flag keeps the compiler from forming them).
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd, verbose, cwd=None):
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=cwd)


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    """Compile every source to an object in parallel (the kernel variants make
    single files slow), link libkvck.so, then the C demo."""
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="kvck_build_") as objdir:
        jobs = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [hipcc(), *compile_flags, *inc, "-c", src, "-o", obj]
            if save_temps:
                cmd.insert(1, "-save-temps")
            jobs.append((cmd, obj))
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = [ex.submit(_run, cmd, verbose, save_temps) for cmd, _ in jobs]
            for f in futs:
                f.result()
        tmp = LIB + ".tmp"
        _run([hipcc(), *HIP_FLAGS, *[obj for _, obj in jobs], "-o", tmp], verbose)
        os.replace(tmp, LIB)
    # a plain C consumer of the C ABI (gcc, C99): no Python or torch involved
    demo_tmp = DEMO + ".tmp"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run([shutil.which("gcc") or "gcc", "-std=c99", "-O2", "-Wall", "-Wextra",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(PKG, "examples", "kvck_demo.c"), "-o", demo_tmp, "-L", PKG, "-lkvck",
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN",
                    "-Wl,-rpath," + os.path.join(rocm, "lib")], check=True)
    os.replace(demo_tmp, DEMO)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="keep intermediate files (ISA) in this directory")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.save_temps, args.verbose))


if __name__ == "__main__":
    sys.exit(main())

"""Structure of the compiled gfx950 kernels (CPU: hipcc cross-compiles, no GPU).

Two properties decide how well the streaming kernels keep HBM busy, and
neither shows in a correctness test:

* every buffer load and store is a single instruction: with a descriptor the
  compiler cannot prove uniform across the wavefront, it wraps the access in
  a loop that compares the descriptor lane by lane (``v_readfirstlane`` and a
  branch back to the same block);
* in the double-buffered main pass, the waits before the arithmetic on one
  buffer leave the other buffer's loads in flight: every ``s_waitcnt vmcnt(N)``
  among the multiply-accumulates keeps N at least that buffer's load count.

The kernels are compiled to AMD assembly here, exactly as the library build
does (same flags), and the assembly is read.
"""

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_kvck_amd", "csrc")
SOURCES = ["kvck_blocks.hip", "kvck_tblocks.hip", "kvck_copy.hip", "kvck_tcopy.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

_ASM = {}


def _compile(src, outdir):
    out = os.path.join(outdir, src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return src, f.read()


def assembly():
    if not _ASM:
        with tempfile.TemporaryDirectory(prefix="kvck_isa_") as d, cf.ThreadPoolExecutor(len(SOURCES)) as ex:
            for src, text in ex.map(lambda s: _compile(s, d), SOURCES):
                _ASM[src] = text
    return _ASM


def kernels(text):
    """{mangled name: [(block label, [instructions])]} for every kernel."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):", text, re.M):
        name = m.group(1)
        end = text.find(".Lfunc_end", m.start())
        blocks, label, cur = [], "entry", []
        for line in text[m.end():end].split("\n"):
            t = line.split(";")[0].strip()
            if not t:
                continue
            if t.endswith(":"):
                blocks.append((label, cur))
                label, cur = t[:-1], []
            elif not t.startswith("."):
                cur.append(t)
        blocks.append((label, cur))
        out[name] = blocks
    return out


def test_no_buffer_access_in_a_per_lane_descriptor_loop():
    found = []
    n_kernels = 0
    for src, text in assembly().items():
        for name, blocks in kernels(text).items():
            n_kernels += 1
            for label, ins in blocks:
                memory = any(i.startswith(("buffer_load", "buffer_store")) for i in ins)
                uniformize = any(i.startswith("v_readfirstlane") for i in ins)
                loops_back = any(i.startswith("s_cbranch") and i.split()[-1] == label for i in ins)
                if memory and uniformize and loops_back:
                    found.append((src, name, label))
    assert n_kernels > 200, n_kernels
    assert not found, found[:5]


def _consume_waits(blocks, min_mads):
    waits = []
    for _, ins in blocks:
        if sum(i.startswith("v_mad_u64_u32") for i in ins) >= min_mads:
            waits += [int(m.group(1)) for i in ins for m in [re.match(r"s_waitcnt vmcnt\((\d+)\)", i)] if m]
    return waits


@pytest.mark.parametrize("variant,other_buffer", [
    # <chunk, slots, heads per unit, planes per unit, pipelined, merged, dense>
    ("blocks_kernelILi16ELi4ELi4ELi1ELb1ELb0ELb0E", 16),   # HND bf16 head 128 (the 147 GB workload)
    ("blocks_kernelILi16ELi4ELi2ELi2ELb1ELb0ELb0E", 16),   # its TP shard: K and V in one unit
    ("blocks_kernelILi16ELi8ELi1ELi1ELb1ELb1ELb0E", 8),    # merged rows
])
def test_pipelined_waits_leave_the_other_buffer_in_flight(variant, other_buffer):
    text = assembly()["kvck_blocks.hip"]
    ks = {n: b for n, b in kernels(text).items() if variant in n}
    assert len(ks) == 1, list(ks)
    waits = _consume_waits(next(iter(ks.values())), min_mads=4)
    assert waits, "no multiply-accumulate block found"
    assert min(waits) >= other_buffer, sorted(set(waits))

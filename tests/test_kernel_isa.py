"""Structure of the compiled gfx950 kernels (CPU: hipcc cross-compiles, no GPU).

Two properties decide how well the streaming kernels keep HBM busy, and
neither shows in a correctness test:

* every buffer load and store is a single instruction: with a descriptor the
  compiler cannot prove uniform across the wavefront, it wraps the access in
  a loop that compares the descriptor lane by lane (``v_readfirstlane`` and a
  branch back to the same block);
* in the double-buffered kernels, the waits before the use of one buffer leave
  the other buffer's loads in flight: every ``s_waitcnt vmcnt(N)`` among the
  multiply-accumulates (or the fused copy's stores) keeps N at least that
  buffer's load count.

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


def _consume_waits(blocks, marker):
    """vmcnt of every wait in the blocks that use loaded data: those with at
    least four `marker` instructions (multiply-accumulates, or the fused
    copy's stores)."""
    waits = []
    for _, ins in blocks:
        if sum(i.startswith(marker) for i in ins) >= 4:
            waits += [int(m.group(1)) for i in ins for m in [re.match(r"s_waitcnt vmcnt\((\d+)\)", i)] if m]
    return waits


MAC, STORE = "v_mad_u64_u32", "buffer_store"


@pytest.mark.parametrize("src,variant,marker,other_buffer", [
    # blocks_kernel<chunk, slots, heads per unit, planes per unit, pipelined, merged, dense>
    ("kvck_blocks.hip", "blocks_kernelILi16ELi4ELi4ELi1ELb1ELb0ELb0E", MAC, 16),  # HND bf16 head 128 (147 GB)
    ("kvck_blocks.hip", "blocks_kernelILi16ELi4ELi2ELi2ELb1ELb0ELb0E", MAC, 16),  # its TP shard: K+V units
    ("kvck_blocks.hip", "blocks_kernelILi16ELi8ELi1ELi1ELb1ELb1ELb0E", MAC, 8),   # merged rows
    # tblocks_kernel<chunk, element bytes, slots, heads per unit, pipelined, dense>: a transposed bf16 plane
    ("kvck_tblocks.hip", "tblocks_kernelILi16ELi2ELi4ELi4ELb1ELb0E", MAC, 16),
    # copy_kernel<chunk, slots, heads per unit, planes per unit, direction, pipelined, merged>: ping-pong save
    ("kvck_copy.hip", "copy_kernelILi16ELi4ELi4ELi1ELi0ELb1ELb0E", STORE, 16),
    ("kvck_copy.hip", "copy_kernelILi16ELi8ELi1ELi1ELi0ELb1ELb1E", STORE, 8),    # ping-pong save, merged rows
    # tcopy_lds_kernel<element bytes, slots, direction>: bf16 save through LDS (checksum by dot products)
    ("kvck_tcopy.hip", "tcopy_lds_kernelILi2ELi4ELi0E", "v_dot2_u32_u16", 4),
])
def test_pipelined_waits_leave_the_other_buffer_in_flight(src, variant, marker, other_buffer):
    text = assembly()[src]
    ks = {n: b for n, b in kernels(text).items() if variant in n}
    assert len(ks) == 1, list(ks)
    waits = _consume_waits(next(iter(ks.values())), marker)
    assert waits, "no block using loaded data found"
    assert min(waits) >= other_buffer, sorted(set(waits))


def _loop_waits(text, variant):
    """vmcnt of every wait inside a loop of the one kernel whose name holds
    `variant` (the compiler marks a loop's blocks in its label comments)."""
    names = [m for m in re.finditer(r"^(_Z\S+):", text, re.M) if variant in m.group(1)]
    assert len(names) == 1, [m.group(1) for m in names]
    m = names[0]
    body = text[m.end():text.find(".Lfunc_end", m.start())]
    waits, in_loop = [], False
    for line in body.split("\n"):
        label = re.match(r"^(\.LBB\S+):(.*)$", line.strip())
        if label:
            in_loop = "Loop" in label.group(2)
            continue
        w = re.match(r"s_waitcnt.*vmcnt\((\d+)\)", line.split(";")[0].strip())
        if w and in_loop:
            waits.append(int(w.group(1)))
    return waits


@pytest.mark.parametrize("chunk,slots", [(16, 8), (16, 4), (16, 2), (8, 8), (8, 4)])
def test_merged_stream_drains_once_per_step(chunk, slots):
    """The planned merged-row checksum streams units through two buffers and
    lets the first buffer's loads land before the second is issued: exactly
    one wait for every load per step, and the wait before the second buffer
    is used leaves the first buffer's `slots` loads in flight.  A second full
    wait (e.g. from a loop with two exits, whose path back to the loop head
    merges a pending buffer) would fail this."""
    variant = f"blocks_kernelILi{chunk}ELi{slots}ELi1ELi1ELb1ELb1ELb0E"
    waits = _loop_waits(assembly()["kvck_blocks.hip"], variant)
    assert waits.count(0) == 1, waits
    assert min(w for w in waits if w) >= slots, waits


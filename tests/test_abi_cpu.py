"""The C-ABI library on the CPU: it loads, exports every symbol include/kvck.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest
import torch

import paged_kv_cache_kvck_amd as kvck
from paged_kv_cache_kvck_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000001000  # a device address that validation never dereferences


def header_functions():
    with open(os.path.join(ROOT, "include", "kvck.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:kvck_status|size_t|const char\s*\*|int32_t)\s+(kvck_\w+)\s*\(",
                                 text, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = kvck.load_library()
    decl = header_functions()
    assert len(decl) == 13
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTS) == decl
    assert kvck.kvck_abi_version() == B.KVCK_ABI_VERSION == 3
    assert kvck.kvck_status_string(-4) == "KVCK_ERR_WORKSPACE"
    assert kvck.kvck_status_string(-7) == "KVCK_ERR_SCRATCH"
    assert kvck.kvck_status_string(7) == "KVCK_UNKNOWN_STATUS"


def test_binding_constants_match_the_header():
    """Every constant the binding restates has the value include/kvck.h defines."""
    with open(os.path.join(ROOT, "include", "kvck.h")) as f:
        text = f.read()
    define = re.compile(r"^#define[ \t]+(KVCK_\w+)[ \t]+(.+?)[ \t]*(?:/\*.*)?$", re.M)
    defines = {m.group(1): m.group(2) for m in define.finditer(text)}

    def value(expr):
        return eval(re.sub(r"(\d+)u\b", r"\1", expr), {})  # integer literals and shifts only

    names = [n for n in dir(B) if n.startswith("KVCK_") and isinstance(getattr(B, n), int) and n in defines]
    assert {"KVCK_ABI_VERSION", "KVCK_MAX_CACHES", "KVCK_MAX_OUT_STRIDE", "KVCK_SCRATCH_BYTES",
            "KVCK_FLAG_BAD_BLOCK_ID", "KVCK_COPY_LOAD"} <= set(names)
    for n in names:
        assert getattr(B, n) == value(defines[n]), n


def test_workspace_sizes():
    assert kvck.kvck_blocks_workspace_bytes(0, 1, 1) == 0
    one = kvck.kvck_blocks_workspace_bytes(1, 256, 512)
    many = kvck.kvck_blocks_workspace_bytes(32, 256, 512)
    assert one % 256 == 0 and many % 256 == 0
    assert many - one >= 32 * 256 * 512 * 8
    assert kvck.kvck_states_workspace_bytes(24, 64, 128) >= 24 * 8 * 128 * 8


def _layout(**kw):
    L = B.kvck_kv_layout()
    d = dict(planes=2, block_size=16, num_heads=8, row_bytes=256, num_blocks=100, plane_stride=100 * 32768,
             block_stride=32768, slot_stride=256, head_stride=4096)
    d.update(kw)
    for k, v in d.items():
        setattr(L, k, v)
    return L


def _call(L=None, ncaches=2, layers=(0, 1), bases=(0, 0), head_begin=0, head_count=8, num_reqs=4, max_blocks=8,
          bt_stride=8, ws_bytes=None, ptr=FAKE, out=FAKE, ws=FAKE, out_stride=1):
    lib = kvck.load_library()
    L = L or _layout()
    ptrs = (ctypes.c_void_p * ncaches)(*([ptr] * ncaches))
    ly = (ctypes.c_int32 * ncaches)(*layers)
    bs = (ctypes.c_int32 * ncaches)(*bases)
    need = lib.kvck_blocks_workspace_bytes(ncaches, num_reqs, max_blocks)
    return lib.kvck_checksum_blocks(ctypes.byref(L), ptrs, ly, bs, ncaches, head_begin, head_count, FAKE, bt_stride,
                                    FAKE, FAKE, FAKE, num_reqs, max_blocks, out, out_stride, 0, ws,
                                    need if ws_bytes is None else ws_bytes, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=_layout(planes=3)), -1),
    (dict(L=_layout(block_size=0)), -1),
    (dict(L=_layout(row_bytes=12)), -2),            # not whole 8-byte pieces
    (dict(L=_layout(slot_stride=-256)), -1),
    (dict(head_count=0), -1),
    (dict(head_begin=7, head_count=2), -1),
    (dict(bases=(0, 65535)), -2),                    # more than MAX_KV_HEADS_PER_LAYER heads
    (dict(layers=(0, -1)), -1),
    (dict(ptr=0), -1),
    (dict(out=0), -1),
    (dict(bt_stride=4), -1),
    (dict(out_stride=0), -1),
    (dict(out_stride=B.KVCK_MAX_OUT_STRIDE + 1), -1),
    (dict(out_stride=0, num_reqs=0), -1),
    (dict(out=FAKE + 4), -3),
    (dict(ws_bytes=64), -4),
    (dict(ws=FAKE + 8), -4),                          # workspace not 256-byte aligned
    (dict(ptr=FAKE + 4, L=_layout(row_bytes=8, slot_stride=8, head_stride=128, block_stride=2048)), -3),
    (dict(L=_layout(row_bytes=16 * 1024 * 2)), -2),  # a row longer than one lane table covers
])
def test_blocks_rejects_before_launch(kw, status):
    assert _call(**kw) == status


def test_blocks_zero_requests_is_a_no_op():
    assert _call(num_reqs=0) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU answer")
def test_valid_call_without_gpu_reports_no_device():
    assert _call() == -6
    # any non-negative int32 layer number passes validation (64-bit slice factors)
    assert _call(layers=(40000, 2**31 - 1)) == -6
    # one replica column of up to KVCK_MAX_OUT_STRIDE
    assert _call(out_stride=B.KVCK_MAX_OUT_STRIDE) == -6
    assert kvck.kvck_platform_supported() is False


def test_states_rejects_before_launch():
    lib = kvck.load_library()
    D = (B.kvck_state_desc * 2)()
    D[0].slot_stride, D[0].row_stride, D[0].row_elems, D[0].elem_bytes = 64 * 8192, 8192, 2048, 4
    D[1].slot_stride, D[1].row_stride, D[1].row_elems, D[1].elem_bytes = 64 * 2048, 2048, 1024, 2
    ptrs = (ctypes.c_void_p * 4)(*([FAKE] * 4))
    ly = (ctypes.c_int32 * 2)(1, 3)
    base = (ctypes.c_int32 * 2)(0, 0)

    def call(nstates=2, elem=None, rows=(0, 64), nrows=64, ws=FAKE, ws_bytes=1 << 20, num_reqs=8, out=FAKE,
             out_stride=1):
        if elem:
            D[1].elem_bytes = elem
        try:
            return lib.kvck_checksum_states(D, nstates, ptrs, ly, base, 2, 160, nrows, rows[0], rows[1], FAKE,
                                            num_reqs, out, out_stride, 0, ws, ws_bytes, None, None)
        finally:
            D[1].elem_bytes = 2

    assert call(elem=1) == -2
    assert call(elem=8) == -2
    assert call(nstates=5) == -2
    assert call(rows=(60, 8)) == -1
    assert call(ws_bytes=8) == -4
    assert call(num_reqs=0) == 0
    assert call(out_stride=0) == -1
    assert call(out=FAKE + 4) == -3
    if not torch.cuda.is_available():
        assert call() == -6
        assert call(out_stride=3) == -6


def test_binding_argument_checks():
    pools = [torch.zeros((2, 4, 16, 2, 64), dtype=torch.bfloat16)]
    L = kvck.kv_layout(pools[0], "NHD")
    assert (L.planes, L.block_size, L.num_heads, L.row_bytes, L.num_blocks) == (2, 16, 2, 128, 4)
    assert (L.plane_stride, L.block_stride, L.slot_stride, L.head_stride) == (4 * 4096, 4096, 256, 128)
    H = kvck.kv_layout(pools[0].permute(0, 1, 3, 2, 4), "HND")
    assert (H.block_size, H.num_heads, H.slot_stride, H.head_stride) == (16, 2, 256, 128)
    M = kvck.kv_layout(torch.zeros((5, 64, 576), dtype=torch.bfloat16), "MLA")
    assert (M.planes, M.num_heads, M.row_bytes, M.block_stride) == (1, 1, 1152, 64 * 1152)
    with pytest.raises(ValueError):
        kvck.kv_layout(pools[0].transpose(3, 4), "NHD")
    bt = torch.zeros((1, 4), dtype=torch.int64)
    with pytest.raises(ValueError):
        kvck.kvck_checksum_blocks(pools, "NHD", [0], bt, torch.zeros(1, dtype=torch.int32),
                                  torch.zeros(1, dtype=torch.int64), torch.zeros(1, dtype=torch.int64))
    # the kernels' error word is one 32-bit value
    with pytest.raises(ValueError):
        kvck.kvck_checksum_blocks(pools, "NHD", [0], bt.to(torch.int32), torch.zeros(1, dtype=torch.int32),
                                  torch.zeros(1, dtype=torch.int64), torch.zeros(1, dtype=torch.int64),
                                  error_flags=torch.zeros(1, dtype=torch.int64))


def test_tags_rejects_before_launch():
    lib = kvck.load_library()

    def call(cs=FAKE, h=FAKE, stride=32, n=16, nbpr=None, mb=0, tagged=FAKE, stored=None, mm=None, cnt=None,
             sp=None, bs=0, columns=1):
        return lib.kvck_tag_checksums(cs, columns, h, stride, 0, n, nbpr, sp, mb, bs, tagged, stored, mm, cnt, None)

    assert call(n=0) == 0
    assert call(n=-1) == -1
    assert call(cs=0) == -1
    assert call(tagged=None) == -1               # neither tagged nor stored
    assert call(mm=FAKE) == -1                   # mismatch output without stored values
    assert call(stride=4) == -1
    assert call(stride=12) == -3
    assert call(h=FAKE + 4) == -3
    assert call(nbpr=FAKE, mb=5) == -1           # n not a multiple of max_blocks
    assert call(sp=FAKE, bs=16) == -1            # start positions without counts
    assert call(nbpr=FAKE, mb=4, sp=FAKE) == -1  # start positions without a block size
    assert call(nbpr=FAKE + 2, mb=4) == -3       # counts not 4-byte aligned
    assert call(nbpr=FAKE, mb=4, sp=FAKE + 4, bs=16) == -3
    assert call(columns=0) == -1
    assert call(columns=B.KVCK_MAX_OUT_STRIDE + 1) == -1
    assert call(cs=FAKE + 4) == -3               # uint64 arrays 8-byte aligned
    assert call(tagged=FAKE + 4) == -3
    if not torch.cuda.is_available():
        assert call() == -6
        assert call(columns=4) == -6


def test_noalloc_rejects_before_launch():
    """The allocation-free variant validates like kvck_checksum_blocks and
    refuses, before any device call, a batch whose position records alone
    exceed the scratch array (32 bytes per request slot)."""
    lib = kvck.load_library()
    L = _layout()

    def call(num_reqs=4, max_blocks=8, out=FAKE, layers=(0, 1), out_stride=1):
        ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
        ly = (ctypes.c_int32 * 2)(*layers)
        bs = (ctypes.c_int32 * 2)(0, 0)
        return lib.kvck_checksum_blocks_noalloc(ctypes.byref(L), ptrs, ly, bs, 2, 0, 8, FAKE, max_blocks, FAKE, FAKE,
                                                FAKE, num_reqs, max_blocks, out, out_stride, 0, None, None)

    assert call(num_reqs=0) == 0
    assert call(out=0) == -1
    assert call(layers=(0, -1)) == -1
    assert call(out_stride=0) == -1
    slots = B.KVCK_SCRATCH_BYTES // 32 + 1024
    assert call(num_reqs=slots // 1024, max_blocks=1024) == -7
    if not torch.cuda.is_available():
        assert call() == -6


def test_output_stride_of_replica_columns():
    """The binding's element stride of an output view: 1 for a dense array, C
    for one column of a row-major (..., C) array; views whose entries are not
    evenly spaced in row-major order, or too few, are refused."""
    cpu = torch.device("cpu")
    values = torch.zeros((4, 6, 3), dtype=torch.uint64)
    assert B._out_stride(values[..., 0], 24, cpu) == 3
    assert B._out_stride(values[..., 2], 24, cpu) == 3
    assert B._out_stride(torch.zeros(24, dtype=torch.int64), 24, cpu) == 1
    assert B._out_stride(values[:1, :, 1], 6, cpu) == 3       # a single request row
    assert B._out_stride(values.view(-1)[::5], 10, cpu) == 5
    with pytest.raises(ValueError):
        B._out_stride(values[..., 0].t(), 24, cpu)             # column-major walk
    assert B._out_stride(values[:, ::2, 0], 12, cpu) == 6     # every other position: still evenly spaced
    with pytest.raises(ValueError):
        B._out_stride(values[:, 0], 12, cpu)                   # rows 18 apart, entries 1 apart
    with pytest.raises(ValueError):
        B._out_stride(values[..., 0], 25, cpu)                 # fewer entries than the call writes
    with pytest.raises(ValueError):
        B._out_stride(torch.zeros(1, dtype=torch.int64).expand(8), 8, cpu)  # entries share memory
    with pytest.raises(ValueError):
        B._out_stride(values[..., 0].to(torch.int32), 24, cpu)
    big = torch.zeros((2, B.KVCK_MAX_OUT_STRIDE + 1), dtype=torch.int64)
    with pytest.raises(ValueError):
        B._out_stride(big[:, 0], 2, cpu)

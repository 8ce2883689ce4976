"""ctypes binding of libkvck (include/kvck.h): argument marshalling only.

Every step of the checksum runs in the HIP kernels of ``libkvck.so``; this
module turns torch tensors into pointers, byte strides and sizes, picks the
current HIP stream, and raises on a negative status.  There is no fallback:
if the library is missing or the device is not a gfx950 GPU, calls fail.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVCK_LIB", os.path.join(_PKG, "libkvck.so"))

KVCK_OK = 0
STATUS_NAMES = {
    0: "KVCK_OK", -1: "KVCK_ERR_INVALID_ARGUMENT", -2: "KVCK_ERR_UNSUPPORTED", -3: "KVCK_ERR_MISALIGNED",
    -4: "KVCK_ERR_WORKSPACE", -5: "KVCK_ERR_HIP", -6: "KVCK_ERR_NO_DEVICE", -7: "KVCK_ERR_SCRATCH",
}
KVCK_ABI_VERSION = 3
KVCK_SCRATCH_BYTES = 32 << 20
KVCK_MAX_OUT_STRIDE = 65536
KVCK_MAX_CACHES = 4096
KVCK_FLAG_BAD_BLOCK_ID = 1
KVCK_FLAG_BAD_REQUEST = 2
KVCK_FLAG_BAD_STATE_SLOT = 4
KVCK_FLAG_STAGING_FULL = 8
KVCK_COPY_SAVE = 0
KVCK_COPY_LOAD = 1

# symbols include/kvck.h declares
EXPORTS = ("kvck_checksum_blocks", "kvck_blocks_workspace_bytes", "kvck_checksum_blocks_noalloc",
           "kvck_checksum_states",
           "kvck_states_workspace_bytes", "kvck_copy_checksum_blocks", "kvck_staging_bytes", "kvck_tag_checksums",
           "kvck_instrument", "kvck_instrument_read",
           "kvck_status_string",
           "kvck_platform_supported", "kvck_abi_version")


class KvckError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}{': ' + what if what else ''}")


class KvckDeviceError(RuntimeError):
    """Error bits the kernels raised in *error_flags."""

    def __init__(self, flags: int):
        self.flags = flags
        names = [n for bit, n in ((1, "BAD_BLOCK_ID"), (2, "BAD_REQUEST"), (4, "BAD_STATE_SLOT"),
                                  (8, "STAGING_FULL")) if flags & bit]
        super().__init__("device reported " + "|".join(names))


class kvck_kv_layout(ctypes.Structure):
    _fields_ = [("planes", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("row_bytes", ctypes.c_int32), ("num_blocks", ctypes.c_int64), ("plane_stride", ctypes.c_int64),
                ("block_stride", ctypes.c_int64), ("slot_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("chunk_bytes", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("chunk_stride", ctypes.c_int64),
                ("plane_begin", ctypes.c_int32), ("plane_count", ctypes.c_int32)]


class kvck_state_desc(ctypes.Structure):
    _fields_ = [("slot_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64), ("row_elems", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32)]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libkvck.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_kv_cache_kvck_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kvck_checksum_blocks.restype = i32
    lib.kvck_checksum_blocks.argtypes = [
        ctypes.POINTER(kvck_kv_layout), ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(i32), i32,
        i32, i32, vp, i64, vp, vp, vp, i32, i32, vp, i64, i32, vp, sz, vp, vp]
    lib.kvck_checksum_blocks_noalloc.restype = i32
    lib.kvck_checksum_blocks_noalloc.argtypes = [
        ctypes.POINTER(kvck_kv_layout), ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(i32), i32,
        i32, i32, vp, i64, vp, vp, vp, i32, i32, vp, i64, i32, vp, vp]
    lib.kvck_blocks_workspace_bytes.restype = sz
    lib.kvck_blocks_workspace_bytes.argtypes = [i32, i32, i32]
    lib.kvck_checksum_states.restype = i32
    lib.kvck_checksum_states.argtypes = [
        ctypes.POINTER(kvck_state_desc), i32, ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(i32), i32,
        i32, i32, i32, i32, vp, i32, vp, i64, i32, vp, sz, vp, vp]
    lib.kvck_states_workspace_bytes.restype = sz
    lib.kvck_states_workspace_bytes.argtypes = [i32, i32, i32]
    lib.kvck_status_string.restype = ctypes.c_char_p
    lib.kvck_status_string.argtypes = [i32]
    lib.kvck_platform_supported.restype = i32
    lib.kvck_platform_supported.argtypes = []
    lib.kvck_abi_version.restype = i32
    lib.kvck_abi_version.argtypes = []
    lib.kvck_copy_checksum_blocks.restype = i32
    lib.kvck_copy_checksum_blocks.argtypes = [
        i32, ctypes.POINTER(kvck_kv_layout), ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(i32), i32,
        i32, i32, vp, i64, vp, vp, vp, i32, i32, vp, i64, vp, i64, i32, vp, sz, vp, vp]
    lib.kvck_staging_bytes.restype = sz
    lib.kvck_staging_bytes.argtypes = [ctypes.POINTER(kvck_kv_layout), i32, i32]
    lib.kvck_tag_checksums.restype = i32
    lib.kvck_tag_checksums.argtypes = [vp, i32, vp, i64, ctypes.c_uint64, i64, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.kvck_instrument.restype = i32
    lib.kvck_instrument.argtypes = [i32]
    lib.kvck_instrument_read.restype = i32
    lib.kvck_instrument_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    if lib.kvck_abi_version() != KVCK_ABI_VERSION:
        raise RuntimeError(f"{p} has ABI version {lib.kvck_abi_version()}, this binding needs {KVCK_ABI_VERSION}: "
                           "rebuild it with `python -m paged_kv_cache_kvck_amd.build`")
    if path is None:
        _lib = lib
    return lib


def kvck_status_string(status: int) -> str:
    return load_library().kvck_status_string(int(status)).decode()


def kvck_platform_supported() -> bool:
    return bool(load_library().kvck_platform_supported())


def kvck_abi_version() -> int:
    return int(load_library().kvck_abi_version())


def kvck_instrument(enable: bool) -> None:
    """Record HIP events around every call's main pass (see include/kvck.h)."""
    _check(load_library().kvck_instrument(int(bool(enable))), "kvck_instrument")


def kvck_instrument_read() -> tuple[float, int]:
    """(summed main-pass milliseconds, calls timed) since the last read."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().kvck_instrument_read(ctypes.byref(ms), ctypes.byref(n)), "kvck_instrument_read")
    return ms.value, n.value


def kvck_blocks_workspace_bytes(num_caches: int, num_reqs: int, max_blocks: int) -> int:
    return int(load_library().kvck_blocks_workspace_bytes(num_caches, num_reqs, max_blocks))


def kvck_states_workspace_bytes(num_layers: int, row_count: int, num_reqs: int) -> int:
    return int(load_library().kvck_states_workspace_bytes(num_layers, row_count, num_reqs))


def _check(status: int, what: str = ""):
    if status != KVCK_OK:
        raise KvckError(int(status), what)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device, allocated=()) -> int:
    """The HIP stream a call's kernels run on: ``stream`` (a torch stream or a
    raw hipStream_t), else the current stream.  The binding fills and allocates
    on the current stream (a zeroed ``out``, the workspace, the flag word), so
    when the call runs elsewhere its stream first waits for the current
    stream's work, and the ``allocated`` tensors are recorded as in use on it:
    the caching allocator then does not hand their memory out again before
    the call's kernels are done."""
    cur = torch.cuda.current_stream(device)
    if stream is None:
        return cur.cuda_stream
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if handle != cur.cuda_stream:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(handle, device=device)
        s.wait_stream(cur)
        for t in allocated:
            if t is not None:
                t.record_stream(s)
    return handle


# ----------------------------------------------------------------- layouts

# Pool tensor layouts the binding understands (semantic shapes):
#   NHD      (2, num_blocks, block_size, num_heads, head_size)   K and V (vLLM flash-attention pool)
#   HND      (2, num_blocks, num_heads, block_size, head_size)   K and V
#   FI_NHD   (num_blocks, 2, block_size, num_heads, head_size)   K and V inside each block
#   FI_HND   (num_blocks, 2, num_heads, block_size, head_size)
#   MLA      (num_blocks, block_size, head_size)                 one latent plane
#   K_NHD / V_NHD   (num_blocks, block_size, num_heads, head_size)   one plane of a K/V slice
#   K_HND / V_HND   (num_blocks, num_heads, block_size, head_size)
#   K_XSPLIT (num_blocks, num_heads, head_size/x, block_size, x)  x-split K plane
#   K_TRANS / V_TRANS (num_blocks, num_heads, head_size, block_size)  element-transposed plane
#            (V_TRANS with K_XSPLIT is the K/V cache of ROCm's paged-attention kernels)
LAYOUT_NAMES = ("NHD", "HND", "FI_NHD", "FI_HND", "MLA", "K_NHD", "V_NHD", "K_HND", "V_HND", "K_XSPLIT",
                "K_TRANS", "V_TRANS")


def kv_layout(cache: torch.Tensor, layout: str) -> kvck_kv_layout:
    """Byte layout (kvck_kv_layout) of a pool tensor in one of LAYOUT_NAMES."""
    es = cache.element_size()
    st = [x * es for x in cache.stride()]
    sh = cache.shape
    if cache.stride(-1) != 1:
        raise ValueError("the innermost dimension must be contiguous")
    L = kvck_kv_layout()

    def need(dims, what):
        if cache.dim() != dims:
            raise ValueError(f"{layout} pools are {what}")

    if layout in ("NHD", "HND"):
        need(5, "(2, num_blocks, ., ., head_size)")
        if sh[0] != 2:
            raise ValueError("the first dimension holds K and V")
        L.planes, L.num_blocks, L.plane_stride, L.block_stride = 2, sh[1], st[0], st[1]
        if layout == "NHD":
            L.block_size, L.num_heads, L.slot_stride, L.head_stride = sh[2], sh[3], st[2], st[3]
        else:
            L.num_heads, L.block_size, L.head_stride, L.slot_stride = sh[2], sh[3], st[2], st[3]
        L.row_bytes = sh[4] * es
    elif layout in ("FI_NHD", "FI_HND"):
        need(5, "(num_blocks, 2, ., ., head_size)")
        if sh[1] != 2:
            raise ValueError("the second dimension holds K and V")
        L.planes, L.num_blocks, L.block_stride, L.plane_stride = 2, sh[0], st[0], st[1]
        if layout == "FI_NHD":
            L.block_size, L.num_heads, L.slot_stride, L.head_stride = sh[2], sh[3], st[2], st[3]
        else:
            L.num_heads, L.block_size, L.head_stride, L.slot_stride = sh[2], sh[3], st[2], st[3]
        L.row_bytes = sh[4] * es
    elif layout == "MLA":
        need(3, "(num_blocks, block_size, head_size)")
        L.planes, L.num_blocks, L.block_size, L.num_heads = 1, sh[0], sh[1], 1
        L.plane_stride, L.block_stride, L.slot_stride, L.head_stride = 0, st[0], st[1], 0
        L.row_bytes = sh[2] * es
    elif layout in ("K_NHD", "V_NHD", "K_HND", "V_HND"):
        need(4, "(num_blocks, ., ., head_size)")
        L.planes, L.plane_begin, L.plane_count = 2, (0 if layout[0] == "K" else 1), 1
        L.num_blocks, L.block_stride = sh[0], st[0]
        if layout.endswith("NHD"):
            L.block_size, L.num_heads, L.slot_stride, L.head_stride = sh[1], sh[2], st[1], st[2]
        else:
            L.num_heads, L.block_size, L.head_stride, L.slot_stride = sh[1], sh[2], st[1], st[2]
        L.row_bytes = sh[3] * es
    elif layout == "K_XSPLIT":
        need(5, "(num_blocks, num_heads, head_size/x, block_size, x)")
        L.planes, L.plane_begin, L.plane_count = 2, 0, 1
        L.num_blocks, L.num_heads, L.block_size = sh[0], sh[1], sh[3]
        L.block_stride, L.head_stride, L.chunk_stride, L.slot_stride = st[0], st[1], st[2], st[3]
        L.chunk_bytes = sh[4] * es
        L.row_bytes = sh[2] * sh[4] * es
    elif layout in ("K_TRANS", "V_TRANS"):
        need(4, "(num_blocks, num_heads, head_size, block_size)")
        L.planes, L.plane_begin, L.plane_count = 2, (0 if layout[0] == "K" else 1), 1
        L.num_blocks, L.num_heads, L.block_size = sh[0], sh[1], sh[3]
        L.block_stride, L.head_stride, L.chunk_stride, L.slot_stride = st[0], st[1], st[2], st[3]
        L.chunk_bytes = es                    # a row is head_size one-element runs
        L.row_bytes = sh[2] * es
    else:
        raise ValueError(f"unknown layout {layout!r}; one of {LAYOUT_NAMES}")
    return L


def _meta(t: torch.Tensor, dtype, name, device, n=None):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor on {device}")
    if n is not None and (t.dim() != 1 or t.shape[0] != n or not t.is_contiguous()):
        raise ValueError(f"{name} must be contiguous with {n} entries")
    return t


class PreparedCaches:
    """A set of pool tensors validated and marshalled once (layout, device
    pointers, layer numbers, global head bases), for calls in a hot loop: pass
    it as ``caches`` to kvck_checksum_blocks / kvck_copy_checksum_blocks.  It
    keeps the tensors alive; their storage must not move between calls."""

    def __init__(self, caches, layout, layer_numbers, global_head_base=None, head_begin: int = 0,
                 head_count: int | None = None, planes: tuple | None = None):
        caches = list(caches)
        if not caches:
            raise ValueError("no caches")
        self.tensors = caches
        self.device = caches[0].device
        self.layout_name = layout
        L = kv_layout(caches[0], layout)
        plane_off = 0
        if planes is not None:
            # a subset (begin, count) of the planes of a pool that holds all of them
            if L.plane_count != 0 or L.planes != 2:
                raise ValueError("planes= selects K or V of a pool holding both")
            L.plane_begin, L.plane_count = int(planes[0]), int(planes[1])
            plane_off = L.plane_begin * L.plane_stride
        ref = caches[0]
        for c in caches[1:]:
            if c.shape != ref.shape or c.stride() != ref.stride() or c.dtype != ref.dtype or c.device != ref.device:
                raise ValueError("every cache of a call must share shape, strides, dtype and device")
        n = len(caches)
        if head_count is None:
            head_count = L.num_heads - head_begin
        if global_head_base is None:
            global_head_base = [head_begin] * n
        elif isinstance(global_head_base, int):
            global_head_base = [global_head_base] * n
        if len(layer_numbers) != n or len(global_head_base) != n:
            raise ValueError("one layer number and one global head base per cache")
        self.layout = L
        self.n = n
        self.head_begin = int(head_begin)
        self.head_count = int(head_count)
        self.ptrs = (ctypes.c_void_p * n)(*[c.data_ptr() + plane_off for c in caches])
        self.layers = (ctypes.c_int32 * n)(*[int(x) for x in layer_numbers])
        self.bases = (ctypes.c_int32 * n)(*[int(x) for x in global_head_base])


def prepare_caches(caches, layout, layer_numbers, global_head_base=None, head_begin: int = 0,
                   head_count: int | None = None, planes: tuple | None = None) -> PreparedCaches:
    return PreparedCaches(caches, layout, layer_numbers, global_head_base, head_begin, head_count, planes)


def _out_stride(out, entries: int, dev) -> int:
    """Element stride of an output tensor whose entries, in row-major order,
    are evenly spaced in memory: 1 for a contiguous tensor, C for one column
    ``values[..., c]`` of a row-major array with C replica columns."""
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.uint64, torch.int64) or out.device != dev:
        raise ValueError(f"out must be a uint64 tensor on {dev}")
    if out.numel() < entries:
        raise ValueError(f"out holds {out.numel()} entries, the call writes up to {entries}")
    if out.is_contiguous():
        return 1
    step = out.stride(-1) if out.dim() else 1
    inner = 1
    for d in range(out.dim() - 1, -1, -1):
        if out.shape[d] > 1 and out.stride(d) != step * inner:
            raise ValueError("out's entries must be evenly spaced in row-major order (e.g. values[..., c])")
        inner *= out.shape[d]
    if not 1 <= step <= KVCK_MAX_OUT_STRIDE:
        raise ValueError(f"out's element stride {step} is outside 1..{KVCK_MAX_OUT_STRIDE}")
    return step


def _blocks_args(caches, layout, layer_numbers, block_table, num_blocks_per_req, start_pos, num_tokens,
                 global_head_base, head_begin, head_count, out, workspace, check, error_flags, planes=None):
    lib = load_library()
    pc = caches if isinstance(caches, PreparedCaches) else PreparedCaches(
        caches, layout, layer_numbers, global_head_base, head_begin, head_count, planes)
    dev = pc.device
    n = pc.n
    _meta(block_table, torch.int32, "block_table", dev)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with contiguous rows")
    R, max_blocks = block_table.shape
    _meta(num_blocks_per_req, torch.int32, "num_blocks_per_req", dev, R)
    _meta(start_pos, torch.int64, "start_pos", dev, R)
    _meta(num_tokens, torch.int64, "num_tokens", dev, R)
    allocated = []
    if out is None:
        out = torch.zeros((R, max_blocks), dtype=torch.uint64, device=dev)
        allocated.append(out)
    out_stride = _out_stride(out, R * max_blocks, dev)
    need = int(lib.kvck_blocks_workspace_bytes(n, R, max_blocks))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        allocated.append(workspace)
    fresh_flags = check and error_flags is None
    error_flags = _flag_word(error_flags, check, dev)
    if fresh_flags:
        allocated.append(error_flags)
    return dict(lib=lib, dev=dev, L=pc.layout, n=n, head_begin=pc.head_begin, head_count=pc.head_count, R=R,
                max_blocks=max_blocks, out=out, out_stride=out_stride, workspace=workspace, error_flags=error_flags, ptrs=pc.ptrs,
                layers=pc.layers, bases=pc.bases, allocated=allocated)


def _flag_word(error_flags, check, dev):
    """The kernels' error word.  With check=True it is a fresh or cleared word,
    and the device is synchronized after clearing it, so the clear lands before
    the call's kernels whichever stream they run on."""
    if error_flags is not None and (error_flags.dtype not in (torch.int32, torch.uint32)
                                    or error_flags.numel() < 1 or error_flags.device != dev):
        raise ValueError(f"error_flags must be a 32-bit tensor on {dev}")
    if not check:
        return error_flags
    if error_flags is None:
        error_flags = torch.zeros(1, dtype=torch.int32, device=dev)
    else:
        error_flags.zero_()
    torch.cuda.synchronize(dev)
    return error_flags


def _finish(a, check):
    if check:
        torch.cuda.synchronize(a["dev"])
        flags = int(a["error_flags"].item())
        if flags:
            raise KvckDeviceError(flags)
    return a["out"]


def kvck_checksum_blocks(caches, layout: str | None, layer_numbers: Sequence[int] | None,
                         block_table: torch.Tensor, num_blocks_per_req: torch.Tensor, start_pos: torch.Tensor,
                         num_tokens: torch.Tensor, global_head_base=None, head_begin: int = 0,
                         head_count: int | None = None, out: torch.Tensor | None = None, accumulate: bool = False,
                         workspace: torch.Tensor | None = None, error_flags: torch.Tensor | None = None,
                         stream=None, check: bool = False, planes: tuple | None = None) -> torch.Tensor:
    """Per block position checksums of paged K/V (see include/kvck.h).

    ``caches`` is a list of pool tensors or a PreparedCaches (then the
    layout, layer, head and plane arguments are taken from it).  ``layout`` is
    one of LAYOUT_NAMES; ``planes=(begin, count)`` restricts a pool holding K
    and V to K (0, 1) or V (1, 1) -- partials over K and V add up to the
    checksum of both.

    Returns ``out``: uint64 (num_reqs, max_blocks) on the caches' device;
    entries past a request's listed positions are left as they were.  A
    given ``out`` may be one replica column ``values[..., c]`` of a
    (num_reqs, max_blocks, C) array (any view whose entries are evenly
    spaced): the call then fills that column.
    ``check=True`` zeroes a flag word, synchronizes, and raises
    ``KvckDeviceError`` if the kernels flagged a bad block id or request.
    """
    a = _blocks_args(caches, layout, layer_numbers, block_table, num_blocks_per_req, start_pos, num_tokens,
                     global_head_base, head_begin, head_count, out, workspace, check, error_flags, planes)
    ws = a["workspace"]
    st = a["lib"].kvck_checksum_blocks(
        ctypes.byref(a["L"]), a["ptrs"], a["layers"], a["bases"], a["n"], a["head_begin"], a["head_count"],
        block_table.data_ptr(), block_table.stride(0), num_blocks_per_req.data_ptr(), start_pos.data_ptr(),
        num_tokens.data_ptr(), a["R"], a["max_blocks"], a["out"].data_ptr(), a["out_stride"], int(bool(accumulate)),
        ws.data_ptr(), ws.numel() * ws.element_size(), _ptr(a["error_flags"]),
        _stream_handle(stream, a["dev"], a["allocated"]))
    _check(st, "kvck_checksum_blocks")
    return _finish(a, check)


class PreparedCall:
    """One kvck_checksum_blocks call with every argument marshalled once, for
    the smallest calls in a hot loop, where the wrapper's checks cost more
    than the kernel: calling the object makes the C call and checks its
    status, nothing else.  Made by prepare_call; it keeps its tensors alive,
    and their storage must not move between calls."""

    def __init__(self, caches: PreparedCaches, block_table, num_blocks_per_req, start_pos, num_tokens, out,
                 workspace, accumulate=False, error_flags=None, stream=None):
        if not isinstance(caches, PreparedCaches):
            raise ValueError("prepare_call takes a PreparedCaches (see prepare_caches)")
        dev = caches.device
        _meta(block_table, torch.int32, "block_table", dev)
        if block_table.dim() != 2 or block_table.stride(1) != 1:
            raise ValueError("block_table must be 2-D with contiguous rows")
        R, max_blocks = block_table.shape
        _meta(num_blocks_per_req, torch.int32, "num_blocks_per_req", dev, R)
        _meta(start_pos, torch.int64, "start_pos", dev, R)
        _meta(num_tokens, torch.int64, "num_tokens", dev, R)
        out_stride = _out_stride(out, R * max_blocks, dev)
        lib = load_library()
        need = int(lib.kvck_blocks_workspace_bytes(caches.n, R, max_blocks))
        if not isinstance(workspace, torch.Tensor) or workspace.device != dev or \
                workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace must be a tensor of at least {need} bytes on {dev}")
        error_flags = _flag_word(error_flags, False, dev)
        self._keep = (caches, block_table, num_blocks_per_req, start_pos, num_tokens, out, workspace, error_flags)
        self.out = out
        self._fn = lib.kvck_checksum_blocks
        self._args = (ctypes.byref(caches.layout), caches.ptrs, caches.layers, caches.bases, caches.n,
                      caches.head_begin, caches.head_count, block_table.data_ptr(), block_table.stride(0),
                      num_blocks_per_req.data_ptr(), start_pos.data_ptr(), num_tokens.data_ptr(), R, max_blocks,
                      out.data_ptr(), out_stride, int(bool(accumulate)), workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), _ptr(error_flags), _stream_handle(stream, dev))

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise KvckError(int(st), "kvck_checksum_blocks")
        return self.out


def prepare_call(caches: PreparedCaches, block_table, num_blocks_per_req, start_pos, num_tokens, out, workspace,
                 accumulate=False, error_flags=None, stream=None) -> PreparedCall:
    """A PreparedCall of kvck_checksum_blocks on prepared caches, with a given
    ``out`` and workspace.  Every call runs on ``stream``, else on the stream
    that is current when the call is prepared (not when it is made); ordering
    ``out``, the workspace and the inputs against other work on other streams
    is the caller's, as with any call given its own buffers."""
    return PreparedCall(caches, block_table, num_blocks_per_req, start_pos, num_tokens, out, workspace, accumulate,
                        error_flags, stream)


def kvck_checksum_blocks_noalloc(caches, layout: str | None, layer_numbers: Sequence[int] | None,
                                 block_table: torch.Tensor, num_blocks_per_req: torch.Tensor, start_pos: torch.Tensor,
                                 num_tokens: torch.Tensor, out: torch.Tensor, global_head_base=None,
                                 head_begin: int = 0, head_count: int | None = None, accumulate: bool = False,
                                 error_flags: torch.Tensor | None = None, stream=None,
                                 planes: tuple | None = None) -> torch.Tensor:
    """kvck_checksum_blocks without a workspace: the library's per-device
    scratch array (KVCK_SCRATCH_BYTES) takes its place, and the call itself
    allocates nothing (see include/kvck.h).  ``out`` is required, so that
    this wrapper allocates nothing either.  Calls that overlap on one device
    share that scratch and race; calls ordered on one stream do not."""
    lib = load_library()
    pc = caches if isinstance(caches, PreparedCaches) else PreparedCaches(
        caches, layout, layer_numbers, global_head_base, head_begin, head_count, planes)
    dev = pc.device
    _meta(block_table, torch.int32, "block_table", dev)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with contiguous rows")
    R, max_blocks = block_table.shape
    _meta(num_blocks_per_req, torch.int32, "num_blocks_per_req", dev, R)
    _meta(start_pos, torch.int64, "start_pos", dev, R)
    _meta(num_tokens, torch.int64, "num_tokens", dev, R)
    out_stride = _out_stride(out, R * max_blocks, dev)
    error_flags = _flag_word(error_flags, False, dev)
    st = lib.kvck_checksum_blocks_noalloc(
        ctypes.byref(pc.layout), pc.ptrs, pc.layers, pc.bases, pc.n, pc.head_begin, pc.head_count,
        block_table.data_ptr(), block_table.stride(0), num_blocks_per_req.data_ptr(), start_pos.data_ptr(),
        num_tokens.data_ptr(), R, max_blocks, out.data_ptr(), out_stride, int(bool(accumulate)), _ptr(error_flags),
        _stream_handle(stream, dev))
    _check(st, "kvck_checksum_blocks_noalloc")
    return out


def kvck_staging_bytes(cache: torch.Tensor, layout: str, num_caches: int, head_count: int | None = None) -> int:
    """Staging bytes per listed position for kvck_copy_checksum_blocks."""
    L = kv_layout(cache, layout)
    return int(load_library().kvck_staging_bytes(ctypes.byref(L), int(num_caches),
                                                 int(L.num_heads if head_count is None else head_count)))


def kvck_copy_checksum_blocks(direction: int, caches, layout: str | None,
                              layer_numbers: Sequence[int] | None, block_table: torch.Tensor,
                              num_blocks_per_req: torch.Tensor, start_pos: torch.Tensor, num_tokens: torch.Tensor,
                              staging: torch.Tensor, global_head_base=None, head_begin: int = 0,
                              head_count: int | None = None, out: torch.Tensor | None = None,
                              accumulate: bool = False, workspace: torch.Tensor | None = None,
                              error_flags: torch.Tensor | None = None, stream=None, check: bool = False,
                              planes: tuple | None = None):
    """A connector save (KVCK_COPY_SAVE: pool -> staging) or load
    (KVCK_COPY_LOAD: staging -> pool) fused with the checksum; see
    include/kvck.h for the staging layout.  Returns the checksums."""
    a = _blocks_args(caches, layout, layer_numbers, block_table, num_blocks_per_req, start_pos, num_tokens,
                     global_head_base, head_begin, head_count, out, workspace, check, error_flags, planes)
    if staging.device != a["dev"] or not staging.is_contiguous():
        raise ValueError("staging must be a contiguous tensor on the caches' device")
    per = int(a["lib"].kvck_staging_bytes(ctypes.byref(a["L"]), a["n"], int(a["head_count"])))
    positions = (staging.numel() * staging.element_size()) // per
    ws = a["workspace"]
    st = a["lib"].kvck_copy_checksum_blocks(
        int(direction), ctypes.byref(a["L"]), a["ptrs"], a["layers"], a["bases"], a["n"], a["head_begin"],
        a["head_count"], block_table.data_ptr(), block_table.stride(0), num_blocks_per_req.data_ptr(),
        start_pos.data_ptr(), num_tokens.data_ptr(), a["R"], a["max_blocks"], staging.data_ptr(), positions,
        a["out"].data_ptr(), a["out_stride"], int(bool(accumulate)), ws.data_ptr(), ws.numel() * ws.element_size(),
        _ptr(a["error_flags"]), _stream_handle(stream, a["dev"], a["allocated"]))
    _check(st, "kvck_copy_checksum_blocks")
    return _finish(a, check)


def state_desc(state: torch.Tensor) -> kvck_state_desc:
    """Shape of a Mamba state (num_slots, num_rows, ...) with contiguous rows."""
    if state.dim() < 3:
        raise ValueError("a state is (num_slots, num_rows, ...)")
    es = state.element_size()
    row = state[0, 0]
    if not row.is_contiguous():
        raise ValueError("each state row must be contiguous")
    d = kvck_state_desc()
    d.slot_stride, d.row_stride = state.stride(0) * es, state.stride(1) * es
    d.row_elems, d.elem_bytes = row.numel(), es
    return d


def kvck_checksum_states(layer_states: Sequence[Sequence[torch.Tensor]], layer_numbers: Sequence[int],
                         slot_ids: torch.Tensor, global_row_base=None, row_begin: int = 0,
                         row_count: int | None = None, out: torch.Tensor | None = None, accumulate: bool = False,
                         workspace: torch.Tensor | None = None, error_flags: torch.Tensor | None = None,
                         stream=None, check: bool = False) -> torch.Tensor:
    """Mamba running-state checksums, one uint64 per request (position 0);
    a given ``out`` may be one replica column ``values[:, c]``."""
    lib = load_library()
    layer_states = [list(s) for s in layer_states]
    nl = len(layer_states)
    if nl == 0 or not layer_states[0]:
        raise ValueError("no states")
    ref = layer_states[0]
    k = len(ref)
    dev = ref[0].device
    for sts in layer_states:
        if len(sts) != k:
            raise ValueError("every layer must hold the same states")
        for a, b in zip(sts, ref):
            if a.shape != b.shape or a.stride() != b.stride() or a.dtype != b.dtype or a.device != dev:
                raise ValueError("states of every layer must share shape, strides, dtype and device")
    slots, rows = ref[0].shape[0], ref[0].shape[1]
    for s in ref:
        if s.shape[0] != slots or s.shape[1] != rows:
            raise ValueError("states of a layer must share (num_slots, num_rows)")
    if row_count is None:
        row_count = rows - row_begin
    if global_row_base is None:
        global_row_base = [row_begin] * nl
    elif isinstance(global_row_base, int):
        global_row_base = [global_row_base] * nl
    _meta(slot_ids, torch.int32, "slot_ids", dev)
    R = slot_ids.numel()
    if not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be contiguous")
    allocated = []
    if out is None:
        out = torch.zeros(R, dtype=torch.uint64, device=dev)
        allocated.append(out)
    out_stride = _out_stride(out, R, dev)
    descs = (kvck_state_desc * k)(*[state_desc(s) for s in ref])
    ptrs = (ctypes.c_void_p * (nl * k))(*[s.data_ptr() for sts in layer_states for s in sts])
    layers = (ctypes.c_int32 * nl)(*[int(x) for x in layer_numbers])
    bases = (ctypes.c_int32 * nl)(*[int(x) for x in global_row_base])
    need = int(lib.kvck_states_workspace_bytes(nl, row_count, R))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        allocated.append(workspace)
    if check and error_flags is None:
        error_flags = _flag_word(None, True, dev)
        allocated.append(error_flags)
    else:
        error_flags = _flag_word(error_flags, check, dev)
    st = lib.kvck_checksum_states(
        descs, k, ptrs, layers, bases, nl, slots, rows, int(row_begin), int(row_count), slot_ids.data_ptr(), R,
        out.data_ptr(), out_stride, int(bool(accumulate)), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _ptr(error_flags), _stream_handle(stream, dev, allocated))
    _check(st, "kvck_checksum_states")
    if check:
        torch.cuda.synchronize(dev)
        flags = int(error_flags.item())
        if flags:
            raise KvckDeviceError(flags)
    return out


def kvck_tag_checksums(checksums: torch.Tensor, block_hashes: torch.Tensor, fingerprint: int,
                       num_blocks_per_req: torch.Tensor | None = None, tagged: torch.Tensor | bool | None = True,
                       stored: torch.Tensor | None = None, mismatch: torch.Tensor | bool | None = None,
                       mismatch_count: torch.Tensor | None = None, stream=None, start_pos: torch.Tensor | None = None,
                       block_size: int = 0, columns: int = 1):
    """Tags of offloaded checksums (the page's block_checksum_tags) and the
    load-time comparison; see include/kvck.h.

    ``checksums``: uint64 tensor (e.g. the (num_reqs, max_blocks) output of
    kvck_checksum_blocks, or with ``columns`` = C a (num_reqs, max_blocks, C)
    array of replica columns, each entry's row summed before tagging);
    ``block_hashes``: uint8 (n, hash_bytes >= 8) tensor, row i the hash of the
    block at entry i.  With ``num_blocks_per_req`` only
    listed positions are touched; ``start_pos`` and ``block_size`` (those of
    the checksum call) also skip requests that call rejected.  Returns
    (tagged, mismatch) -- each a tensor or None.
    """
    lib = load_library()
    dev = checksums.device
    columns = int(columns)
    if not 1 <= columns <= KVCK_MAX_OUT_STRIDE or checksums.numel() % columns:
        raise ValueError(f"columns must be in 1..{KVCK_MAX_OUT_STRIDE} and divide the checksum count")
    n = checksums.numel() // columns
    if checksums.dtype not in (torch.uint64, torch.int64) or not checksums.is_contiguous():
        raise ValueError("checksums must be a contiguous uint64 tensor")
    if block_hashes.dtype != torch.uint8 or block_hashes.dim() != 2 or block_hashes.shape[0] != n \
            or block_hashes.stride(1) != 1 or block_hashes.device != dev:
        raise ValueError("block_hashes must be a uint8 (n, hash_bytes) tensor with contiguous rows")
    max_blocks = 0
    if num_blocks_per_req is not None:
        _meta(num_blocks_per_req, torch.int32, "num_blocks_per_req", dev)
        max_blocks = n // max(1, num_blocks_per_req.numel())
        if start_pos is not None:
            _meta(start_pos, torch.int64, "start_pos", dev, num_blocks_per_req.numel())
    elif start_pos is not None:
        raise ValueError("start_pos needs num_blocks_per_req")
    allocated = []
    if tagged is True:
        tagged = torch.zeros(n, dtype=torch.uint64, device=dev)
        allocated.append(tagged)
    elif tagged is False:
        tagged = None
    if mismatch is True or (mismatch is None and stored is not None):
        mismatch = torch.zeros(n, dtype=torch.uint8, device=dev)
        allocated.append(mismatch)
    elif mismatch is False:
        mismatch = None
    st = lib.kvck_tag_checksums(checksums.data_ptr(), columns, block_hashes.data_ptr(), block_hashes.stride(0),
                                ctypes.c_uint64(int(fingerprint) & ((1 << 64) - 1)), n, _ptr(num_blocks_per_req),
                                _ptr(start_pos), max_blocks, int(block_size), _ptr(tagged), _ptr(stored),
                                _ptr(mismatch), _ptr(mismatch_count), _stream_handle(stream, dev, allocated))
    _check(st, "kvck_tag_checksums")
    return tagged, mismatch

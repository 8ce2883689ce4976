"""numpy oracle of the KV-cache block checksum (test infrastructure only).

Source of every formula: the vLLM API page
"vllm.distributed.kv_transfer.kv_checksum.checksum".

Plain transcription of the definition, vectorised only over the tokens and
heads of one (block position, cache).  All arithmetic is numpy ``uint64``,
which wraps modulo 2^64 exactly as the definition asks; no floating point is
used.  Nothing here is blocked, fused or reordered beyond what the definition
states: a slice checksum ``s`` is formed per (layer, head), multiplied by its
factor ``m`` and summed.

Cache tensors are taken in *semantic* shapes, indexed by name, never through
byte strides:

``"NHD"``  (2, num_blocks, block_size, num_heads, head_size)  plane 0 = K, 1 = V
           (the vLLM pool shape "K/V, kernel_num_blocks, kernel_block_size,
           num_kv_heads, head_size" on the page "[vLLM 源码解析] KV Cache",
           section "reshape kv_cache").
``"HND"``  (2, num_blocks, num_heads, block_size, head_size)  -- not on the
           pages; the head-major permutation of the same pool.
``"MLA"``  (num_blocks, block_size, head_size)  one latent plane, one head.
``"FI_NHD"`` (num_blocks, 2, block_size, num_heads, head_size) and ``"FI_HND"``
           (num_blocks, 2, num_heads, block_size, head_size): K and V kept
           together inside each block.

Readings of points the pages leave open:

* A token's slice bytes are its K row (head_size elements in memory order)
  followed by its V row; pieces 0 .. P/2-1 come from K.  MLA: the latent row.
* Elements are raw bits; the dtype only fixes the byte count.
* Position ``pos`` holds tokens ``pos*block_size + i``; ``num_tokens`` counts
  from the request's first token.
* Mamba: slice g of a layer is row g of every state of that layer, concatenated
  in the order the states are given, elements in C order, numbered from 0.
"""

from __future__ import annotations

import numpy as np

# Page attribute MAX_KV_HEADS_PER_LAYER (2^16): the H of the slice factor, a
# fixed upper bound on KV heads per layer; a group above it gets no checksum.
MAX_KV_HEADS_PER_LAYER = 1 << 16
# Page attribute BLOCK_CHECKSUM_BYTES: one int64 per block.
BLOCK_CHECKSUM_BYTES = 8

LAYOUTS = ("NHD", "HND", "MLA", "FI_NHD", "FI_HND")

_U64 = np.uint64
_MASK = (1 << 64) - 1


def num_valid_tokens(position: int, block_size: int, num_tokens: int) -> int:
    """Slots of block ``position`` that hold one of the request's first
    ``num_tokens`` tokens (page helper of the same name).  The block spans
    tokens [first, first + block_size) with first = position*block_size; the
    count is the length of that span's overlap with [0, num_tokens)."""
    first = position * block_size
    last = min(first + block_size, num_tokens)
    return last - first if last > first else 0


def slice_factor(layer: int, head: int) -> int:
    """m = 2 * (layer * H + head) + 1 mod 2^64 (module docstring, item 2)."""
    return (2 * (layer * MAX_KV_HEADS_PER_LAYER + head) + 1) & _MASK


def _block_size(cache: np.ndarray, layout: str) -> int:
    if layout in ("NHD", "FI_NHD"):
        return cache.shape[2]
    if layout in ("HND", "FI_HND"):
        return cache.shape[3]
    if layout == "MLA":
        return cache.shape[1]
    raise ValueError(f"unknown layout {layout!r}")


def _num_heads(cache: np.ndarray, layout: str) -> int:
    if layout in ("NHD", "FI_NHD"):
        return cache.shape[3]
    if layout in ("HND", "FI_HND"):
        return cache.shape[2]
    return 1


def _num_blocks(cache: np.ndarray, layout: str) -> int:
    return cache.shape[1] if layout in ("NHD", "HND") else cache.shape[0]


def _token_rows(cache: np.ndarray, layout: str, b: int, v: int, h0: int, n: int) -> np.ndarray:
    """Bytes of the first ``v`` tokens of block ``b`` for local heads h0..h0+n-1.

    Returns uint8 (v, n, row_bytes): per token and head, the K row then the V
    row -- a slice is the K and V of one head, token after token (module
    docstring, item 1)."""
    if layout == "NHD":
        planes = [cache[p, b, :v, h0:h0 + n, :] for p in (0, 1)]
    elif layout == "HND":
        planes = [np.swapaxes(cache[p, b, h0:h0 + n, :v, :], 0, 1) for p in (0, 1)]
    elif layout == "FI_NHD":
        planes = [cache[b, p, :v, h0:h0 + n, :] for p in (0, 1)]
    elif layout == "FI_HND":
        planes = [np.swapaxes(cache[b, p, h0:h0 + n, :v, :], 0, 1) for p in (0, 1)]
    elif layout == "MLA":
        if (h0, n) != (0, 1):
            raise ValueError("an MLA cache has exactly one head")
        planes = [cache[b, :v, None, :]]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    rows = [np.ascontiguousarray(p).view(np.uint8).reshape(v, n, -1) for p in planes]
    return np.concatenate(rows, axis=2)


def checksum_position(caches, layout, layer_numbers, global_head_base, block_id,
                      position, num_tokens, head_begin=0, head_count=None) -> int:
    """Checksum c of one block position, summed over the given caches.

    ``caches[i]`` is one layer's cache (semantic shape above), numbered
    ``layer_numbers[i]``; its local head ``head_begin + k`` is global head
    ``global_head_base[i] + k``.  Returns a Python int in [0, 2^64).
    """
    if position < 0:
        raise ValueError("negative block position")
    c = _U64(0)
    for cache, layer, g0 in zip(caches, layer_numbers, global_head_base):
        bs = _block_size(cache, layout)
        nh = _num_heads(cache, layout)
        n = nh - head_begin if head_count is None else head_count
        if g0 + n > MAX_KV_HEADS_PER_LAYER:
            raise ValueError("more KV heads than MAX_KV_HEADS_PER_LAYER: not checksummed")
        v = num_valid_tokens(position, bs, num_tokens)
        if v == 0:
            continue
        if not 0 <= block_id < _num_blocks(cache, layout):
            raise IndexError(f"block id {block_id} outside the pool")
        rows = _token_rows(cache, layout, block_id, v, head_begin, n)
        if rows.shape[2] % 8:
            raise ValueError("a token's slice bytes are not a whole number of 8-byte pieces")
        # little-endian 8-byte pieces x, shape (v tokens, n heads, P pieces)
        x = rows.view("<u8")
        P = x.shape[2]
        with np.errstate(over="ignore"):
            # token position t in the request, piece index j = t*P + p
            t = _U64(position * bs) + np.arange(v, dtype=_U64)
            j = t[:, None] * _U64(P) + np.arange(P, dtype=_U64)[None, :]
            odd = _U64(2) * j + _U64(1)
            # s per (layer, head) slice: sum_j x_j (2j+1)
            s = (x * odd[:, None, :]).sum(axis=(0, 2), dtype=_U64)
            heads = _U64(g0) + np.arange(n, dtype=_U64)
            m = _U64(2) * (_U64(layer) * _U64(MAX_KV_HEADS_PER_LAYER) + heads) + _U64(1)
            c = c + (m * s).sum(dtype=_U64)
    return int(c)


def checksum_blocks(caches, layout, layer_numbers, global_head_base, block_table,
                    num_blocks, start_pos, num_tokens, head_begin=0, head_count=None) -> np.ndarray:
    """Per-position checksums of a batch of requests.

    Request r lists ``num_blocks[r]`` blocks, ``block_table[r, k]`` at block
    position ``start_pos[r] + k`` (``KVChecksumBlocks.groups`` gives a start
    position, then one block id for each following position);
    slots at or past ``num_tokens[r]`` are not checksummed.

    Returns uint64 (num_reqs, block_table.shape[1]); positions a request does
    not list are 0.
    """
    block_table = np.asarray(block_table)
    R, max_blocks = block_table.shape
    out = np.zeros((R, max_blocks), dtype=_U64)
    for r in range(R):
        for k in range(int(num_blocks[r])):
            out[r, k] = checksum_position(
                caches, layout, layer_numbers, global_head_base, int(block_table[r, k]),
                int(start_pos[r]) + k, int(num_tokens[r]), head_begin, head_count)
    return out


def _as_unsigned(state: np.ndarray) -> np.ndarray:
    """Mamba elements are "read unsigned": reinterpret 2- or 4-byte elements."""
    if state.dtype.itemsize == 2:
        return state.view(np.uint16)
    if state.dtype.itemsize == 4:
        return state.view(np.uint32)
    raise ValueError("Mamba state elements must be 2 or 4 bytes")


def checksum_states(layer_states, layer_numbers, global_row_base, slot_ids,
                    row_begin=0, row_count=None) -> np.ndarray:
    """Mamba running-state checksums, one value per request (position 0).

    ``layer_states[l]`` lists the states of Mamba layer ``layer_numbers[l]``,
    each shaped (state_slots, rows, ...); ``slot_ids[r]`` is request r's state
    slot.  Local row ``row_begin + g`` is global row ``global_row_base[l] + g``
    and forms one slice; its pieces are the row's elements of every state, in
    the given state order, read as unsigned 2- or 4-byte integers (Mamba
    paragraph of the module docstring).
    """
    out = np.zeros(len(slot_ids), dtype=_U64)
    for r, b in enumerate(slot_ids):
        c = _U64(0)
        for states, layer, g0 in zip(layer_states, layer_numbers, global_row_base):
            rows = states[0].shape[1]
            n = rows - row_begin if row_count is None else row_count
            if g0 + n > MAX_KV_HEADS_PER_LAYER:
                raise ValueError("more rows than MAX_KV_HEADS_PER_LAYER: not checksummed")
            for g in range(n):
                rho = row_begin + g
                x = np.concatenate([
                    np.ascontiguousarray(_as_unsigned(st)[int(b), rho]).reshape(-1).astype(_U64)
                    for st in states])
                with np.errstate(over="ignore"):
                    e = np.arange(x.size, dtype=_U64)
                    s = (x * (_U64(2) * e + _U64(1))).sum(dtype=_U64)
                    m = _U64(slice_factor(layer, g0 + g))
                    c = c + m * s
        out[r] = c
    return out

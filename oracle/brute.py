"""Pure-Python brute force of the KV-cache block checksum (test infrastructure only).

Independent of ``kv_checksum``: one piece at a time, unbounded Python integers,
one reduction mod 2^64 at the very end.  Meant for tiny inputs only (thousands
of pieces); it pins the numpy oracle.

Definition (vLLM API page "vllm.distributed.kv_transfer.kv_checksum.checksum",
module docstring items 1 and 2, Mamba paragraph):

    s(layer, head) = sum_j x_j (2j + 1),   j = t*P + p
    c(position)    = sum_{layer, head} (2 (layer*65536 + head) + 1) * s   mod 2^64

Layouts are the semantic shapes documented in ``oracle.kv_checksum``.
"""

from __future__ import annotations

H = 1 << 16


def _valid(position, block_size, num_tokens):
    # tokens of the block that are among the first num_tokens, counted one by one
    return sum(1 for t in range(position * block_size, (position + 1) * block_size)
               if t < num_tokens)


def _row_bytes(cache, layout, plane, b, i, h) -> bytes:
    if layout == "NHD":
        return cache[plane, b, i, h, :].tobytes()
    if layout == "HND":
        return cache[plane, b, h, i, :].tobytes()
    if layout == "FI_NHD":
        return cache[b, plane, i, h, :].tobytes()
    if layout == "FI_HND":
        return cache[b, plane, h, i, :].tobytes()
    if layout == "MLA":
        return cache[b, i, :].tobytes()
    raise ValueError(layout)


def position_checksum(caches, layout, layer_numbers, global_head_base, block_id, position,
                      num_tokens, head_begin=0, head_count=None) -> int:
    total = 0
    for cache, layer, g0 in zip(caches, layer_numbers, global_head_base):
        if layout in ("NHD", "FI_NHD"):
            bs, nh, planes = cache.shape[2], cache.shape[3], (0, 1)
        elif layout in ("HND", "FI_HND"):
            bs, nh, planes = cache.shape[3], cache.shape[2], (0, 1)
        else:
            bs, nh, planes = cache.shape[1], 1, (0,)
        n = nh - head_begin if head_count is None else head_count
        v = _valid(position, bs, num_tokens)
        for k in range(n):
            h = head_begin + k
            m = 2 * (layer * H + g0 + k) + 1
            s = 0
            for i in range(v):
                t = position * bs + i
                token = b"".join(_row_bytes(cache, layout, pl, block_id, i, h) for pl in planes)
                P = len(token) // 8
                assert P * 8 == len(token)
                for p in range(P):
                    x = int.from_bytes(token[8 * p:8 * p + 8], "little")
                    s += x * (2 * (t * P + p) + 1)
            total += m * s
    return total % (1 << 64)


def blocks(caches, layout, layer_numbers, global_head_base, block_table, num_blocks,
           start_pos, num_tokens, head_begin=0, head_count=None):
    """dict {(r, k): c} for every listed position."""
    res = {}
    for r in range(len(num_blocks)):
        for k in range(int(num_blocks[r])):
            res[(r, k)] = position_checksum(
                caches, layout, layer_numbers, global_head_base, int(block_table[r][k]),
                int(start_pos[r]) + k, int(num_tokens[r]), head_begin, head_count)
    return res


def states(layer_states, layer_numbers, global_row_base, slot_ids, row_begin=0, row_count=None):
    """list of per-request Mamba checksums (position 0)."""
    res = []
    for b in slot_ids:
        total = 0
        for sts, layer, g0 in zip(layer_states, layer_numbers, global_row_base):
            rows = sts[0].shape[1]
            n = rows - row_begin if row_count is None else row_count
            for g in range(n):
                elems = []
                for st in sts:
                    w = st.dtype.itemsize
                    raw = st[int(b), row_begin + g].tobytes()
                    elems += [int.from_bytes(raw[q:q + w], "little") for q in range(0, len(raw), w)]
                s = sum(x * (2 * e + 1) for e, x in enumerate(elems))
                total += (2 * (layer * H + g0 + g) + 1) * s
        res.append(total % (1 << 64))
    return res

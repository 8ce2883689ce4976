"""Seeded synthetic inputs: request lengths, block tables, KV pools, Mamba states.

Shared by the tests, the smoke check and the benchmark, on both sides of the
parity check.  It holds none of the checksum arithmetic: only shapes, random
contents and paging (which token lives in which slot of which block).

Metadata always comes from ``numpy.random.default_rng(seed)``.  Bulk contents
come from numpy on the host for small pools and from torch's device generator
for large ones; the oracle always reads the bytes the device holds, so
bit-exactness never depends on reproducing a random stream.

Shapes follow the vLLM paged pool of the page "[vLLM 源码解析] KV Cache"
(section "reshape kv_cache": K/V, num_blocks, block_size, num_kv_heads,
head_size; e.g. GPT-2's (2, 18545, 16, 12, 64) per layer).  Block ids of a
request are consecutive slices of a random permutation of the pool, so they
are distinct and non-contiguous, as that page's block-table example shows.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ELEM_BYTES = {"fp8": 1, "bf16": 2, "fp16": 2, "fp32": 4}
# host dtype that carries the raw bits of each element type
HOST_BITS = {"fp8": np.uint8, "bf16": np.uint16, "fp16": np.uint16, "fp32": np.uint32}


@dataclass
class Requests:
    """Block lists of a batch of requests (``KVChecksumBlocks`` per request)."""

    block_size: int
    num_tokens: np.ndarray      # int64 [R]
    start_pos: np.ndarray       # int64 [R]  position of the first listed block
    num_blocks: np.ndarray      # int32 [R]  listed positions
    block_table: np.ndarray     # int32 [R, max_blocks]; unlisted entries are -1

    @property
    def num_reqs(self) -> int:
        return int(self.num_tokens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def listed(self):
        """(r, k) of every listed position, request-major."""
        return [(r, k) for r in range(self.num_reqs) for k in range(int(self.num_blocks[r]))]


def uniform_lengths(rng: np.random.Generator, num_reqs: int, lo: int, hi: int) -> np.ndarray:
    """Inclusive uniform integer lengths."""
    return rng.integers(lo, hi + 1, size=num_reqs).astype(np.int64)


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks needed to hold ``num_tokens`` tokens from token 0."""
    return -(-int(num_tokens) // block_size)


def splitmix64_bytes(seed: int, nbytes: int) -> np.ndarray:
    """``nbytes`` bytes of the splitmix64 stream seeded with ``seed`` (the
    published generator of Steele, Lea and Flood: the state advances by
    0x9E3779B97F4A7C15 and each output is two xor-shift-multiply rounds of
    it), each 64-bit output giving 8 bytes little-endian.  Programs outside
    Python (the C example) draw the same bytes from their own copy."""
    n = (nbytes + 7) // 8
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + np.arange(1, n + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z.astype("<u8").view(np.uint8)[:nbytes]


def page_requests(rng: np.random.Generator, lengths, block_size: int, pool_blocks: int | None = None,
                  start_pos=None, extra_blocks=None, spare_frac: float = 0.05) -> tuple[Requests, int]:
    """Lay requests out on random, distinct, non-contiguous pool blocks.

    Request r lists the positions ``start_pos[r] .. blocks_for(N_r) - 1``
    (plus ``extra_blocks[r]`` positions past its last token, which hold no
    valid slot).  Returns the requests and the pool size used.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    R = lengths.shape[0]
    start = np.zeros(R, np.int64) if start_pos is None else np.asarray(start_pos, np.int64)
    extra = np.zeros(R, np.int64) if extra_blocks is None else np.asarray(extra_blocks, np.int64)
    nb = np.array([max(0, blocks_for(n, block_size) - s) + e
                   for n, s, e in zip(lengths, start, extra)], dtype=np.int32)
    total = int(nb.sum())
    if pool_blocks is None:
        pool_blocks = max(1, int(np.ceil(total * (1.0 + spare_frac))))
    if pool_blocks < total:
        raise ValueError(f"pool of {pool_blocks} blocks cannot hold {total} listed blocks")
    perm = rng.permutation(pool_blocks).astype(np.int32)
    max_blocks = max(1, int(nb.max()) if R else 1)
    table = np.full((R, max_blocks), -1, dtype=np.int32)
    off = 0
    for r in range(R):
        table[r, :nb[r]] = perm[off:off + nb[r]]
        off += int(nb[r])
    return Requests(block_size, lengths, start, nb, table), pool_blocks


def pool_shape(layout: str, num_blocks: int, block_size: int, num_heads: int, head_size: int):
    """Semantic shape of one layer's paged pool."""
    if layout == "NHD":
        return (2, num_blocks, block_size, num_heads, head_size)
    if layout == "HND":
        return (2, num_blocks, num_heads, block_size, head_size)
    if layout == "MLA":
        if num_heads != 1:
            raise ValueError("MLA pools hold one latent head")
        return (num_blocks, block_size, head_size)
    if layout == "FI_NHD":
        return (num_blocks, 2, block_size, num_heads, head_size)
    if layout == "FI_HND":
        return (num_blocks, 2, num_heads, block_size, head_size)
    raise ValueError(layout)


def host_random_bits(rng: np.random.Generator, shape, elem: str) -> np.ndarray:
    """Uniform random bit patterns carried in the unsigned dtype of ``elem``."""
    dt = HOST_BITS[elem]
    info = np.iinfo(dt)
    return rng.integers(0, int(info.max) + 1, size=shape, dtype=dt)


# ---------------------------------------------------------------- token paging

def token_locations(req: Requests, r: int):
    """(positions, slots) of tokens start_pos*bs .. N-1 of request r, as the
    listed positions hold them: token t sits at block position t // bs,
    slot t % bs."""
    bs = req.block_size
    t0 = int(req.start_pos[r]) * bs
    t = np.arange(t0, int(req.num_tokens[r]), dtype=np.int64)
    return t // bs - int(req.start_pos[r]), t % bs


def repage_numpy(src, src_layout: str, src_req: Requests, dst, dst_layout: str, dst_req: Requests):
    """Copy every request's tokens from one pool into another pool with a
    different block size and/or layout (same tokens, same heads)."""
    for r in range(src_req.num_reqs):
        ks, ss = token_locations(src_req, r)
        kd, sd = token_locations(dst_req, r)
        bsrc = src_req.block_table[r, ks]
        bdst = dst_req.block_table[r, kd]
        rows = _gather_rows(src, src_layout, bsrc, ss)
        _scatter_rows(dst, dst_layout, bdst, sd, rows)


def _gather_rows(pool, layout, blocks, slots):
    """Rows of tokens (blocks[t], slots[t]) as (planes, tokens, heads, D)."""
    if layout == "NHD":
        return pool[:, blocks, slots]
    if layout == "HND":
        # a slice between the two index arrays puts the token axis first
        planes = [pool[p][blocks, :, slots] for p in range(pool.shape[0])]
        if isinstance(pool, np.ndarray):
            return np.stack(planes, axis=0)
        import torch
        return torch.stack(planes, 0)
    return pool[blocks, slots][None, :, None, :]


def _scatter_rows(pool, layout, blocks, slots, rows):
    if layout == "NHD":
        pool[:, blocks, slots] = rows
    elif layout == "HND":
        for p in range(pool.shape[0]):
            pool[p][blocks, :, slots] = rows[p]
    else:
        pool[blocks, slots] = rows[0, :, 0, :]


def repage_torch(src, src_layout, src_req: Requests, dst, dst_layout, dst_req: Requests):
    """Device version of ``repage_numpy`` (torch tensors, same indexing)."""
    import torch
    dev = src.device
    for r in range(src_req.num_reqs):
        ks, ss = token_locations(src_req, r)
        kd, sd = token_locations(dst_req, r)
        bsrc = torch.from_numpy(src_req.block_table[r, ks].astype(np.int64)).to(dev)
        bdst = torch.from_numpy(dst_req.block_table[r, kd].astype(np.int64)).to(dev)
        ss_t = torch.from_numpy(ss).to(dev)
        sd_t = torch.from_numpy(sd).to(dev)
        rows = _gather_rows(src, src_layout, bsrc, ss_t)
        _scatter_rows(dst, dst_layout, bdst, sd_t, rows)


# ---------------------------------------------------------------- named workloads

@dataclass
class AttnWorkload:
    """One KV-cache group of paged attention layers."""

    name: str
    layout: str
    layer_numbers: list
    num_heads: int
    head_size: int
    elem: str
    values: str                       # "bits" (uniform bit patterns) or "normal"
    req: Requests
    pool_blocks: int
    seed: int
    head_begin: int = 0
    head_count: int | None = None
    global_head_base: list | None = None
    notes: dict = field(default_factory=dict)

    @property
    def num_layers(self) -> int:
        return len(self.layer_numbers)

    @property
    def heads_used(self) -> int:
        return self.num_heads - self.head_begin if self.head_count is None else self.head_count

    @property
    def planes(self) -> int:
        return 1 if self.layout == "MLA" else 2

    @property
    def shape(self):
        return pool_shape(self.layout, self.pool_blocks, self.req.block_size, self.num_heads, self.head_size)

    @property
    def bases(self):
        if self.global_head_base is not None:
            return list(self.global_head_base)
        return [self.head_begin] * self.num_layers

    def valid_tokens(self) -> int:
        """Tokens whose slots the listed positions hold (all layers alike)."""
        bs = self.req.block_size
        tot = 0
        for r in range(self.req.num_reqs):
            lo = int(self.req.start_pos[r]) * bs
            hi = min(int(self.req.num_tokens[r]), (int(self.req.start_pos[r]) + int(self.req.num_blocks[r])) * bs)
            tot += max(0, hi - lo)
        return tot

    def valid_bytes(self) -> int:
        """Cache bytes the checksum covers: valid tokens x layers x heads x planes x row."""
        return (self.valid_tokens() * self.num_layers * self.heads_used * self.planes
                * self.head_size * ELEM_BYTES[self.elem])

    def host_pools(self):
        """Seeded host pools (numpy), one per layer."""
        rng = np.random.default_rng(self.seed + 1000)
        if self.values != "bits":
            raise ValueError("host pools carry uniform random bits")
        return [host_random_bits(rng, self.shape, self.elem) for _ in self.layer_numbers]

    def device_pools(self, device="cuda"):
        """Seeded device pools (torch), one per layer."""
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(self.seed)
        pools = []
        for _ in self.layer_numbers:
            pools.append(device_fill(self.shape, self.elem, self.values, g, device))
        return pools


def device_fill(shape, elem, values, g, device):
    import torch
    if values == "normal":
        dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[elem]
        return torch.randn(shape, dtype=dt, device=device, generator=g)
    # uniform bits: fill the raw bytes
    dt = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[ELEM_BYTES[elem]]
    t = torch.empty(shape, dtype=dt, device=device)
    t.view(torch.uint8).random_(0, 256, generator=g)
    return t


def tiny(seed: int = 1) -> AttnWorkload:
    """2 layers x 2 KV heads, head 64 bf16, block 16, NHD pool of 16 blocks,
    one 50-token request on 4 shuffled block ids (last block partial)."""
    rng = np.random.default_rng(seed)
    req, nb = page_requests(rng, [50], 16, pool_blocks=16)
    return AttnWorkload("tiny", "NHD", [0, 1], 2, 64, "bf16", "bits", req, nb, seed)


def gpt2(seed: int = 2, num_reqs: int = 64, lo: int = 128, hi: int = 2048, layout="NHD",
         block_size: int = 16, pool_blocks: int | None = 18545, layers: int = 12, elem="fp16") -> AttnWorkload:
    """GPT-2-shaped: 12 layers x 12 KV heads, head 64, fp16 bits, block 16,
    pool (2, 18545, 16, 12, 64) per layer, 64 requests of 128..2048 tokens."""
    rng = np.random.default_rng(seed)
    lengths = uniform_lengths(rng, num_reqs, lo, hi)
    req, nb = page_requests(rng, lengths, block_size, pool_blocks=pool_blocks)
    return AttnWorkload("gpt2", layout, list(range(layers)), 12, 64, elem, "bits", req, nb, seed)


def llama3_8b(seed: int = 3, num_reqs: int = 256, lo: int = 512, hi: int = 8192, layers: int = 32,
              head_begin: int = 0, head_count: int | None = None, global_base: int | None = None) -> AttnWorkload:
    """Llama-3-8B-shaped: 32 layers x 8 KV heads, head 128, bf16 normal(0,1),
    block 16, HND pool with 5 % spare blocks, 256 requests of 512..8192 tokens.
    ``head_begin/head_count/global_base`` select a TP shard over heads."""
    rng = np.random.default_rng(seed)
    lengths = uniform_lengths(rng, num_reqs, lo, hi)
    req, nb = page_requests(rng, lengths, 16, spare_frac=0.05)
    base = head_begin if global_base is None else global_base
    return AttnWorkload("llama3_8b", "HND", list(range(layers)), 8, 128, "bf16", "normal", req, nb, seed,
                        head_begin=head_begin, head_count=head_count,
                        global_head_base=[base] * layers)


def mla(seed: int = 4, num_reqs: int = 64, lo: int = 128, hi: int = 2048, block_size: int = 64,
        layers: int = 61) -> AttnWorkload:
    """MLA-style: 61 layers x 1 latent head of 576 bf16 dims."""
    rng = np.random.default_rng(seed)
    lengths = uniform_lengths(rng, num_reqs, lo, hi)
    req, nb = page_requests(rng, lengths, block_size)
    return AttnWorkload("mla", "MLA", list(range(layers)), 1, 576, "bf16", "bits", req, nb, seed)


@dataclass
class MambaWorkload:
    """A KV-cache group of Mamba layers: running states, one slot per request."""

    name: str
    layer_numbers: list
    state_shapes: list          # per state: (rows, ...) without the slot dim
    state_elems: list           # per state: element type name
    slots: int
    slot_ids: np.ndarray        # int32 [R]
    seed: int
    row_begin: int = 0
    row_count: int | None = None
    global_row_base: list | None = None

    @property
    def rows(self) -> int:
        return self.state_shapes[0][0]

    @property
    def rows_used(self) -> int:
        return self.rows - self.row_begin if self.row_count is None else self.row_count

    @property
    def bases(self):
        if self.global_row_base is not None:
            return list(self.global_row_base)
        return [self.row_begin] * len(self.layer_numbers)

    def row_bytes(self) -> int:
        tot = 0
        for shp, el in zip(self.state_shapes, self.state_elems):
            tot += int(np.prod(shp[1:])) * ELEM_BYTES[el]
        return tot

    def valid_bytes(self) -> int:
        return len(self.slot_ids) * len(self.layer_numbers) * self.rows_used * self.row_bytes()

    def host_states(self):
        rng = np.random.default_rng(self.seed + 1000)
        return [[host_random_bits(rng, (self.slots,) + tuple(shp), el)
                 for shp, el in zip(self.state_shapes, self.state_elems)] for _ in self.layer_numbers]

    def device_states(self, device="cuda"):
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(self.seed)
        return [[device_fill((self.slots,) + tuple(shp), el, "normal", g, device)
                 for shp, el in zip(self.state_shapes, self.state_elems)] for _ in self.layer_numbers]


def hybrid(seed: int = 5, num_reqs: int = 128, lo: int = 512, hi: int = 8192, attn_layers: int = 24,
           slots: int = 160, rows: int = 64):
    """24 attention layers (8 KV heads, head 128, bf16, block 16, HND) at layer
    numbers 0, 2, .., 46, interleaved with 24 Mamba layers at 1, 3, .., 47
    holding an fp32 SSM state [rows x 128 x 16] and an fp16 conv state
    [rows x 4 x 256]; each request owns one random state slot."""
    rng = np.random.default_rng(seed)
    lengths = uniform_lengths(rng, num_reqs, lo, hi)
    req, nb = page_requests(rng, lengths, 16, spare_frac=0.05)
    attn = AttnWorkload("hybrid_attn", "HND", [2 * i for i in range(attn_layers)], 8, 128, "bf16", "normal",
                        req, nb, seed)
    slot_ids = rng.permutation(slots)[:num_reqs].astype(np.int32)
    mamba = MambaWorkload("hybrid_mamba", [2 * i + 1 for i in range(attn_layers)],
                          [(rows, 128, 16), (rows, 4, 256)], ["fp32", "fp16"], slots, slot_ids, seed + 7)
    return attn, mamba

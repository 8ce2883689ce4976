// Paged K/V block checksums on gfx950.
//
// Definition (vLLM API page "vllm.distributed.kv_transfer.kv_checksum.checksum",
// module docstring items 1 and 2):
//   s(layer, head) = sum_j x_j (2j + 1),  j = t*P + p,  x_j little-endian uint64
//   c(position)    = sum_{layer, head} m s,  m = 2 (layer*65536 + global_head) + 1
// all mod 2^64.
//
// Up to three launches per call, all on the caller's stream:
//   plan    request arrays -> compact list of listed positions (PosRecord):
//           block id, first token t0 = pos*block_size, valid slots v (the
//           block's slots whose token lies below num_tokens, as the page's
//           helper num_valid_tokens counts them), output index.  Bad ids and
//           requests are flagged.
//           Small calls skip it: their main pass (the DENSE variants) derives
//           each task's record from the request arrays with the same rules.
//   blocks  one wavefront per task (group of caches, position): streams the
//           valid rows of the block's pages with 16-byte loads and accumulates
//           sum over pieces of x * m * (2j + 1) in 64-bit registers, then
//           reduces the 64 lanes and writes one uint64 per task.
//   reduce  sums the per-group partials of each position in a fixed order
//           (skipped when the call has one group).  Addition mod 2^64 is
//           associative and commutative, so results are bit-exact whatever
//           the task order or launch shape.
#include <atomic>
#include <map>
#include <mutex>

#include "kvck_device.h"

namespace kvck {
namespace {

// ----------------------------------------------------------------- plan

// Exclusive prefix sum of the listed positions per request (one workgroup).
__global__ __launch_bounds__(1024) void plan_scan_kernel(const int32_t* __restrict__ nbpr,
                                                         const int64_t* __restrict__ start_pos,
                                                         int32_t num_reqs, int32_t max_blocks,
                                                         int64_t max_start, int32_t* __restrict__ prefix,
                                                         uint32_t* __restrict__ n_items,
                                                         uint32_t* __restrict__ error_flags) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < num_reqs; base += 1024) {
    const int r = base + tid;
    int n = 0;
    if (r < num_reqs) {
      n = nbpr[r];
      if (bad_request(n, start_pos[r], max_blocks, max_start)) {
        if (error_flags) atomicOr(error_flags, KVCK_FLAG_BAD_REQUEST);
        n = 0;
      }
    }
    buf[tid] = n;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int t = tid >= o ? buf[tid - o] : 0;
      __syncthreads();
      buf[tid] += t;
      __syncthreads();
    }
    const int incl = buf[tid];
    const int c = carry;
    if (r < num_reqs) prefix[r] = c + incl - n;
    __syncthreads();
    if (tid == 1023) carry = c + incl;
    __syncthreads();
  }
  if (tid == 0) {
    prefix[num_reqs] = carry;
    *n_items = (uint32_t)carry;
  }
}

// One thread per (request, listed position): the position's record.
__global__ __launch_bounds__(256) void plan_fill_kernel(
    const int32_t* __restrict__ block_table, int64_t bt_stride, const int64_t* __restrict__ start_pos,
    const int64_t* __restrict__ num_tokens, int32_t num_reqs, int32_t max_blocks, int32_t block_size,
    int64_t num_blocks, int64_t out_stride, const int32_t* __restrict__ prefix, PosRecord* __restrict__ recs,
    uint32_t* __restrict__ error_flags) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_reqs * max_blocks) return;
  const int32_t r = (int32_t)(idx / max_blocks);
  const int32_t k = (int32_t)(idx - (int64_t)r * max_blocks);
  const int32_t p0 = prefix[r];
  if (k >= prefix[r + 1] - p0) return;
  const int64_t t0 = (start_pos[r] + k) * (int64_t)block_size;
  int32_t v = valid_slots(num_tokens[r], t0, block_size);
  const int32_t b = block_table[(int64_t)r * bt_stride + k];
  if (v > 0 && (b < 0 || (int64_t)b >= num_blocks)) {
    if (error_flags) atomicOr(error_flags, KVCK_FLAG_BAD_BLOCK_ID);
    v = 0;
  }
  PosRecord rec;
  rec.t0 = t0;
  rec.out_idx = idx * out_stride;
  rec.block = b;
  rec.valid = v;
  rec.pad = 0;
  recs[p0 + k] = rec;
}

// Both plan steps in one launch, for batches of at most 1024 requests: every
// workgroup loads the clamped per-request counts into LDS and scans them
// itself, then writes the records of its 256 (request, position) slots.
__global__ __launch_bounds__(1024) void plan_small_kernel(
    const int32_t* __restrict__ block_table, int64_t bt_stride, const int32_t* __restrict__ nbpr,
    const int64_t* __restrict__ start_pos, const int64_t* __restrict__ num_tokens, int32_t num_reqs,
    int32_t max_blocks, int32_t block_size, int64_t num_blocks, int64_t max_start, int64_t out_stride,
    uint32_t* __restrict__ n_items, PosRecord* __restrict__ recs, uint32_t* __restrict__ error_flags) {
  __shared__ int32_t scan[1024];
  const int tid = threadIdx.x;
  int n = 0;
  if (tid < num_reqs) {
    n = nbpr[tid];
    if (bad_request(n, start_pos[tid], max_blocks, max_start)) {
      if (blockIdx.x == 0 && error_flags) atomicOr(error_flags, KVCK_FLAG_BAD_REQUEST);
      n = 0;
    }
  }
  scan[tid] = n;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int t = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += t;
    __syncthreads();
  }
  if (blockIdx.x == 0 && tid == 0) *n_items = (uint32_t)scan[1023];
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + tid;
  if (idx >= (int64_t)num_reqs * max_blocks) return;
  const int32_t r = (int32_t)(idx / max_blocks);
  const int32_t k = (int32_t)(idx - (int64_t)r * max_blocks);
  const int32_t end = scan[r];
  const int32_t p0 = r > 0 ? scan[r - 1] : 0;
  if (k >= end - p0) return;
  const int64_t t0 = (start_pos[r] + k) * (int64_t)block_size;
  int32_t v = valid_slots(num_tokens[r], t0, block_size);
  const int32_t b = block_table[(int64_t)r * bt_stride + k];
  if (v > 0 && (b < 0 || (int64_t)b >= num_blocks)) {
    if (error_flags) atomicOr(error_flags, KVCK_FLAG_BAD_BLOCK_ID);
    v = 0;
  }
  PosRecord rec;
  rec.t0 = t0;
  rec.out_idx = idx * out_stride;
  rec.block = b;
  rec.valid = v;
  rec.pad = 0;
  recs[p0 + k] = rec;
}

// ----------------------------------------------------------------- main pass
//
// Task = (group of `caches_per_task` caches, listed position), one wavefront
// each; waves stride over the tasks group-major, so the waves resident at any
// time read a few layers' pools.  A task's result is one uint64 (a partial
// over its caches), reduced by the second pass unless the call has one group.
//
// Lane table: a row group is up to `rows_per_group` consecutive slots of one
// (plane, head); its rows hold rows_per_group*chunks_per_row chunks of CHUNK
// bytes, and lane l owns chunks l, l+64, .., l+64(S-1): slot row[s], byte
// offset off[s] inside the group, and piece term urel[s] = 2*(row*P + q),
// q the chunk's first piece inside its plane row.  The same table serves every
// plane, head, cache and position, so the inner loop only adds offsets.
//
// A unit is the loads of one (cache, row group, PU planes, batch of HU heads):
// PU*HU*S chunks per lane (PU = 2 lets a unit carry K and V when a call has
// too few heads to fill HU).  For a chunk of pieces xa (piece q) and xb (piece q+1)
// of token t, plane pl, head h:
//   xa*m*u + xb*m*(u + 2) = m*((xa + xb)*u + 2*xb),  u = 2(tP + q) + 1,
// u per lane and plane, m uniform per head.
//
// PIPE = false: each unit's loads are issued, then consumed.
// PIPE = true:  two unit buffers in ping-pong, so the loads of unit i+1 are in
//               flight while unit i is consumed, across the caches of a task
//               (for planned merged rows also across the wave's tasks).
// MERGED:       pools whose heads sit side by side in a slot (NHD-like): a
//               lane-table row is the slot's whole run of heads, so a load
//               instruction covers contiguous bytes even when one head's row
//               is short; each chunk carries its own head's factor m.
// DENSE:        a call planned in place: tasks index every (request, block
//               slot) and each wave runs exactly one task (the grid covers them
//               all), so no request pointer stays live across the unit loop.
// Weighted sum of one unit's chunks: x[p][h][s] is chunk s (lane-table entry)
// of plane step p and head h0 + h of a row group whose first piece term is
// up0 (2(t*P + plane piece offset) + 1 for the group's first token t);
// chunk pieces xa, xb contribute m((xa + xb)u + 2xb) with u = up0 + urel[s].
template <int CHUNK, int S, int HU, int PU, bool MERGED>
__device__ __forceinline__ uint64_t unit_sum(const typename ChunkType<CHUNK>::T (&x)[PU][HU][S],
                                             const LaneTable<S>& lt, const uint32_t (&lhead)[S], uint64_t up0,
                                             uint64_t plane_term, uint64_t mb, int h0) {
  uint64_t acc = 0;
#pragma unroll
  for (int p = 0; p < PU; ++p) {
    const uint64_t up = up0 + (uint64_t)p * plane_term;
#pragma unroll
    for (int h = 0; h < HU; ++h) {
      // sh: sum of the unit's terms; sl (merged rows): the same weighted by
      // each chunk's local head, so that sum_s t_s (mb + 2 head_s) costs one
      // 64-bit multiply per unit: mb * sh + 2 sl
      uint64_t sh = 0, sl = 0;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint64_t u = up + lt.urel[s];
        const uint64_t xa = (uint64_t)x[p][h][s].x | ((uint64_t)x[p][h][s].y << 32);
        uint64_t t;
        if constexpr (CHUNK == 16) {
          const uint64_t xb = (uint64_t)x[p][h][s].z | ((uint64_t)x[p][h][s].w << 32);
          t = (xa + xb) * u + (xb << 1);
        } else {
          t = xa * u;
        }
        sh += t;
        if constexpr (MERGED) sl += t * (uint64_t)lhead[s];
      }
      if constexpr (MERGED)
        acc += sh * mb + (sl << 1);
      else
        acc += sh * (mb + 2ull * (uint64_t)(h0 + h));
    }
  }
  return acc;
}

// What the consuming side needs of an issued unit (all uniform).
struct UnitDesc {
  uint64_t t0;       // first token of the unit's block
  int64_t out_idx;   // the task's output entry (direct writes)
  int64_t task;      // the task (its group and listed position)
  int cache, group, plane, hbatch;
  bool live;         // a real unit (else every load was out of range)
  bool last;         // the task's last unit: reduce and write after it
};

template <int CHUNK, int S, int HU, int PU, bool PIPE, bool MERGED, bool DENSE>
__global__ __launch_bounds__(kBlockThreads) void blocks_kernel(const BlocksArgs a) {
  using V = typename ChunkType<CHUNK>::T;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = wave_index();
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n_items = DENSE ? a.max_items : (int64_t)read_const(a.n_items);
  const int lpt = a.caches_per_task;
  const int ngroups = (a.num_caches + lpt - 1) / lpt;
  const int64_t total = n_items * ngroups;
  if (wave >= total) return;

  LaneTable<S> lt;
  lt.template init<CHUNK>(lane, a);
  uint32_t lhead[S];  // local head of each lane chunk (merged rows only)
  if constexpr (MERGED) lt.heads(lane, a, lhead);
  const uint64_t P = (uint64_t)a.pieces;
  const int rg = a.rows_per_group;
  const uint64_t plane_term = 2ull * (P / (uint64_t)a.planes_total);
  const int nhb = (a.heads + HU - 1) / HU;

  if constexpr (PIPE && !DENSE && MERGED) {
    // Planned, pipelined, merged rows: the wave's tasks (wave, wave + nwaves,
    // ...) form one stream of units.  The issue side runs one unit ahead of
    // the consuming side -- also into the next task -- so loads stay in
    // flight across task boundaries: a task's reduction, its write and the
    // next task's record are taken while the other buffer's loads are under
    // way.  Merged rows (short rows, single latent heads) have few units
    // per task and gain from it (same-box A/B: fp8 64-byte rows +0.8-0.9
    // points of 8 TB/s, MLA +0.4-0.8); pools of separate head rows, whose
    // tasks are long, ran 0.1-1.1 points slower with it and keep one task at
    // a time.
    const int nplanes = a.planes / PU;  // plane steps per row group (PU divides planes)
    int64_t i_task = wave;              // task of the next unit to issue
    int i_left = 0;                     // its units still to issue (0: read its record first)
    int i_ngr = 1;
    int32_t i_v = 0;
    uint64_t i_t0 = 0;
    int64_t i_boff = 0, i_out = 0;
    UnitCursor ic{0, 0, 0, 0};
    // Issue the stream's next unit into x, described by d; past the stream's
    // end every load is out of range (zeros, no memory touched).
    auto issue = [&](V(&x)[PU][HU][S], UnitDesc& d) {
      if (i_left == 0 && i_task < total) {
        const int64_t grp = i_task / n_items;
        const TaskRecord rec = task_record<false>(a, i_task - grp * n_items, false, lane);
        const int c_begin = (int)grp * lpt;
        const int c_end = min(a.num_caches, c_begin + lpt);
        i_v = rec.valid;
        i_t0 = rec.t0;
        i_out = rec.out_idx;
        i_boff = (int64_t)rec.block * a.block_stride;
        i_ngr = max(1, (i_v + rg - 1) / rg);
        // a position with no valid slot still gets one (empty) unit, so its
        // zero is written like any other task's result
        i_left = i_v > 0 ? i_ngr * nplanes * nhb * (c_end - c_begin) : 1;
        ic = UnitCursor{c_begin, 0, 0, 0};
      }
      const bool live = i_task < total;
      const int rows = live ? min(rg, i_v - ic.group * rg) : 0;
      // uniform by construction; taken through readfirstlane because the
      // compiler cannot prove it across the stream's loop, and a descriptor
      // it believes divergent costs a per-lane loop around every load
      const uint8_t* base = reinterpret_cast<const uint8_t*>(
          uniform64(reinterpret_cast<int64_t>(a.base[live ? ic.cache : 0] + i_boff +
                                              (int64_t)(ic.group * rg) * a.slot_stride +
                                              (int64_t)(ic.plane * PU) * a.plane_stride)));
      uint32_t voff[S];
#pragma unroll
      for (int s = 0; s < S; ++s) voff[s] = lt.row[s] < rows ? lt.off[s] : kOOB;
#pragma unroll
      for (int p = 0; p < PU; ++p) {
#pragma unroll
        for (int h = 0; h < HU; ++h) {
          const int hh = ic.hbatch * HU + h;
          const uint32_t hmask = hh < a.heads ? 0u : kOOB;
          const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)p * a.plane_stride + (int64_t)hh * a.head_stride);
#pragma unroll
          for (int s = 0; s < S; ++s) x[p][h][s] = load_chunk<CHUNK>(rs, voff[s] | hmask);
        }
      }
      d.t0 = i_t0;
      d.out_idx = i_out;
      d.task = i_task;
      d.cache = live ? ic.cache : 0;  // a dead unit is consumed too: keep its factor index in range
      d.group = ic.group;
      d.plane = ic.plane;
      d.hbatch = ic.hbatch;
      d.live = live;
      d.last = live && i_left == 1;
      if (live) {
        // a plane's row groups back to back (same-box A/B, twenty interleaved
        // rounds: fp8 64-byte rows +0.5 points of 8 TB/s at blocks 16 and 64;
        // MLA, one plane, unchanged)
        ic.next_group_first(nhb, nplanes, i_ngr);
        if (--i_left == 0) i_task += nwaves;
      }
    };
    uint64_t acc = 0;
    // Consume a live unit; after a task's last unit, reduce and write.
    // Returns the unit's own sum, which depends on every chunk of x.
    auto consume = [&](const V(&x)[PU][HU][S], const UnitDesc& d) {
      const uint64_t up0 = 2ull * (d.t0 + (uint64_t)(d.group * rg)) * P + 1ull + a.piece_base +
                           (uint64_t)(d.plane * PU) * plane_term;
      const uint64_t us = unit_sum<CHUNK, S, HU, PU, MERGED>(x, lt, lhead, up0, plane_term, a.mbase[d.cache],
                                                             d.hbatch * HU);
      acc += us;
      if (d.last) {
        const uint64_t tot = wave_sum(acc);
        acc = 0;
        if (lane == 0) {
          if (a.direct) {
            // the entry is this task's alone: read it with a scalar load,
            // whose wait does not also wait for the unit loads in flight
            uint64_t* o = a.out + d.out_idx;
            *o = a.accumulate ? read_const(o) + tot : tot;
          } else {
            const int64_t grp = d.task / n_items;
            a.partials[(int64_t)(a.group_offset + grp) * a.max_items + (d.task - grp * n_items)] = tot;
          }
        }
      }
      return us;
    };
    // Both buffers are issued and consumed at every step (past the stream's
    // end with every load out of range; such a unit's data are zeros, so its
    // sum is 0 and, not being a task's last unit, it writes nothing), and the
    // loop has a single exit, so the compiler's waits follow the buffers: the
    // wait before consuming B leaves A's loads in flight.  B's loads, though,
    // are issued only once A's have landed (wait_vector_memory), so a wave
    // has one or two units in flight, not always two.  These short-row pools
    // read faster that way: same-box A/B, twelve interleaved rounds, against
    // two units always in flight: fp8 64-byte rows at blocks 16 / 64 +0.8 /
    // +0.5 points of 8 TB/s, MLA at blocks 16 / 64 +1.8 / +0.2.  order_after
    // keeps a buffer's next loads after the last use of its data, so each
    // buffer keeps its registers.
    V A[PU][HU][S], B[PU][HU][S];
    UnitDesc da, db;
    issue(A, da);  // live: the wave has at least one task
    do {
      wait_vector_memory();
      issue(B, db);
      order_after(consume(A, da));
      issue(A, da);
      order_after(consume(B, db));
    } while (da.live);  // uniform; once A is past the end, so is every later unit
    return;
  }

  for (int64_t task = wave; task < total; task += nwaves) {
    const int64_t grp = task / n_items;
    const int64_t item = task - grp * n_items;
    const int c_begin = (int)grp * lpt;
    const int c_end = min(a.num_caches, c_begin + lpt);
    const TaskRecord rec = task_record<DENSE>(a, item, a.group_offset + grp == 0, lane);
    // Dense variants run one task per wave (their grid covers every task), so
    // they leave the loop after it; only their slots can be unlisted.
    if (!rec.listed) break;  // uniform
    const int32_t v = rec.valid;
    const int32_t blk = rec.block;
    const uint64_t t0 = rec.t0;
    uint64_t acc = 0;
    if (v > 0) {
      const int64_t blk_off = (int64_t)blk * a.block_stride;
      const int ngr = (v + rg - 1) / rg;
      const int nplanes = a.planes / PU;  // plane steps per row group (PU divides planes)
      const int nunits = ngr * nplanes * nhb * (c_end - c_begin);
      UnitCursor ic{c_begin, 0, 0, 0}, cc{c_begin, 0, 0, 0};

      // `live` false: a unit past the task's last one, every load out of range
      auto issue = [&](V(&x)[PU][HU][S], bool live) {
        const int rows = live ? min(rg, v - ic.group * rg) : 0;
        const uint8_t* base = a.base[live ? ic.cache : c_begin] + blk_off + (int64_t)(ic.group * rg) * a.slot_stride +
                              (int64_t)(ic.plane * PU) * a.plane_stride;
        uint32_t voff[S];
#pragma unroll
        for (int s = 0; s < S; ++s) voff[s] = lt.row[s] < rows ? lt.off[s] : kOOB;
#pragma unroll
        for (int p = 0; p < PU; ++p) {
#pragma unroll
          for (int h = 0; h < HU; ++h) {
            const int hh = ic.hbatch * HU + h;
            const uint32_t hmask = hh < a.heads ? 0u : kOOB;
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(base + (int64_t)p * a.plane_stride + (int64_t)hh * a.head_stride);
#pragma unroll
            for (int s = 0; s < S; ++s) x[p][h][s] = load_chunk<CHUNK>(rs, voff[s] | hmask);
          }
        }
        if (live) ic.next(nhb, nplanes, ngr);
      };
      auto consume = [&](const V(&x)[PU][HU][S]) {
        const uint64_t up0 = 2ull * (t0 + (uint64_t)(cc.group * rg)) * P + 1ull + a.piece_base +
                             (uint64_t)(cc.plane * PU) * plane_term;
        acc += unit_sum<CHUNK, S, HU, PU, MERGED>(x, lt, lhead, up0, plane_term, a.mbase[cc.cache], cc.hbatch * HU);
        cc.next(nhb, nplanes, ngr);
      };

      if constexpr (PIPE) {
        // Both buffers are issued at every step, past the task's last unit
        // with every load out of range (zeros, no memory touched): with no
        // branch around an issue, the waits before consuming one buffer count
        // the other buffer's loads as still to come, and leave them in flight.
        // order_after keeps a buffer's next loads after the last use of its
        // data, so each buffer keeps its registers across steps.
        V A[PU][HU][S], B[PU][HU][S];
        issue(A, true);
        for (int ui = 0; ui < nunits; ui += 2) {
          issue(B, ui + 1 < nunits);
          consume(A);
          order_after(acc);
          issue(A, ui + 2 < nunits);
          if (ui + 1 < nunits) consume(B);
          order_after(acc);
        }
      } else {
        for (int ui = 0; ui < nunits; ++ui) {
          V A[PU][HU][S];
          issue(A, true);
          consume(A);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      if (a.direct) {
        uint64_t* o = a.out + rec.out_idx;
        *o = a.accumulate ? *o + acc : acc;
      } else {
        a.partials[(int64_t)(a.group_offset + grp) * a.max_items + item] = acc;
      }
    }
    if constexpr (DENSE) break;
  }
}

// ----------------------------------------------------------------- second pass

__global__ __launch_bounds__(256) void reduce_kernel(const uint64_t* __restrict__ partials, int64_t stride,
                                                     int32_t splits, const uint32_t* __restrict__ n_items,
                                                     int64_t n_fixed, const PosRecord* __restrict__ recs,
                                                     uint64_t* __restrict__ out, int64_t out_stride,
                                                     int32_t accumulate) {
  const int64_t n = n_items ? (int64_t)*n_items : n_fixed;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint64_t s = 0;
    for (int32_t sp = 0; sp < splits; ++sp) s += partials[(int64_t)sp * stride + i];
    const int64_t o = recs ? recs[i].out_idx : i * out_stride;
    out[o] = accumulate ? out[o] + s : s;
  }
}

// Same sum, one wavefront per output: lanes stride over the partials, then
// the wave reduces.  Used when each output has many partials.
__global__ __launch_bounds__(256) void reduce_wave_kernel(const uint64_t* __restrict__ partials, int64_t stride,
                                                          int32_t splits, const uint32_t* __restrict__ n_items,
                                                          int64_t n_fixed, const PosRecord* __restrict__ recs,
                                                          uint64_t* __restrict__ out, int64_t out_stride,
                                                          int32_t accumulate) {
  const int64_t n = n_items ? (int64_t)*n_items : n_fixed;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t i = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; i < n; i += waves) {
    uint64_t s = 0;
    for (int32_t sp = lane; sp < splits; sp += kWave) s += partials[(int64_t)sp * stride + i];
    s = wave_sum(s);
    if (lane == 0) {
      const int64_t o = recs ? recs[i].out_idx : i * out_stride;
      out[o] = accumulate ? out[o] + s : s;
    }
  }
}

// Second pass of a call planned in place: one wavefront per (r, k) slot, the
// partials of listed positions summed in split order (lanes stride over the
// splits); other slots are left untouched.
__global__ __launch_bounds__(256) void reduce_dense_kernel(const uint64_t* __restrict__ partials, int64_t stride,
                                                           int32_t splits, const int32_t* __restrict__ nbpr,
                                                           const int64_t* __restrict__ start_pos, int32_t max_blocks,
                                                           int64_t max_start, uint64_t* __restrict__ out,
                                                           int64_t out_stride, int32_t accumulate) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t i = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; i < stride; i += waves) {
    const int32_t r = (int32_t)i / max_blocks;  // stride = num_reqs * max_blocks < 2^31
    const int32_t k = (int32_t)i - r * max_blocks;
    const int32_t n = nbpr[r];
    if (bad_request(n, start_pos[r], max_blocks, max_start) || k >= n) continue;
    uint64_t s = 0;
    for (int32_t sp = lane; sp < splits; sp += kWave) s += partials[(int64_t)sp * stride + i];
    s = wave_sum(s);
    if (lane == 0) {
      uint64_t* o = out + i * out_stride;
      *o = accumulate ? *o + s : s;
    }
  }
}

template <int CHUNK, int S, int PU, bool PIPE, bool MERGED, bool DENSE>
constexpr auto pick_kernel() {
  constexpr int hu = MERGED ? 1 : (16 / (S * PU) > 0 ? 16 / (S * PU) : 1);
  return &blocks_kernel<CHUNK, S, hu, PU, PIPE, MERGED, DENSE>;
}

using BlocksFn = void (*)(const BlocksArgs);

template <int CHUNK, int PU, bool PIPE, bool MERGED, bool DENSE>
BlocksFn blocks_fn_slots(int slots) {
  switch (slots) {
    case 1: return pick_kernel<CHUNK, 1, PU, PIPE, MERGED, DENSE>();
    case 2: return pick_kernel<CHUNK, 2, PU, PIPE, MERGED, DENSE>();
    case 4: return pick_kernel<CHUNK, 4, PU, PIPE, MERGED, DENSE>();
    case 8: return pick_kernel<CHUNK, 8, 1, PIPE, MERGED, DENSE>();
    case 16: return pick_kernel<CHUNK, 16, 1, PIPE, MERGED, DENSE>();
  }
  return nullptr;
}

template <bool DENSE>
BlocksFn blocks_fn_plan(const BlocksShape& shp) {
  if (shp.merged) {
    if (shp.pipelined)  // lane tables of at most 8 slots (the host's rule)
      return shp.slots > 8 ? nullptr
                           : (shp.chunk == 16 ? blocks_fn_slots<16, 1, true, true, DENSE>(shp.slots)
                                              : blocks_fn_slots<8, 1, true, true, DENSE>(shp.slots));
    return shp.chunk == 16 ? blocks_fn_slots<16, 1, false, true, DENSE>(shp.slots)
                           : blocks_fn_slots<8, 1, false, true, DENSE>(shp.slots);
  }
  if (shp.pipelined) {
    if (shp.planes_per_unit == 2)
      return shp.chunk == 16 ? blocks_fn_slots<16, 2, true, false, DENSE>(shp.slots)
                             : blocks_fn_slots<8, 2, true, false, DENSE>(shp.slots);
    return shp.chunk == 16 ? blocks_fn_slots<16, 1, true, false, DENSE>(shp.slots)
                           : blocks_fn_slots<8, 1, true, false, DENSE>(shp.slots);
  }
  return shp.chunk == 16 ? blocks_fn_slots<16, 1, false, false, DENSE>(shp.slots)
                         : blocks_fn_slots<8, 1, false, false, DENSE>(shp.slots);
}

// Pipelined units may carry both planes (PU = 2); the unpipelined kernel and
// wide lane tables (S >= 8) always take one plane per unit.  Merged rows take
// one plane per unit and pipeline with lane tables of up to 8 slots.  Every
// variant exists planned and planned in place.
BlocksFn blocks_fn(const BlocksShape& shp) {
  return shp.dense ? blocks_fn_plan<true>(shp) : blocks_fn_plan<false>(shp);
}

}  // namespace

int device_cus(int device) {
  static std::atomic<int> cached[64];
  if (device >= 0 && device < 64) {
    const int c = cached[device].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
    cus = 256;
  if (device >= 0 && device < 64) cached[device].store(cus, std::memory_order_relaxed);
  return cus;
}

int kernel_occupancy(const void* fn, int device, int fallback) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find({fn, device});
    if (it != cache.end()) return it->second;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kBlockThreads, 0) != hipSuccess || per_cu <= 0)
    per_cu = fallback;
  std::lock_guard<std::mutex> g(mu);
  cache[{fn, device}] = per_cu;
  return per_cu;
}

// Workgroups per CU a launch uses: `preferred`, at most what fits, or
// KVCK_GRID_PER_CU=n where set (an A/B switch; results are identical).
int workgroups_per_cu(int fits, int preferred) {
  int n = preferred < fits ? preferred : fits;
  if (const char* e = getenv("KVCK_GRID_PER_CU")) {
    const int f = atoi(e);
    if (f >= 1) n = f < fits ? f : fits;
  }
  return n < 1 ? 1 : n;
}

hipError_t launch_plan(const int32_t* block_table, int64_t bt_stride, const int32_t* nbpr,
                       const int64_t* start_pos, const int64_t* num_tokens, int32_t num_reqs,
                       int32_t max_blocks, int32_t block_size, int64_t num_blocks, int64_t out_stride,
                       void* workspace, uint32_t* error_flags, hipStream_t stream) {
  const BlocksWorkspace w = BlocksWorkspace::make(1, num_reqs, max_blocks);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* n_items = reinterpret_cast<uint32_t*>(ws);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + w.prefix_off);
  PosRecord* recs = reinterpret_cast<PosRecord*>(ws + w.recs_off);
  const int64_t max_start = INT64_MAX / block_size - max_blocks;
  const int64_t items = (int64_t)num_reqs * max_blocks;
  if (num_reqs <= 1024) {
    hipLaunchKernelGGL(plan_small_kernel, dim3((unsigned)((items + 1023) / 1024)), dim3(1024), 0, stream,
                       block_table, bt_stride, nbpr, start_pos, num_tokens, num_reqs, max_blocks, block_size,
                       num_blocks, max_start, out_stride, n_items, recs, error_flags);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, nbpr, start_pos, num_reqs, max_blocks,
                     max_start, prefix, n_items, error_flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t grid = (items + 255) / 256;
  hipLaunchKernelGGL(plan_fill_kernel, dim3((unsigned)grid), dim3(256), 0, stream, block_table, bt_stride,
                     start_pos, num_tokens, num_reqs, max_blocks, block_size, num_blocks, out_stride, prefix, recs,
                     error_flags);
  return hipGetLastError();
}

int blocks_grid(const BlocksShape& shp, int device, int64_t max_tasks) {
  BlocksFn fn = blocks_fn(shp);
  const int fits = kernel_occupancy(reinterpret_cast<const void*>(fn), device, 2);
  const int per_cu = workgroups_per_cu(fits, kMainWorkgroupsPerCU);
  const int64_t waves_per_block = kBlockThreads / kWave;
  const int64_t need = (max_tasks + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)per_cu * device_cus(device);
  if (shp.dense) return (int)(need > 0 ? need : 1);  // one task per wave (at most kDenseMaxTasks)
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

hipError_t launch_blocks(const BlocksArgs& a, const BlocksShape& shp, int grid, hipStream_t stream) {
  BlocksFn fn = blocks_fn(shp);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<BlocksArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(kBlockThreads), args, 0, stream);
}

hipError_t launch_reduce(const uint64_t* partials, int64_t stride, int32_t splits, const uint32_t* n_items,
                         int64_t n_fixed, const PosRecord* recs, uint64_t* out, int64_t out_stride,
                         int32_t accumulate, hipStream_t stream) {
  if (splits >= 64) {
    int64_t grid = (stride + 3) / 4;
    if (grid > 4096) grid = 4096;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(reduce_wave_kernel, dim3((unsigned)grid), dim3(256), 0, stream, partials, stride, splits,
                       n_items, n_fixed, recs, out, out_stride, accumulate);
    return hipGetLastError();
  }
  int64_t grid = (stride + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)grid), dim3(256), 0, stream, partials, stride, splits, n_items,
                     n_fixed, recs, out, out_stride, accumulate);
  return hipGetLastError();
}

hipError_t launch_reduce_dense(const uint64_t* partials, int64_t stride, int32_t splits, const int32_t* nbpr,
                               const int64_t* start_pos, int32_t max_blocks, int64_t max_start, uint64_t* out,
                               int64_t out_stride, int32_t accumulate, hipStream_t stream) {
  int64_t grid = (stride + 3) / 4;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(reduce_dense_kernel, dim3((unsigned)grid), dim3(256), 0, stream, partials, stride, splits, nbpr,
                     start_pos, max_blocks, max_start, out, out_stride, accumulate);
  return hipGetLastError();
}

}  // namespace kvck

// Device-side helpers shared by the kernels of libkvck (not part of the ABI).
#pragma once

#include "kvck_internal.h"

namespace kvck {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int CHUNK>
struct ChunkType;
template <>
struct ChunkType<16> {
  using T = u32x4;
};
template <>
struct ChunkType<8> {
  using T = u32x2;
};

// Cache bytes are read exactly once: buffer loads with the non-temporal bit.
// The base address of the run lives in the (uniform) resource descriptor and
// each lane supplies a 32-bit byte offset.  A lane whose offset is kOOB or more
// is past num_records: a buffer load then returns zeros and touches no memory,
// which is how masked-off lanes and heads are handled without branches.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)kOOB, 0x00020000);
}

template <int CHUNK>
__device__ __forceinline__ typename ChunkType<CHUNK>::T load_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (CHUNK == 16)
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
  else
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kNonTemporal);
}

// Wavefront of the calling lane within its workgroup, and within the grid.
// threadIdx.x / 64 is the same on every lane of a wavefront, but the compiler
// cannot prove it; taken through readfirstlane it is a scalar, and so is all
// that derives from it (task, cache, page address).  Without that, each
// buffer load whose descriptor derives from it is wrapped in a loop that
// compares the descriptor across lanes.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}
__device__ __forceinline__ int64_t wave_index() {
  return (int64_t)blockIdx.x * (kBlockThreads / kWave) + wave_in_block();
}

// A 64-bit value moved across lanes by one DPP control, as two 32-bit halves;
// lanes of rows outside ROW_MASK get 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp_move(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}

// Sum of a 64-bit value over the 64 lanes of a wavefront, mod 2^64 (every lane
// gets it).  DPP steps, no LDS: pairs and quads (quad_perm), half-rows and
// rows of 16 (row_half_mirror, row_mirror), then row 0 into row 1 and row 2
// into row 3 (row_bcast:15), rows 0-1 into rows 2-3 (row_bcast:31); lane 63
// ends with the total.  Halves move separately; every add carries in 64 bits.
__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  v += dpp_move<0xb1>(v);        // quad_perm [1,0,3,2]
  v += dpp_move<0x4e>(v);        // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);       // row_half_mirror
  v += dpp_move<0x140>(v);       // row_mirror
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, kWave - 1);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), kWave - 1);
  return ((uint64_t)hi << 32) | lo;
}


// Lane chunk f of a row group -> row r, run of the row, chunk cr of the run.
// Rows in one piece are walked row by row (f = r * chunks_per_row + chunk).
// Rows stored as several runs (the x-split K layout, whose runs of all slots
// sit together) are walked in memory order, run by run and within a run slot
// by slot, so a load instruction still covers contiguous bytes.  Either way
// f < rows_per_group * chunks_per_row enumerates every (row, chunk) once.
struct LaneChunk {
  int r, run, cr;
};
__device__ __forceinline__ LaneChunk lane_chunk(int f, const BlocksArgs& a) {
  LaneChunk q;
  if (a.run_major) {
    q.cr = f % a.chunks_per_run;
    const int t = f / a.chunks_per_run;
    q.r = t % a.rows_per_group;
    q.run = t / a.rows_per_group;
  } else {
    q.r = f / a.chunks_per_row;
    const int c = f - q.r * a.chunks_per_row;
    q.run = c / a.chunks_per_run;
    q.cr = c - q.run * a.chunks_per_run;
  }
  return q;
}

template <int S>
struct LaneTable {
  int row[S];
  uint32_t off[S];
  uint32_t urel[S];
  template <int CHUNK>
  __device__ __forceinline__ void init(int lane, const BlocksArgs& a) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int f = lane + kWave * s;
      const LaneChunk q = lane_chunk(f, a);
      const int c = q.run * a.chunks_per_run + q.cr;  // chunk of the row
      row[s] = f < a.rows_per_group * a.chunks_per_row ? q.r : 0x7fffffff;
      off[s] = (uint32_t)((int64_t)q.r * a.slot_stride + (int64_t)q.run * a.chunk_stride + (int64_t)q.cr * CHUNK);
      // a merged row holds several heads' rows back to back: pieces count from its head's row
      const int cin = c - (c / a.chunks_per_head) * a.chunks_per_head;
      urel[s] = (uint32_t)(2u * (uint32_t)q.r * (uint32_t)a.pieces + (uint32_t)(CHUNK / 4) * (uint32_t)cin);
    }
  }
  // Local head of each chunk in a merged row (0 when rows are single heads).
  __device__ __forceinline__ void heads(int lane, const BlocksArgs& a, uint32_t (&h)[S]) const {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const LaneChunk q = lane_chunk(lane + kWave * s, a);
      h[s] = (uint32_t)((q.run * a.chunks_per_run + q.cr) / a.chunks_per_head);
    }
  }
};

// A request whose listed count is outside [0, max_blocks] or whose start
// position is negative or so large that a token index would overflow lists
// nothing (and is reported as a bad request).
__device__ __forceinline__ bool bad_request(int32_t n, int64_t start, int32_t max_blocks, int64_t max_start) {
  return n < 0 || n > max_blocks || start < 0 || start > max_start;
}

// Valid slots of the block whose first token is t0 (what the page's helper
// num_valid_tokens counts): the length of the overlap of its token span
// [t0, t0 + block_size) with the request's tokens [0, num_tokens).  Callers
// keep t0 <= INT64_MAX - block_size.
__device__ __forceinline__ int32_t valid_slots(int64_t num_tokens, int64_t t0, int32_t block_size) {
  const int64_t end = num_tokens < t0 + block_size ? num_tokens : t0 + block_size;
  return end > t0 ? (int32_t)(end - t0) : 0;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// An empty statement that reads v and may touch memory: v is complete before
// it, and no load moves above it.  Placed between the last use of a load
// buffer and its next loads, it keeps the two from overlapping, so a buffer
// reloaded in a loop keeps its registers instead of being copied back (and
// waited for) at every step.
__device__ __forceinline__ void order_after(uint64_t v) { asm volatile("" ::"v"(v) : "memory"); }

// Wait until every vector memory access the wave has issued is complete
// (s_waitcnt vmcnt(0); the scalar-memory and export counters are not waited
// for).
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Read-only inputs of a launch (the plan, the request arrays) read through
// the constant address space: at a uniform address that is a scalar load,
// counted apart from the vector loads of cache bytes, so waiting for a task's
// record does not also wait for the cache loads still in flight.
template <class T>
__device__ __forceinline__ T read_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// What a task needs of its position.  `listed` is false for dense slots past
// a request's listed count (or of a bad request): such tasks write nothing.
struct TaskRecord {
  uint64_t t0;
  int64_t out_idx;
  int32_t block, valid;
  bool listed;
};

// Record of task item `item`, uniform over the wave.  Planned calls read the
// plan's compact list; dense calls derive it from the request arrays with the
// plan's rules (bad requests list nothing, an id outside the pool in a block
// with valid slots contributes 0), and `report` lets one task per slot raise
// the error bits.  DENSE is a template parameter so that the planned kernels
// keep none of the request pointers live.
template <bool DENSE>
__device__ __forceinline__ TaskRecord task_record(const BlocksArgs& a, int64_t item, bool report, int lane) {
  TaskRecord t;
  if constexpr (!DENSE) {
    const PosRecord* rp = a.recs + item;
    t.valid = __builtin_amdgcn_readfirstlane(read_const(&rp->valid));
    t.block = __builtin_amdgcn_readfirstlane(read_const(&rp->block));
    t.t0 = (uint64_t)uniform64(read_const(&rp->t0));
    t.out_idx = read_const(&rp->out_idx);
    t.listed = true;
    return t;
  }
  const int32_t r = (int32_t)item / a.max_blocks;  // item < 2^31
  const int32_t k = (int32_t)item - r * a.max_blocks;
  // four independent loads; the table entry is in bounds for every k < max_blocks
  const int32_t n = __builtin_amdgcn_readfirstlane(read_const(a.nbpr + r));
  const int64_t s = uniform64(read_const(a.start_pos + r));
  const int64_t ntok = uniform64(read_const(a.num_tokens + r));
  const int32_t b = __builtin_amdgcn_readfirstlane(read_const(a.block_table + (int64_t)r * a.bt_stride + k));
  t.out_idx = item * a.out_stride;
  t.block = b;
  t.valid = 0;
  t.t0 = 0;
  t.listed = false;
  if (bad_request(n, s, a.max_blocks, a.max_start)) {
    if (report && k == 0 && lane == 0 && a.req_flags) atomicOr(a.req_flags, KVCK_FLAG_BAD_REQUEST);
    return t;
  }
  if (k >= n) return t;
  t.listed = true;
  const int64_t t0 = (s + k) * (int64_t)a.block_size;
  t.t0 = (uint64_t)t0;
  t.valid = valid_slots(ntok, t0, a.block_size);
  if (t.valid > 0 && (b < 0 || (int64_t)b >= a.num_blocks)) {
    if (report && lane == 0 && a.req_flags) atomicOr(a.req_flags, KVCK_FLAG_BAD_BLOCK_ID);
    t.valid = 0;
  }
  return t;
}

// Position of the next unit of a task: cache, row group, plane, head batch.
// Both orders visit the nhb * planes * ngr units of every cache once.
struct UnitCursor {
  int cache, group, plane, hbatch;
  // head batches, then planes, then row groups, then caches
  __device__ __forceinline__ void next(int nhb, int planes, int ngr) {
    if (++hbatch == nhb) {
      hbatch = 0;
      if (++plane == planes) {
        plane = 0;
        if (++group == ngr) {
          group = 0;
          ++cache;
        }
      }
    }
  }
  // head batches, then row groups, then planes, then caches: a plane's row
  // groups are visited back to back, so consecutive units of a block lie side
  // by side in memory instead of alternating between its K and V planes
  __device__ __forceinline__ void next_group_first(int nhb, int planes, int ngr) {
    if (++hbatch == nhb) {
      hbatch = 0;
      if (++group == ngr) {
        group = 0;
        if (++plane == planes) {
          plane = 0;
          ++cache;
        }
      }
    }
  }
};

}  // namespace kvck

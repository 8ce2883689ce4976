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

// Sum of a 64-bit value over the 64 lanes of a wavefront (every lane gets it).
__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
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

// Position of the next unit of a task: cache, row group, plane, head batch.
struct UnitCursor {
  int cache, group, plane, hbatch;
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
};

}  // namespace kvck

// Block checksums of K/V planes stored element-transposed, on gfx950: element
// d of slot i's row sits at d * elem_stride + i * ES, so one element index of
// all the block's slots is contiguous (the V layout
// [num_blocks, num_heads, head_size, block_size] of ROCm's paged-attention
// kernels).  The checksum is the one of the vLLM API page
// "vllm.distributed.kv_transfer.kv_checksum.checksum"; a token's row is still
// its head_size elements in order, read as little-endian 8-byte pieces.
//
// No element gather is needed: a piece is the little-endian packing of
// PER_PIECE = 8/ES consecutive elements, so for element d of token t
//   x_q (2j + 1) = sum over its elements e_d * 2^(8 ES (d mod PER_PIECE)) * u,
//   u = 2 (t P + pb + d / PER_PIECE) + 1      (pb: first piece of the plane),
// and a 16-byte chunk holds element d of N = 16/ES consecutive slots t0+k, whose
// terms sum to ((u0 E + 2 P K) << 8 ES (d mod PER_PIECE)) with
// E = sum_k e_k, K = sum_k k e_k over the valid slots and u0 the u of slot t0.
//
// Task = (group of caches, listed position), one wavefront each, as in the
// main pass; a unit is HU heads x S chunks per lane of one element-row group,
// with the same out-of-range buffer offsets masking unused lanes and heads.
// PIPE: two unit buffers in ping-pong, as in the main pass's pipelined kernel.
// DENSE: planned in place, one task per wave, as in the main pass.
#include "kvck_tdevice.h"

namespace kvck {
namespace {

template <int CHUNK, int ES, int S, int HU, bool PIPE, bool DENSE>
__global__ __launch_bounds__(kBlockThreads) void tblocks_kernel(const BlocksArgs a) {
  using V = typename ChunkType<CHUNK>::T;
  constexpr int N = CHUNK / ES;        // slots per chunk
  constexpr int PER_PIECE = 8 / ES;    // elements per 8-byte piece
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = wave_index();
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n_items = DENSE ? a.max_items : (int64_t)*a.n_items;
  const int lpt = a.caches_per_task;
  const int ngroups = (a.num_caches + lpt - 1) / lpt;
  const int64_t total = n_items * ngroups;
  if (wave >= total) return;

  // lane table of one element-row group of a (block, head): chunk f = lane + 64 s
  // holds element row f / cpe of the group, slots (f mod cpe) * N onward
  const int cpe = a.chunks_per_row;
  const int rge = a.rows_per_group;
  int erow[S];
  uint32_t off[S], slot0[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int f = lane + kWave * s;
    const int r = f / cpe;
    const int q = f - r * cpe;
    erow[s] = f < rge * cpe ? r : 0x7fffffff;
    off[s] = (uint32_t)((int64_t)r * a.chunk_stride + (int64_t)q * CHUNK);
    slot0[s] = (uint32_t)(q * N);
  }
  const int D = a.row_bytes / ES;                 // elements per row
  const int ngr = (D + rge - 1) / rge;            // element-row groups
  const uint64_t P = (uint64_t)a.pieces;
  const int nhb = (a.heads + HU - 1) / HU;

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
      // valid slots of each lane chunk, and the chunk's u without the element's piece
      int nvalid[S];
      uint64_t ubase[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int left = v - (int)slot0[s];
        nvalid[s] = left < 0 ? 0 : (left > N ? N : left);
        ubase[s] = 2ull * (t0 + slot0[s]) * P + 1ull + a.piece_base;
      }
      // units: (cache, element-row group, head batch), cache-major
      struct Cursor {
        int cache, group, hbatch;
        __device__ __forceinline__ void next(int nhb_, int ngr_) {
          if (++hbatch == nhb_) {
            hbatch = 0;
            if (++group == ngr_) {
              group = 0;
              ++cache;
            }
          }
        }
      };
      const int nunits = (c_end - c_begin) * ngr * nhb;
      Cursor ic{c_begin, 0, 0}, cc{c_begin, 0, 0};
      // `live` false: a unit past the task's last one, every load out of range
      auto issue = [&](V(&x)[HU][S], bool live) {
        const int rows = live ? min(rge, D - ic.group * rge) : 0;
        const uint8_t* gbase =
            a.base[live ? ic.cache : c_begin] + blk_off + (int64_t)(ic.group * rge) * a.chunk_stride;
#pragma unroll
        for (int h = 0; h < HU; ++h) {
          const int hh = ic.hbatch * HU + h;
          const uint32_t hmask = hh < a.heads ? 0u : kOOB;
          const __amdgpu_buffer_rsrc_t rs = make_rsrc(gbase + (int64_t)hh * a.head_stride);
#pragma unroll
          for (int s = 0; s < S; ++s)
            x[h][s] = load_chunk<CHUNK>(rs, (erow[s] < rows && nvalid[s] > 0 ? off[s] : kOOB) | hmask);
        }
        if (live) ic.next(nhb, ngr);
      };
      auto consume = [&](const V(&x)[HU][S]) {
        const uint64_t mb = a.mbase[cc.cache];
#pragma unroll
        for (int h = 0; h < HU; ++h) {
          uint64_t sh = 0;
#pragma unroll
          for (int s = 0; s < S; ++s) {
            // element index; masked lanes read zeros, so any d is harmless there
            const uint32_t d = (uint32_t)(cc.group * rge) + (uint32_t)erow[s];
            uint64_t E, K;
            chunk_sums<ES>(x[h][s], nvalid[s], E, K);
            const uint64_t u0 = ubase[s] + 2ull * (d / PER_PIECE);
            sh += (u0 * E + 2ull * P * K) << (8 * ES * (d % PER_PIECE));
          }
          acc += sh * (mb + 2ull * (uint64_t)(cc.hbatch * HU + h));
        }
        cc.next(nhb, ngr);
      };
      if constexpr (PIPE) {
        // Both buffers are issued at every step (past the last unit with every
        // load out of range) and order_after keeps a buffer's next loads after
        // the last use of its data, as in the row-layout kernel: the waits for
        // one buffer then leave the other's loads in flight.
        V A[HU][S], B[HU][S];
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
          V A[HU][S];
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

using TFn = void (*)(const BlocksArgs);

template <int CHUNK, int ES, int S, bool PIPE, bool DENSE>
constexpr TFn tpick() {
  return &tblocks_kernel<CHUNK, ES, S, (16 / S > 0 ? 16 / S : 1), PIPE, DENSE>;
}

// The pipelined kernel double-buffers lane tables of at most 4 slots.
template <int CHUNK, int ES, bool DENSE>
TFn tfn_slots(int slots, bool pipe) {
  switch (slots) {
    case 1: return pipe ? tpick<CHUNK, ES, 1, true, DENSE>() : tpick<CHUNK, ES, 1, false, DENSE>();
    case 2: return pipe ? tpick<CHUNK, ES, 2, true, DENSE>() : tpick<CHUNK, ES, 2, false, DENSE>();
    case 4: return pipe ? tpick<CHUNK, ES, 4, true, DENSE>() : tpick<CHUNK, ES, 4, false, DENSE>();
    case 8: return pipe ? nullptr : tpick<CHUNK, ES, 8, false, DENSE>();
    case 16: return pipe ? nullptr : tpick<CHUNK, ES, 16, false, DENSE>();
  }
  return nullptr;
}

template <bool DENSE>
TFn tfn_plan(const BlocksShape& shp) {
  const bool pipe = shp.pipelined;
  if (shp.chunk == 16) {
    switch (shp.elem_bytes) {
      case 1: return tfn_slots<16, 1, DENSE>(shp.slots, pipe);
      case 2: return tfn_slots<16, 2, DENSE>(shp.slots, pipe);
      case 4: return tfn_slots<16, 4, DENSE>(shp.slots, pipe);
    }
  } else {
    switch (shp.elem_bytes) {
      case 1: return tfn_slots<8, 1, DENSE>(shp.slots, pipe);
      case 2: return tfn_slots<8, 2, DENSE>(shp.slots, pipe);
      case 4: return tfn_slots<8, 4, DENSE>(shp.slots, pipe);
    }
  }
  return nullptr;
}

// Every variant exists planned and planned in place.
TFn tfn(const BlocksShape& shp) { return shp.dense ? tfn_plan<true>(shp) : tfn_plan<false>(shp); }

}  // namespace

int tblocks_grid(const BlocksShape& shp, int device, int64_t max_tasks) {
  TFn fn = tfn(shp);
  const int fits = fn ? kernel_occupancy(reinterpret_cast<const void*>(fn), device, 2) : 1;
  const int per_cu = workgroups_per_cu(fits, kAllThatFit);
  const int64_t waves_per_block = kBlockThreads / kWave;
  const int64_t need = (max_tasks + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)per_cu * device_cus(device);
  if (shp.dense) return (int)(need > 0 ? need : 1);  // one task per wave (at most kDenseMaxTasks)
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

hipError_t launch_tblocks(const BlocksArgs& a, const BlocksShape& shp, int grid, hipStream_t stream) {
  TFn fn = tfn(shp);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<BlocksArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(kBlockThreads), args, 0, stream);
}

}  // namespace kvck

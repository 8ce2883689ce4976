// Fused copy + checksum of paged K/V blocks on gfx950: a connector's save
// (pool -> staging buffer) or load (staging buffer -> pool) that also yields
// the block checksums of the vLLM API page
// "vllm.distributed.kv_transfer.kv_checksum.checksum", from one read and one
// write of every valid row.
//
// Staging layout: listed positions in request order (entry e of request r's
// k-th listed position is sum_{r'<r} listed(r') + k), and per entry one block
// image per cache of the call, in cache order; an image is
//   [plane][head][slot][row_bytes]      (planes x head_count x block_size rows)
// holding only the valid slots of the position (slots at or past num_tokens
// are neither read nor written, on either side).
//
// The kernel keeps the main pass's task structure, with a second lane table
// for the staging side: each unit is loaded from one side, stored to the other
// and folded into the checksum.  For a load a wave holds one unit buffer (more
// resident waves keep more stores in flight); a save runs the ping-pong
// variant (PIPE), which keeps unit i+1's loads in flight while unit i is
// stored, at one workgroup per CU.  Positions are visited grouped by block id
// (order_kernel below).  MERGED: pools whose heads sit side by side in a slot
// with short rows are walked as one row per slot (as in the checksum pass),
// and each lane chunk's staging offset lands in its own head's image rows.
#include "kvck_device.h"

namespace kvck {
namespace {

// Cache policy of the stores: non-temporal on both sides, and on a load (the
// pool side, block by block) device scope as well (SC1), which writes the
// lines through rather than leaving them in the issuing XCD's L2.  Same-box
// A/B on the 128-request llama3-shaped batch: load 24.62 -> 24.39 ms with it
// (plain or SC0 stores: 25.12); the save's staging stores are fastest without
// it (23.23 -> 23.35 ms with it).
constexpr int kStoreDeviceScope = 16;  // SC1 bit of the buffer instruction's cache policy

template <int CHUNK, int POL>
__device__ __forceinline__ void store_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                            const typename ChunkType<CHUNK>::T& v) {
  if constexpr (CHUNK == 16)
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, POL);
  else
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, POL);
}

template <int CHUNK, int S, int HU, int PU, int DIR, bool PIPE, bool MERGED>
__global__ __launch_bounds__(kBlockThreads) void copy_kernel(const CopyArgs ca) {
  using V = typename ChunkType<CHUNK>::T;
  const BlocksArgs& a = ca.b;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = wave_index();
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n_items = (int64_t)*a.n_items;
  const int lpt = a.caches_per_task;
  const int ngroups = (a.num_caches + lpt - 1) / lpt;
  const int64_t total = n_items * ngroups;
  if (wave >= total) return;

  LaneTable<S> lt;
  lt.template init<CHUNK>(lane, a);
  uint32_t lhead[S];  // local head of each lane chunk (merged rows only)
  if constexpr (MERGED) lt.heads(lane, a, lhead);
  const int64_t img_head = (int64_t)ca.block_size * a.row_bytes;
  const int64_t img_plane = ca.image_bytes / a.planes;  // head_count images of one plane
  uint32_t ioff[S];  // staging-side offsets of the same chunks: rows are row_bytes apart
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const LaneChunk q = lane_chunk(lane + kWave * s, a);
    const int c = q.run * a.chunks_per_run + q.cr;  // chunk of the (merged) row
    if constexpr (MERGED) {
      const int cin = c - (int)lhead[s] * a.chunks_per_head;
      ioff[s] = (uint32_t)((int64_t)lhead[s] * img_head + (int64_t)q.r * a.row_bytes + (int64_t)cin * CHUNK);
    } else {
      ioff[s] = (uint32_t)((int64_t)q.r * a.row_bytes + (int64_t)c * CHUNK);
    }
  }
  const uint64_t P = (uint64_t)a.pieces;
  const int rg = a.rows_per_group;
  const uint64_t plane_term = 2ull * (P / (uint64_t)a.planes_total);
  const int nhb = (a.heads + HU - 1) / HU;

  for (int64_t task = wave; task < total; task += nwaves) {
    const int64_t grp = task / n_items;
    const int64_t idx = task - grp * n_items;
    // listed position (staging entry) the task covers, in the visiting order
    const int64_t item = ca.order ? (int64_t)__builtin_amdgcn_readfirstlane(read_const(ca.order + idx)) : idx;
    const int c_begin = (int)grp * lpt;
    const int c_end = min(a.num_caches, c_begin + lpt);
    const TaskRecord rec = task_record<false>(a, item, false, lane);
    int32_t v = rec.valid;
    const int32_t blk = rec.block;
    const uint64_t t0 = rec.t0;
    const int64_t out_idx = rec.out_idx;
    if (item >= ca.staging_positions) {
      if (v > 0 && lane == 0 && ca.error_flags) atomicOr(ca.error_flags, KVCK_FLAG_STAGING_FULL);
      v = 0;
    }
    uint64_t acc = 0;
    if (v > 0) {
      const int64_t blk_off = (int64_t)blk * a.block_stride;
      uint8_t* const img0 = ca.staging + (item * ca.num_caches_total + ca.cache_offset) * ca.image_bytes;
      const int ngr = (v + rg - 1) / rg;
      const int nplanes = a.planes / PU;
      const int nunits = ngr * nplanes * nhb * (c_end - c_begin);
      UnitCursor ic{c_begin, 0, 0, 0}, cc{c_begin, 0, 0, 0};

      // base of (cache, group, plane, head) on the pool side and on the staging side
      auto pool_base = [&](const UnitCursor& u, int p, int hh) {
        return a.base[u.cache] + blk_off + (int64_t)(u.group * rg) * a.slot_stride +
               (int64_t)(u.plane * PU + p) * a.plane_stride + (int64_t)hh * a.head_stride;
      };
      auto img_base = [&](const UnitCursor& u, int p, int hh) {
        return img0 + (int64_t)u.cache * ca.image_bytes + (int64_t)(u.plane * PU + p) * img_plane +
               (int64_t)hh * img_head + (int64_t)(u.group * rg) * a.row_bytes;
      };
      // `live` false: a unit past the task's last one, every load out of range
      auto issue = [&](V(&x)[PU][HU][S], bool live) {
        const int rows = live ? min(rg, v - ic.group * rg) : 0;
        UnitCursor u = ic;
        if (!live) u.cache = c_begin;
#pragma unroll
        for (int p = 0; p < PU; ++p) {
#pragma unroll
          for (int h = 0; h < HU; ++h) {
            const int hh = u.hbatch * HU + h;
            const uint32_t hmask = hh < a.heads ? 0u : kOOB;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(DIR == 0 ? pool_base(u, p, hh) : img_base(u, p, hh));
#pragma unroll
            for (int s = 0; s < S; ++s)
              x[p][h][s] = load_chunk<CHUNK>(rs, (lt.row[s] < rows ? (DIR == 0 ? lt.off[s] : ioff[s]) : kOOB) | hmask);
          }
        }
        if (live) ic.next(nhb, nplanes, ngr);
      };
      auto store_consume = [&](const V(&x)[PU][HU][S]) {
        const int rows = min(rg, v - cc.group * rg);
        const uint64_t mb = a.mbase[cc.cache];
#pragma unroll
        for (int p = 0; p < PU; ++p) {
          const uint64_t up = 2ull * (t0 + (uint64_t)(cc.group * rg)) * P + 1ull + a.piece_base +
                              (uint64_t)(cc.plane * PU + p) * plane_term;
#pragma unroll
          for (int h = 0; h < HU; ++h) {
            const int hh = cc.hbatch * HU + h;
            const uint32_t hmask = hh < a.heads ? 0u : kOOB;
            const __amdgpu_buffer_rsrc_t rd = make_rsrc(DIR == 0 ? img_base(cc, p, hh) : pool_base(cc, p, hh));
            // as in the checksum kernel: mb * sh + 2 sl for merged rows
            uint64_t sh = 0, sl = 0;
#pragma unroll
            for (int s = 0; s < S; ++s) {
              store_chunk<CHUNK, DIR == 0 ? kNonTemporal : kNonTemporal | kStoreDeviceScope>(
                  rd, (lt.row[s] < rows ? (DIR == 0 ? ioff[s] : lt.off[s]) : kOOB) | hmask, x[p][h][s]);
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
              acc += sh * (mb + 2ull * (uint64_t)hh);
          }
        }
        cc.next(nhb, nplanes, ngr);
      };

      if constexpr (PIPE) {
        // Both buffers are issued at every step (past the last unit with every
        // load out of range) and order_after keeps a buffer's next loads after
        // the last use of its data, as in the checksum kernel.
        V A[PU][HU][S], B[PU][HU][S];
        issue(A, true);
        for (int ui = 0; ui < nunits; ui += 2) {
          issue(B, ui + 1 < nunits);
          store_consume(A);
          order_after(acc);
          issue(A, ui + 2 < nunits);
          if (ui + 1 < nunits) store_consume(B);
          order_after(acc);
        }
      } else {
        for (int ui = 0; ui < nunits; ++ui) {
          V A[PU][HU][S];
          issue(A, true);
          store_consume(A);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      if (a.direct) {
        uint64_t* o = a.out + out_idx;
        *o = a.accumulate ? *o + acc : acc;
      } else {
        a.partials[(int64_t)(a.group_offset + grp) * a.max_items + item] = acc;
      }
    }
  }
}

// Visiting order of the fused copy: the listed positions grouped by block id
// (a counting sort into kOrderBins buckets of block ids, in one workgroup, its
// histogram in 128 KiB of LDS), so the waves resident at any moment touch
// nearby pool blocks.  The order within a bucket is whatever the atomics give;
// results never depend on it.  Same-box A/B over the 128-request llama3-shaped
// batch (73k pool blocks), whole calls: listing order 24.38 ms load / 23.27 ms
// save; 8192 buckets 24.11 / 22.75; 32768 buckets 23.93 / 22.73 (the sort
// itself ~0.07 ms).
constexpr int kOrderBins = 32768;
constexpr int kOrderThreads = 1024;
constexpr int kOrderUnroll = 8;

__device__ __forceinline__ uint32_t order_bin(const PosRecord* recs, int64_t i, int shift) {
  // a negative id (flagged, no valid slots) in the first bucket, one past the pool in the last
  const int32_t b = recs[i].block;
  const uint32_t q = (uint32_t)b >> shift;
  return b < 0 ? 0u : (q < (uint32_t)kOrderBins ? q : (uint32_t)kOrderBins - 1u);
}

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const PosRecord* __restrict__ recs,
                                                              const uint32_t* __restrict__ n_items, int shift,
                                                              int32_t* __restrict__ order) {
  __shared__ uint32_t hist[kOrderBins];
  __shared__ uint32_t sums[kOrderThreads];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)*n_items;
  for (int b = tid; b < kOrderBins; b += kOrderThreads) hist[b] = 0;
  __syncthreads();
  constexpr int64_t kStep = (int64_t)kOrderThreads * kOrderUnroll;
  for (int64_t i0 = 0; i0 < n; i0 += kStep) {
    uint32_t bin[kOrderUnroll];
#pragma unroll
    for (int k = 0; k < kOrderUnroll; ++k) {
      const int64_t i = i0 + (int64_t)k * kOrderThreads + tid;
      bin[k] = i < n ? order_bin(recs, i, shift) : kOrderBins;
    }
#pragma unroll
    for (int k = 0; k < kOrderUnroll; ++k)
      if (bin[k] < kOrderBins) atomicAdd(&hist[bin[k]], 1u);
  }
  __syncthreads();
  // exclusive scan: each thread owns kOrderBins / kOrderThreads consecutive buckets
  constexpr int kPer = kOrderBins / kOrderThreads;
  uint32_t own = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) own += hist[tid * kPer + j];
  sums[tid] = own;
  __syncthreads();
  for (int o = 1; o < kOrderThreads; o <<= 1) {
    const uint32_t t = tid >= o ? sums[tid - o] : 0u;
    __syncthreads();
    sums[tid] += t;
    __syncthreads();
  }
  uint32_t run = sums[tid] - own;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t c = hist[tid * kPer + j];
    hist[tid * kPer + j] = run;
    run += c;
  }
  __syncthreads();
  for (int64_t i0 = 0; i0 < n; i0 += kStep) {
    uint32_t bin[kOrderUnroll];
#pragma unroll
    for (int k = 0; k < kOrderUnroll; ++k) {
      const int64_t i = i0 + (int64_t)k * kOrderThreads + tid;
      bin[k] = i < n ? order_bin(recs, i, shift) : kOrderBins;
    }
#pragma unroll
    for (int k = 0; k < kOrderUnroll; ++k)
      if (bin[k] < kOrderBins) order[atomicAdd(&hist[bin[k]], 1u)] = (int32_t)(i0 + (int64_t)k * kOrderThreads + tid);
  }
}

using CopyFn = void (*)(const CopyArgs);

template <int CHUNK, int S, int PU, int DIR, bool MERGED>
CopyFn pick(bool pipe) {
  constexpr int hu = MERGED ? 1 : (16 / (S * PU) > 0 ? 16 / (S * PU) : 1);
  return pipe ? &copy_kernel<CHUNK, S, hu, PU, DIR, true, MERGED> : &copy_kernel<CHUNK, S, hu, PU, DIR, false, MERGED>;
}

template <int CHUNK, int PU, int DIR, bool MERGED = false>
CopyFn copy_fn_slots(int slots, bool pipe) {
  switch (slots) {
    case 1: return pick<CHUNK, 1, PU, DIR, MERGED>(pipe);
    case 2: return pick<CHUNK, 2, PU, DIR, MERGED>(pipe);
    case 4: return pick<CHUNK, 4, PU, DIR, MERGED>(pipe);
    case 8: return pick<CHUNK, 8, 1, DIR, MERGED>(pipe);
    case 16: return pick<CHUNK, 16, 1, DIR, MERGED>(pipe);
  }
  return nullptr;
}

// Merged rows take one plane per unit.
template <int DIR>
CopyFn copy_fn_dir(const BlocksShape& shp) {
  const bool pipe = shp.copy_buffers == 2;
  if (shp.merged)
    return shp.chunk == 16 ? copy_fn_slots<16, 1, DIR, true>(shp.slots, pipe)
                           : copy_fn_slots<8, 1, DIR, true>(shp.slots, pipe);
  if (shp.planes_per_unit == 2)
    return shp.chunk == 16 ? copy_fn_slots<16, 2, DIR>(shp.slots, pipe) : copy_fn_slots<8, 2, DIR>(shp.slots, pipe);
  return shp.chunk == 16 ? copy_fn_slots<16, 1, DIR>(shp.slots, pipe) : copy_fn_slots<8, 1, DIR>(shp.slots, pipe);
}

CopyFn copy_fn(const BlocksShape& shp, int direction) {
  return direction == KVCK_COPY_SAVE ? copy_fn_dir<0>(shp) : copy_fn_dir<1>(shp);
}

}  // namespace

int copy_grid(const BlocksShape& shp, int direction, int device, int64_t max_tasks) {
  CopyFn fn = copy_fn(shp, direction);
  const int fits = fn ? kernel_occupancy(reinterpret_cast<const void*>(fn), device, 1) : 1;
  // the save's ping-pong kernel at one workgroup per CU; otherwise as many as fit
  const int per_cu = workgroups_per_cu(
      fits, shp.copy_buffers == 2 && direction == KVCK_COPY_SAVE ? kMainWorkgroupsPerCU : kAllThatFit);
  const int cus = device_cus(device);
  const int64_t waves_per_block = kBlockThreads / kWave;
  const int64_t need = (max_tasks + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)per_cu * cus;
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

hipError_t launch_order(const PosRecord* recs, const uint32_t* n_items, int64_t num_blocks, int32_t* order,
                        hipStream_t stream) {
  // bucket = block >> shift, with every block id of the pool below kOrderBins << shift
  int shift = 0;
  while (shift < 31 && ((num_blocks - 1) >> shift) >= kOrderBins) ++shift;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, recs, n_items, shift, order);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, const BlocksShape& shp, int direction, int grid, hipStream_t stream) {
  CopyFn fn = copy_fn(shp, direction);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<CopyArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(kBlockThreads), args, 0, stream);
}

}  // namespace kvck

// Mamba running-state checksums on gfx950.
//
// Mamba paragraph of the vLLM API page
// "vllm.distributed.kv_transfer.kv_checksum.checksum": for a Mamba group the
// request's running state stands in for its blocks (position 0); when the
// layer's TP split is known, each global row along that split is a slice, and
// the pieces are the row's elements (2 or 4 bytes each) as unsigned integers.
// Slice g = row g of every state of the layer, concatenated in state order,
// elements numbered e = 0, 1, ..:
//   s(g) = sum over e of x_e (2e + 1);  c = sum over (layer, g) of m s(g),
//   m = 2 (layer*65536 + g) + 1, all modulo 2^64.
//
// Task = (request, layer, group of rows), one wavefront each.  Lanes stream the
// row's 16-byte chunks; a chunk of 4-byte elements x0..x3 starting at element e
// adds sum_i x_i (2(e+i) + 1); a chunk of 2-byte elements x0..x7 adds
// u*X + 2*Y with u = 2e + 1, X = sum x_i, Y = sum i*x_i (both fit 32 bits).
#include "kvck_device.h"

namespace kvck {
namespace {

__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint64_t chunk_u32(u32x4 x, uint32_t u) {
  return (uint64_t)x.x * u + (uint64_t)x.y * (u + 2u) + (uint64_t)x.z * (u + 4u) + (uint64_t)x.w * (u + 6u);
}

__device__ __forceinline__ uint64_t chunk_u16(u32x4 x, uint32_t u) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t X = 0, Y = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0xffffu, hi = w[i] >> 16;
    X += lo + hi;
    Y += (2u * i) * lo + (2u * i + 1u) * hi;
  }
  return (uint64_t)X * u + 2ull * Y;
}

// Loads in flight per lane per batch.  Same-box interleaved A/B on the hybrid
// model's 24 Mamba layers (2.01 GB): 2 loads (128 chunks, a whole fp16 conv
// row) read 0.8-1.3 points of 8 TB/s faster than 8, and 1 or 4 were slower;
// fewer registers leave room for more resident waves.
constexpr int kUnroll = 2;

__global__ __launch_bounds__(kBlockThreads) void states_kernel(const StatesArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * (kBlockThreads / kWave) + (threadIdx.x / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t splits = (int64_t)a.num_layers * a.groups_per_layer;
  const int64_t total = splits * a.num_reqs;
  for (int64_t task = wave; task < total; task += nwaves) {
    // request-major: the waves resident at once read whole slots' states (a
    // slot's rows are contiguous) rather than the same rows of many slots,
    // whose addresses lie a slot's size apart and crowd the same HBM channels
    const int32_t r = (int32_t)(task / splits);
    const int32_t split = (int32_t)(task - (int64_t)r * splits);
    const int32_t l = split / a.groups_per_layer;
    const int32_t grp = split - l * a.groups_per_layer;
    const int32_t slot = a.slot_ids[r];
    uint64_t acc = 0;
    if (slot < 0 || slot >= a.num_slots) {
      if (lane == 0 && a.error_flags) atomicOr(a.error_flags, KVCK_FLAG_BAD_STATE_SLOT);
    } else {
      const int32_t g_begin = grp * a.rows_per_task;
      const int32_t g_end = min(a.row_count, g_begin + a.rows_per_task);
      for (int32_t g = g_begin; g < g_end; ++g) {
        uint64_t s = 0;
        for (int st = 0; st < a.nstates; ++st) {
          const uint8_t* rowp = a.ptr[l][st] + (int64_t)slot * a.slot_stride[st] +
                                (int64_t)(a.row_begin + g) * a.row_stride[st];
          const int32_t nch = a.row_chunks[st];
          const bool wide = a.elem_bytes[st] == 4;
          const uint32_t e0 = (uint32_t)a.elem_off[st];
          const uint32_t per_chunk = wide ? 4u : 8u;
          for (int32_t c0 = 0; c0 < nch; c0 += kWave * kUnroll) {
            u32x4 x[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
              const int32_t c = c0 + k * kWave + lane;
              x[k] = c < nch ? load16(rowp + (int64_t)c * 16) : u32x4(0);
            }
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
              const uint32_t c = (uint32_t)(c0 + k * kWave + lane);
              const uint32_t u = 2u * (e0 + c * per_chunk) + 1u;
              s += wide ? chunk_u32(x[k], u) : chunk_u16(x[k], u);
            }
          }
        }
        acc += s * (a.mbase[l] + 2ull * (uint64_t)g);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      if (a.direct) {
        uint64_t* o = a.out + (int64_t)r * a.out_stride;
        *o = a.accumulate ? *o + acc : acc;
      } else {
        a.partials[(int64_t)(a.split_offset + split) * a.num_reqs + r] = acc;
      }
    }
  }
}

}  // namespace

int states_grid(int device, int64_t tasks) {
  const int fits = kernel_occupancy(reinterpret_cast<const void*>(&states_kernel), device, 2);
  const int per_cu = workgroups_per_cu(fits, kAllThatFit);
  const int cus = device_cus(device);
  const int64_t need = (tasks + (kBlockThreads / kWave) - 1) / (kBlockThreads / kWave);
  const int64_t cap = (int64_t)per_cu * cus;
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

hipError_t launch_states(const StatesArgs& a, int grid, hipStream_t stream) {
  void* args[] = {const_cast<StatesArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&states_kernel), dim3(grid), dim3(kBlockThreads), args, 0,
                         stream);
}

}  // namespace kvck

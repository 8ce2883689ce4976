// Fused copy + checksum of element-transposed K/V planes on gfx950: a
// connector's save (pool -> staging) or load (staging -> pool) for planes
// stored [num_blocks, num_heads, head_size, block_size] (ROCm's
// paged-attention V layout), with the checksum of the vLLM API page
// "vllm.distributed.kv_transfer.kv_checksum.checksum".
//
// The staging image is the same as for every other layout, [head][slot][row]
// with a token's row its head_size elements in order, so a block saved from
// one layout loads into another.  The pool holds the transpose of that image
// per (block, head), so the copy transposes it, in one of two ways:
//  - tcopy_lds_kernel (16-byte chunks, the default): through a per-wave LDS
//    region holding the image in staging form, so that both the pool side and
//    the staging side move whole contiguous chunks;
//  - tcopy_kernel (8-byte chunks, small blocks): in registers, the image cut
//    into N x N tiles of ES-byte elements (N = CHUNK / ES, the elements of one
//    chunk), a tile held by N consecutive lanes, one chunk each, and a
//    butterfly exchange between those lanes turning pool chunks (one element
//    index of N slots) into staging chunks (N elements of one slot) and back.
// Either way the checksum is taken on the pool-side form of each chunk,
// exactly as in the element-transposed checksum pass.
//
// Valid slots only: a save reads pool chunks holding at least one valid slot
// and stores the staging rows of valid slots; a load reads the staging rows of
// valid slots and writes exactly their elements into the pool (a chunk that
// straddles the last valid slot is written element by element).
#include "kvck_tdevice.h"

namespace kvck {
namespace {

// In-register transpose of an N x N tile (N = W * 4 / ES elements of ES bytes)
// spread over N consecutive lanes, lane j holding row j in w[0..W): afterwards
// lane j holds column j.  Stage d (a power of two below N) exchanges, between
// lanes j and j ^ d, the elements whose index bit d differs from the lane's
// bit d; after all stages element (j, e) sits at (e, j).
template <int ES, int W>
__device__ __forceinline__ void tile_transpose(uint32_t (&w)[W], int j) {
  constexpr int EPD = 4 / ES;  // elements per 32-bit word
  constexpr int N = W * EPD;
#pragma unroll
  for (int d = N / 2; d >= 1; d >>= 1) {
    const bool hi = (j & d) != 0;
    uint32_t p[W];
#pragma unroll
    for (int i = 0; i < W; ++i) p[i] = (uint32_t)__shfl_xor((int)w[i], d, kWave);
    if (d >= EPD) {
      // whole words: word i takes the partner's word i ^ dd where bit dd of i
      // differs from the lane's bit
      const int dd = d / EPD;
      uint32_t n[W];
#pragma unroll
      for (int i = 0; i < W; ++i) n[i] = (((i & dd) != 0) != hi) ? p[i ^ dd] : w[i];
#pragma unroll
      for (int i = 0; i < W; ++i) w[i] = n[i];
    } else {
      // within words: blocks of d elements (8*ES*d bits) trade places
      const int bits = 8 * ES * d;
      const uint32_t lo = bits == 16 ? 0x0000ffffu : 0x00ff00ffu;  // blocks with element bit d clear
#pragma unroll
      for (int i = 0; i < W; ++i)
        w[i] = hi ? (((p[i] >> bits) & lo) | (w[i] & ~lo)) : ((w[i] & lo) | ((p[i] & lo) << bits));
    }
  }
}

template <int CHUNK>
__device__ __forceinline__ void store_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                            const typename ChunkType<CHUNK>::T& v) {
  if constexpr (CHUNK == 16)
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kNonTemporal);
  else
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kNonTemporal);
}

// Element k of a chunk (ES bytes, zero-extended).
template <int ES, int W>
__device__ __forceinline__ uint32_t element(const uint32_t (&w)[W], int k) {
  constexpr int EPD = 4 / ES;
  const uint32_t word = w[k / EPD];
  return ES == 4 ? word : (word >> (8 * ES * (k % EPD))) & ((1u << (8 * ES)) - 1u);
}

template <int ES>
__device__ __forceinline__ void store_element(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  if constexpr (ES == 4)
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kNonTemporal);
  else if constexpr (ES == 2)
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, (int)off, 0, kNonTemporal);
  else
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, r, (int)off, 0, kNonTemporal);
}

// DIR 0: save (pool -> staging); DIR 1: load (staging -> pool).
template <int CHUNK, int ES, int S, int HU, int DIR>
__global__ __launch_bounds__(kBlockThreads) void tcopy_kernel(const CopyArgs ca) {
  using V = typename ChunkType<CHUNK>::T;
  constexpr int N = CHUNK / ES;       // elements per chunk, either side
  constexpr int W = CHUNK / 4;        // 32-bit words per chunk
  constexpr int PER_PIECE = 8 / ES;   // elements per 8-byte piece
  const BlocksArgs& a = ca.b;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = wave_index();
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n_items = (int64_t)*a.n_items;
  const int lpt = a.caches_per_task;
  const int ngroups = (a.num_caches + lpt - 1) / lpt;
  const int64_t total = n_items * ngroups;
  if (wave >= total) return;

  // Tile table of one element-row group of a (block, head): lane chunk
  // f = lane + 64 s is row j = f mod N of tile t = f / N, and tile t covers
  // element rows [c N, c N + N) x slots [q N, q N + N).  Pool form: element
  // row c N + j of slots q N.. (offset (c N + j) * chunk_stride + q * CHUNK);
  // staging form: elements c N.. of slot q N + j (offset
  // (q N + j) * row_bytes + c N ES).  Tiles are numbered along the side that
  // is stored, so that a store instruction writes long runs: along staging
  // rows for a save (c fastest), along pool element rows for a load (q fastest).
  const int cpe = a.chunks_per_row;  // block_size / N
  const int rge = a.rows_per_group;  // element rows per group, a multiple of N
  const int ctiles = rge / N;        // tile rows of a group
  const int j = lane % N;
  uint32_t prow[S], crow[S], q0[S], poff[S], soff[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int f = lane + kWave * s;
    const int t = f / N;
    const int c = DIR == 0 ? t % ctiles : t / cpe;
    const int q = DIR == 0 ? t / ctiles : t - c * cpe;
    const bool in = f < rge * cpe;
    prow[s] = in ? (uint32_t)(c * N + j) : 0x7fffffffu;  // pool-form element row (in the group)
    crow[s] = in ? (uint32_t)(c * N) : 0x7fffffffu;      // staging-form first element (in the group)
    q0[s] = (uint32_t)(q * N);                            // pool-form first slot
    poff[s] = (uint32_t)((int64_t)(c * N + j) * a.chunk_stride + (int64_t)q * CHUNK);
    soff[s] = (uint32_t)((int64_t)(q * N + j) * a.row_bytes + (int64_t)c * N * ES);
  }
  const int D = a.row_bytes / ES;
  const int ngr = (D + rge - 1) / rge;
  const uint64_t P = (uint64_t)a.pieces;
  const int nhb = (a.heads + HU - 1) / HU;
  const int64_t img_head = (int64_t)ca.block_size * a.row_bytes;

  for (int64_t task = wave; task < total; task += nwaves) {
    const int64_t grp = task / n_items;
    const int64_t item = task - grp * n_items;
    const int c_begin = (int)grp * lpt;
    const int c_end = min(a.num_caches, c_begin + lpt);
    const TaskRecord rec = task_record<false>(a, item, false, lane);
    int32_t v = rec.valid;
    const uint64_t t0 = rec.t0;
    if (item >= ca.staging_positions) {
      if (v > 0 && lane == 0 && ca.error_flags) atomicOr(ca.error_flags, KVCK_FLAG_STAGING_FULL);
      v = 0;
    }
    uint64_t acc = 0;
    if (v > 0) {
      const int64_t blk_off = (int64_t)rec.block * a.block_stride;
      uint8_t* const img0 = ca.staging + (item * ca.num_caches_total + ca.cache_offset) * ca.image_bytes;
      // valid slots of each pool-form chunk and its u before the element's piece
      int nvalid[S];
      uint64_t ubase[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int left = v - (int)q0[s];
        nvalid[s] = left < 0 ? 0 : (left > N ? N : left);
        ubase[s] = 2ull * (t0 + q0[s]) * P + 1ull + a.piece_base;
      }
      const bool straddle = (v % N) != 0;  // some chunk holds the last valid slot and invalid ones
      const int nunits = (c_end - c_begin) * ngr * nhb;
      int cache = c_begin, group = 0, hbatch = 0;
      for (int ui = 0; ui < nunits; ++ui) {
        const int rows = min(rge, D - group * rge);
        const uint8_t* pgroup = a.base[cache] + blk_off + (int64_t)(group * rge) * a.chunk_stride;
        uint8_t* sgroup = img0 + (int64_t)cache * ca.image_bytes + (int64_t)(group * rge) * ES;
        V x[HU][S];
        // loads: pool chunks holding a valid slot (save) or staging rows of valid slots (load)
#pragma unroll
        for (int h = 0; h < HU; ++h) {
          const int hh = hbatch * HU + h;
          const uint32_t hmask = hh < a.heads ? 0u : kOOB;
          if constexpr (DIR == 0) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(pgroup + (int64_t)hh * a.head_stride);
#pragma unroll
            for (int s = 0; s < S; ++s)
              x[h][s] = load_chunk<CHUNK>(rs, ((int)prow[s] < rows && (int)q0[s] < v ? poff[s] : kOOB) | hmask);
          } else {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(sgroup + (int64_t)hh * img_head);
#pragma unroll
            for (int s = 0; s < S; ++s)
              x[h][s] = load_chunk<CHUNK>(rs, ((int)crow[s] < rows && (int)(q0[s] + j) < v ? soff[s] : kOOB) | hmask);
          }
        }
        const uint64_t mb = a.mbase[cache];
#pragma unroll
        for (int h = 0; h < HU; ++h) {
          const int hh = hbatch * HU + h;
          const uint32_t hmask = hh < a.heads ? 0u : kOOB;
          const __amdgpu_buffer_rsrc_t rp = make_rsrc(pgroup + (int64_t)hh * a.head_stride);
          const __amdgpu_buffer_rsrc_t rst = make_rsrc(sgroup + (int64_t)hh * img_head);
          uint64_t sh = 0;
#pragma unroll
          for (int s = 0; s < S; ++s) {
            uint32_t w[W];
#pragma unroll
            for (int i = 0; i < W; ++i) w[i] = x[h][s][i];
            if constexpr (DIR == 1) tile_transpose<ES, W>(w, j);  // staging rows -> pool form
            // checksum of the pool-form chunk: element row d of slots q0.. (masked lanes hold zeros)
            {
              V xv;
#pragma unroll
              for (int i = 0; i < W; ++i) xv[i] = w[i];
              uint64_t E, K;
              chunk_sums<ES>(xv, nvalid[s], E, K);
              const uint32_t d = (uint32_t)(group * rge) + prow[s];
              const uint64_t u0 = ubase[s] + 2ull * (d / PER_PIECE);
              sh += (u0 * E + 2ull * P * K) << (8 * ES * (d % PER_PIECE));
            }
            if constexpr (DIR == 0) {
              tile_transpose<ES, W>(w, j);  // pool form -> staging rows
              V y;
#pragma unroll
              for (int i = 0; i < W; ++i) y[i] = w[i];
              store_chunk<CHUNK>(rst, ((int)crow[s] < rows && (int)(q0[s] + j) < v ? soff[s] : kOOB) | hmask, y);
            } else {
              V y;
#pragma unroll
              for (int i = 0; i < W; ++i) y[i] = w[i];
              const bool row_ok = (int)prow[s] < rows;
              store_chunk<CHUNK>(rp, (row_ok && nvalid[s] == N ? poff[s] : kOOB) | hmask, y);
              if (straddle) {  // uniform: the chunk holding the last valid slot, element by element
                const bool part = row_ok && nvalid[s] > 0 && nvalid[s] < N;
#pragma unroll
                for (int k = 0; k < N - 1; ++k)
                  store_element<ES>(rp, (part && k < nvalid[s] ? poff[s] + (uint32_t)(k * ES) : kOOB) | hmask,
                                    element<ES, W>(w, k));
              }
            }
          }
          acc += sh * (mb + 2ull * (uint64_t)hh);
        }
        if (++hbatch == nhb) {
          hbatch = 0;
          if (++group == ngr) {
            group = 0;
            ++cache;
          }
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
  }
}

// The same copy with the transpose staged through LDS (the choice whenever
// chunks are 16 bytes): the register transpose leaves the side that is not
// stored touching one 16-byte piece of each of many lines per instruction,
// more of them as block_size grows.
// Here both sides move whole contiguous chunks: pool chunks in pool order
// (element row by element row), staging chunks in staging order (slot by
// slot), and each wave's LDS region holds the group's image in staging form,
// [slot][element], a row of pitch bytes.  Pool chunks go in and out element
// by element.  The 16-byte columns of slot s are XOR-swizzled by
// (s / N) * nd mod 2^k (nd: the columns one instruction's element rows span;
// 2^k: the largest power of two dividing the row's column count), so the
// slot groups one instruction writes or reads land in different banks.
template <int ES>
__device__ __forceinline__ void lds_store_element(uint8_t* lds, uint32_t addr, uint32_t v) {
  if constexpr (ES == 4)
    *reinterpret_cast<uint32_t*>(lds + addr) = v;
  else if constexpr (ES == 2)
    *reinterpret_cast<uint16_t*>(lds + addr) = (uint16_t)v;
  else
    lds[addr] = (uint8_t)v;
}

template <int ES>
__device__ __forceinline__ uint32_t lds_load_element(const uint8_t* lds, uint32_t addr) {
  if constexpr (ES == 4)
    return *reinterpret_cast<const uint32_t*>(lds + addr);
  else if constexpr (ES == 2)
    return *reinterpret_cast<const uint16_t*>(lds + addr);
  else
    return lds[addr];
}

extern __shared__ __attribute__((aligned(16))) uint8_t tcopy_lds[];

// Row pitch of a wave's LDS region (one row per slot, block_size rows): the
// group's elements rounded up to whole 16-byte columns.
__host__ __device__ inline int64_t tcopy_lds_pitch(int32_t rows_per_group, int es) {
  return ((int64_t)rows_per_group * es + 15) / 16 * 16;
}

// DIR 0: save (pool -> staging); DIR 1: load (staging -> pool).  16-byte chunks.
template <int ES, int S, int DIR>
__global__ __launch_bounds__(kBlockThreads) void tcopy_lds_kernel(const CopyArgs ca) {
  using V = typename ChunkType<16>::T;
  constexpr int N = 16 / ES;
  constexpr int EPD = 4 / ES;
  constexpr int PER_PIECE = 8 / ES;
  const BlocksArgs& a = ca.b;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = wave_index();
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n_items = (int64_t)*a.n_items;
  const int lpt = a.caches_per_task;
  const int ngroups = (a.num_caches + lpt - 1) / lpt;
  const int64_t total = n_items * ngroups;
  if (wave >= total) return;

  const int bs = ca.block_size;
  const int cpe = a.chunks_per_row;  // pool chunks per element row: block_size / N
  const int rge = a.rows_per_group;  // element rows per group, a multiple of N
  const uint32_t pitch = (uint32_t)tcopy_lds_pitch(rge, ES);
  const uint32_t cols = pitch / 16;
  const uint32_t kmask = (cols & (0u - cols)) - 1u;
  const uint32_t nd = (uint32_t)max(1, kWave / cpe * ES / 16);  // columns of one instruction's element rows
  uint8_t* const lds = tcopy_lds + wave_in_block() * (int64_t)bs * pitch;
  const int cps = rge * ES / 16;     // staging chunks of a slot's row segment (full group)

  // pool side: chunk f is element row d = f / cpe, slots q N.. (q = f mod cpe)
  // staging side: chunk f is column c = f mod cps of slot sl = f / cps
  int prow[S], srow[S], q0[S], scol[S];
  uint32_t poff[S], soff[S], lpool[S], lstg[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int f = lane + kWave * s;
    const bool pin = f < rge * cpe;
    const int d = f / cpe, q = f - (f / cpe) * cpe;
    prow[s] = pin ? d : 0x7fffffff;
    q0[s] = q * N;
    poff[s] = (uint32_t)((int64_t)d * a.chunk_stride + (int64_t)q * 16);
    const uint32_t dcol = (uint32_t)(d * ES);
    lpool[s] = (uint32_t)(q * N) * pitch + ((((dcol >> 4) ^ (((uint32_t)q * nd) & kmask)) << 4) | (dcol & 15u));
    const bool sin = f < bs * cps;
    const int sl = f / cps, c = f - (f / cps) * cps;
    srow[s] = sin ? sl : 0x7fffffff;
    scol[s] = c;
    soff[s] = (uint32_t)((int64_t)sl * a.row_bytes + (int64_t)c * 16);
    lstg[s] = (uint32_t)sl * pitch + ((((uint32_t)c) ^ ((((uint32_t)sl / N) * nd) & kmask)) << 4);
  }
  const int D = a.row_bytes / ES;
  const int ngr = (D + rge - 1) / rge;
  const uint64_t P = (uint64_t)a.pieces;
  const int64_t img_head = (int64_t)bs * a.row_bytes;

  for (int64_t task = wave; task < total; task += nwaves) {
    const int64_t grp = task / n_items;
    const int64_t item = task - grp * n_items;
    const int c_begin = (int)grp * lpt;
    const int c_end = min(a.num_caches, c_begin + lpt);
    const TaskRecord rec = task_record<false>(a, item, false, lane);
    int32_t v = rec.valid;
    const uint64_t t0 = rec.t0;
    if (item >= ca.staging_positions) {
      if (v > 0 && lane == 0 && ca.error_flags) atomicOr(ca.error_flags, KVCK_FLAG_STAGING_FULL);
      v = 0;
    }
    uint64_t acc = 0;
    if (v > 0) {
      const int64_t blk_off = (int64_t)rec.block * a.block_stride;
      uint8_t* const img0 = ca.staging + (item * ca.num_caches_total + ca.cache_offset) * ca.image_bytes;
      int nvalid[S];
      uint64_t ubase[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int left = v - q0[s];
        nvalid[s] = left < 0 ? 0 : (left > N ? N : left);
        ubase[s] = 2ull * (t0 + (uint64_t)q0[s]) * P + 1ull + a.piece_base;
      }
      const bool straddle = (v % N) != 0;
      const int nunits = (c_end - c_begin) * ngr * a.heads;
      // units: (cache, element-row group, head), cache-major
      struct Cursor {
        int cache, group, hh;
        __device__ __forceinline__ void next(int heads, int ngr_) {
          if (++hh == heads) {
            hh = 0;
            if (++group == ngr_) {
              group = 0;
              ++cache;
            }
          }
        }
      };
      Cursor ic{c_begin, 0, 0}, cc{c_begin, 0, 0};
      auto pool_rsrc = [&](const Cursor& u) {
        return make_rsrc(a.base[u.cache] + blk_off + (int64_t)(u.group * rge) * a.chunk_stride +
                         (int64_t)u.hh * a.head_stride);
      };
      auto stg_rsrc = [&](const Cursor& u) {
        return make_rsrc(img0 + (int64_t)u.cache * ca.image_bytes + (int64_t)u.hh * img_head +
                         (int64_t)(u.group * rge) * ES);
      };
      // `live` false: a unit past the task's last one, every load out of range
      auto issue = [&](V(&x)[S], bool live) {
        Cursor u = ic;
        if (!live) u.cache = c_begin;
        const int rows = live ? min(rge, D - u.group * rge) : 0;
        if constexpr (DIR == 0) {
          const __amdgpu_buffer_rsrc_t rp = pool_rsrc(u);
#pragma unroll
          for (int s = 0; s < S; ++s) x[s] = load_chunk<16>(rp, prow[s] < rows && q0[s] < v ? poff[s] : kOOB);
        } else {
          const int seg = rows * ES / 16;  // staging chunks of this group's row segment
          const __amdgpu_buffer_rsrc_t rst = stg_rsrc(u);
#pragma unroll
          for (int s = 0; s < S; ++s) x[s] = load_chunk<16>(rst, srow[s] < v && scol[s] < seg ? soff[s] : kOOB);
        }
        if (live) ic.next(a.heads, ngr);
      };
      auto process = [&](const V(&x)[S]) {
        const int rows = min(rge, D - cc.group * rge);
        const int seg = rows * ES / 16;
        const __amdgpu_buffer_rsrc_t rp = pool_rsrc(cc);
        const __amdgpu_buffer_rsrc_t rst = stg_rsrc(cc);
        uint64_t sh = 0;
        if constexpr (DIR == 0) {
          // checksum of each pool chunk, then its elements into the staging form
#pragma unroll
          for (int s = 0; s < S; ++s) {
            uint64_t E, K;
            chunk_sums<ES>(x[s], nvalid[s], E, K);
            const uint32_t d = (uint32_t)(cc.group * rge) + (uint32_t)prow[s];
            sh += ((ubase[s] + 2ull * (d / PER_PIECE)) * E + 2ull * P * K) << (8 * ES * (d % PER_PIECE));
            if (prow[s] < rge) {
#pragma unroll
              for (int k = 0; k < N; ++k)
                lds_store_element<ES>(lds, lpool[s] + (uint32_t)k * pitch,
                                      ES == 4 ? x[s][k] : (x[s][k / EPD] >> (8 * ES * (k % EPD))));
            }
          }
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int s = 0; s < S; ++s) {
            V y = srow[s] < bs ? *reinterpret_cast<const V*>(lds + lstg[s]) : V(0);
            store_chunk<16>(rst, srow[s] < v && scol[s] < seg ? soff[s] : kOOB, y);
          }
          __builtin_amdgcn_wave_barrier();
        } else {
          // staging rows into the staging form, then pool chunks gathered element by element
#pragma unroll
          for (int s = 0; s < S; ++s)
            if (srow[s] < bs) *reinterpret_cast<V*>(lds + lstg[s]) = x[s];
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int s = 0; s < S; ++s) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (prow[s] < rge) {
#pragma unroll
              for (int k = 0; k < N; ++k)
                w[k / EPD] |= lds_load_element<ES>(lds, lpool[s] + (uint32_t)k * pitch) << (8 * ES * (k % EPD));
            }
            V xv;
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = w[i];
            uint64_t E, K;
            chunk_sums<ES>(xv, nvalid[s], E, K);
            const uint32_t d = (uint32_t)(cc.group * rge) + (uint32_t)prow[s];
            sh += ((ubase[s] + 2ull * (d / PER_PIECE)) * E + 2ull * P * K) << (8 * ES * (d % PER_PIECE));
            const bool row_ok = prow[s] < rows;
            store_chunk<16>(rp, row_ok && nvalid[s] == N ? poff[s] : kOOB, xv);
            if (straddle) {  // uniform: the chunk holding the last valid slot, element by element
              const bool part = row_ok && nvalid[s] > 0 && nvalid[s] < N;
#pragma unroll
              for (int k = 0; k < N - 1; ++k)
                store_element<ES>(rp, part && k < nvalid[s] ? poff[s] + (uint32_t)(k * ES) : kOOB,
                                  element<ES, 4>(w, k));
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
        acc += sh * (a.mbase[cc.cache] + 2ull * (uint64_t)cc.hh);
        cc.next(a.heads, ngr);
      };
      // Two unit buffers: the loads of the next unit are in flight while this
      // one goes through LDS.  Both are issued at every step (past the last
      // unit with every load out of range) and order_after keeps a buffer's
      // reload after the last use of its data, as in the checksum kernel.
      V A[S], B[S];
      issue(A, true);
      for (int ui = 0; ui < nunits; ui += 2) {
        issue(B, ui + 1 < nunits);
        process(A);
        order_after(acc);
        issue(A, ui + 2 < nunits);
        if (ui + 1 < nunits) process(B);
        order_after(acc);
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
  }
}

using TCopyFn = void (*)(const CopyArgs);

template <int CHUNK, int ES, int DIR>
TCopyFn tcopy_slots(int slots) {
  switch (slots) {
    case 1: return &tcopy_kernel<CHUNK, ES, 1, 8, DIR>;
    case 2: return &tcopy_kernel<CHUNK, ES, 2, 4, DIR>;
    case 4: return &tcopy_kernel<CHUNK, ES, 4, 2, DIR>;
    case 8: return &tcopy_kernel<CHUNK, ES, 8, 1, DIR>;
    case 16: return &tcopy_kernel<CHUNK, ES, 16, 1, DIR>;
  }
  return nullptr;
}

template <int ES, int DIR>
TCopyFn tcopy_lds_slots(int slots) {
  switch (slots) {
    case 1: return &tcopy_lds_kernel<ES, 1, DIR>;
    case 2: return &tcopy_lds_kernel<ES, 2, DIR>;
    case 4: return &tcopy_lds_kernel<ES, 4, DIR>;
    case 8: return &tcopy_lds_kernel<ES, 8, DIR>;
  }
  return nullptr;
}

template <int DIR>
TCopyFn tcopy_dir(const BlocksShape& shp) {
  if (shp.lds_transpose) {
    if (shp.chunk != 16) return nullptr;
    switch (shp.elem_bytes) {
      case 1: return tcopy_lds_slots<1, DIR>(shp.slots);
      case 2: return tcopy_lds_slots<2, DIR>(shp.slots);
      case 4: return tcopy_lds_slots<4, DIR>(shp.slots);
    }
    return nullptr;
  }
  if (shp.chunk == 16) {
    switch (shp.elem_bytes) {
      case 1: return tcopy_slots<16, 1, DIR>(shp.slots);
      case 2: return tcopy_slots<16, 2, DIR>(shp.slots);
      case 4: return tcopy_slots<16, 4, DIR>(shp.slots);
    }
  } else {
    switch (shp.elem_bytes) {
      case 1: return tcopy_slots<8, 1, DIR>(shp.slots);
      case 2: return tcopy_slots<8, 2, DIR>(shp.slots);
      case 4: return tcopy_slots<8, 4, DIR>(shp.slots);
    }
  }
  return nullptr;
}

TCopyFn tcopy_fn(const BlocksShape& shp, int direction) {
  return direction == KVCK_COPY_SAVE ? tcopy_dir<0>(shp) : tcopy_dir<1>(shp);
}

// Dynamic LDS of one workgroup of the LDS variant: a region per wave.
size_t tcopy_lds_bytes(const BlocksShape& shp, int32_t block_size) {
  return shp.lds_transpose ? (size_t)(kBlockThreads / kWave) * (size_t)block_size *
                                 (size_t)tcopy_lds_pitch(shp.rows_per_group, shp.elem_bytes)
                           : 0;
}

}  // namespace

int tcopy_grid(const BlocksShape& shp, int direction, int device, int64_t max_tasks, int32_t block_size) {
  TCopyFn fn = tcopy_fn(shp, direction);
  int per_cu = fn ? kernel_occupancy(reinterpret_cast<const void*>(fn), device, 1) : 1;
  const size_t lds = tcopy_lds_bytes(shp, block_size);
  if (lds > 0) {
    // the occupancy query counts no dynamic LDS: bound it by the CU's LDS
    int per_cu_lds = 0;
    if (hipDeviceGetAttribute(&per_cu_lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) != hipSuccess ||
        per_cu_lds <= 0)
      per_cu_lds = 64 * 1024;
    const int by_lds = (int)((size_t)per_cu_lds / lds);
    per_cu = by_lds < 1 ? 1 : (by_lds < per_cu ? by_lds : per_cu);
  }
  per_cu = workgroups_per_cu(per_cu, kAllThatFit);
  const int64_t waves_per_block = kBlockThreads / kWave;
  const int64_t need = (max_tasks + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)per_cu * device_cus(device);
  return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

hipError_t launch_tcopy(const CopyArgs& a, const BlocksShape& shp, int direction, int grid, hipStream_t stream) {
  TCopyFn fn = tcopy_fn(shp, direction);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<CopyArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(kBlockThreads), args,
                         tcopy_lds_bytes(shp, a.block_size), stream);
}

}  // namespace kvck

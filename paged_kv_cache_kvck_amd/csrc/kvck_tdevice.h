// Device helpers of the element-transposed kernels (checksum pass and fused
// copy): per-chunk element sums.  Not part of the ABI.
#pragma once

#include "kvck_device.h"

namespace kvck {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// E and K of one chunk: sums of its elements and of k * element over the first
// `valid` of its N = CHUNK/ES slots (elements read unsigned).  Each word is
// masked to its valid elements, then 2-byte elements go through the packed
// u16 dot product and 1-byte elements through the u8 one (E with weights 1,
// K with weights k); sums stay below 2^32 (at most 16 elements of 16 bits).
template <int ES, typename V>
__device__ __forceinline__ void chunk_sums(const V& x, int valid, uint64_t& E, uint64_t& K) {
  constexpr int WORDS = sizeof(V) / 4;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&x);
  if constexpr (ES == 4) {
    uint64_t e = 0, k = 0;
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      const uint64_t v = i < valid ? (uint64_t)w[i] : 0ull;
      e += v;
      k += (uint64_t)i * v;
    }
    E = e;
    K = k;
  } else if constexpr (ES == 2) {
    uint32_t e = 0, k = 0;
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      const int m = valid - 2 * i;  // valid elements of this word, clamped below
      const uint32_t mask = m >= 2 ? 0xffffffffu : (m == 1 ? 0x0000ffffu : 0u);
      const u16x2 v = __builtin_bit_cast(u16x2, w[i] & mask);
      e = __builtin_amdgcn_udot2(v, u16x2{1, 1}, e, false);
      k = __builtin_amdgcn_udot2(v, u16x2{(uint16_t)(2 * i), (uint16_t)(2 * i + 1)}, k, false);
    }
    E = e;
    K = k;
  } else {
    uint32_t e = 0, k = 0;
#pragma unroll
    for (int i = 0; i < WORDS; ++i) {
      const int m = valid - 4 * i;
      const uint32_t mask = m >= 4 ? 0xffffffffu : (m <= 0 ? 0u : (1u << (8 * m)) - 1u);
      const uint32_t v = w[i] & mask;
      const uint32_t kw = (uint32_t)(4 * i) | ((uint32_t)(4 * i + 1) << 8) | ((uint32_t)(4 * i + 2) << 16) |
                          ((uint32_t)(4 * i + 3) << 24);
      e = __builtin_amdgcn_udot4(v, 0x01010101u, e, false);
      k = __builtin_amdgcn_udot4(v, kw, k, false);
    }
    E = e;
    K = k;
  }
}

}  // namespace kvck

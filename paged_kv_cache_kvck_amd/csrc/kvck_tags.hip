// Offloaded-checksum tags and load-time comparison on gfx950.
//
// vLLM API page "vllm.distributed.kv_transfer.kv_checksum.checksum", function
// block_checksum_tags: a block's tag is the little-endian value of its hash's
// leading 8 bytes, XOR the group's fingerprint; XOR-ing an offloaded checksum
// (one uint64 per block, BLOCK_CHECKSUM_BYTES) with it ties that checksum to
// its own block hash and group of layers.  The value offloaded with a block
// is its row of partial checksums summed (class KVChecksumGroup, field
// stored), the row holding one column per replica key.  Here, per listed
// position i with columns c:
//   t_i = (sum_c checksum_{i,c}) ^ LE64(hash_i[0..8)) ^ fingerprint
// is written (the value to offload) and/or compared with the stored value
// (a load of offloaded KV), mismatches flagged per position and counted.
#include "kvck_device.h"

namespace kvck {
namespace {

__global__ __launch_bounds__(256) void tags_kernel(const uint64_t* __restrict__ checksums, int32_t columns,
                                                   const uint8_t* __restrict__ hashes, int64_t hash_stride,
                                                   uint64_t fingerprint, int64_t n, const int32_t* __restrict__ nbpr,
                                                   const int64_t* __restrict__ start_pos, int32_t max_blocks,
                                                   int64_t max_start, uint64_t* __restrict__ tagged,
                                                   const uint64_t* __restrict__ stored, uint8_t* __restrict__ mismatch,
                                                   uint32_t* __restrict__ count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < n; base += stride) {
    const int64_t i = base + threadIdx.x;
    bool live = i < n;
    if (live && nbpr) {
      // the checksum pass's rule: a bad request lists nothing (its entries
      // were never written, so they are neither tagged nor compared)
      const int64_t r = i / max_blocks;
      const int32_t nr = nbpr[r];
      live = !bad_request(nr, start_pos ? start_pos[r] : 0, max_blocks, max_start) &&
             (int32_t)(i - r * max_blocks) < nr;
    }
    bool bad = false;
    if (live) {
      // little-endian hosts and devices: a 64-bit load is the LE value of the 8 bytes
      const uint64_t tag = *reinterpret_cast<const uint64_t*>(hashes + i * hash_stride) ^ fingerprint;
      uint64_t c = 0;
      for (int32_t k = 0; k < columns; ++k) c += checksums[i * columns + k];
      const uint64_t t = c ^ tag;
      if (tagged) tagged[i] = t;
      if (stored) {
        bad = t != stored[i];
        if (mismatch) mismatch[i] = bad ? 1 : 0;
      }
    }
    if (count) {
      // one atomic per wavefront
      const uint64_t votes = __ballot(bad);
      if ((threadIdx.x & (kWave - 1)) == 0 && votes) atomicAdd(count, (uint32_t)__popcll(votes));
    }
  }
}

}  // namespace

hipError_t launch_tags(const uint64_t* checksums, int32_t columns, const uint8_t* hashes, int64_t hash_stride,
                       uint64_t fingerprint, int64_t n, const int32_t* nbpr, const int64_t* start_pos, int32_t max_blocks,
                       int64_t max_start, uint64_t* tagged, const uint64_t* stored, uint8_t* mismatch,
                       uint32_t* count, hipStream_t stream) {
  int64_t grid = (n + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(tags_kernel, dim3((unsigned)grid), dim3(256), 0, stream, checksums, columns, hashes, hash_stride,
                     fingerprint, n, nbpr, start_pos, max_blocks, max_start, tagged, stored, mismatch, count);
  return hipGetLastError();
}

}  // namespace kvck

/*
 * libkvck from plain C: no Python, no torch -- the HIP runtime for device
 * memory and the C ABI of include/kvck.h for the checksums.
 *
 *   paged_kv_cache_kvck_amd/kvck_demo          (built by paged_kv_cache_kvck_amd.build)
 *
 * Three layers (numbers 0, 7, 31) of an NHD pool (2, 24 blocks, 16 slots,
 * 4 heads, head 64, 2-byte elements) whose bytes come from splitmix64 (the
 * published generator of Steele, Lea and Flood: state += 0x9E3779B97F4A7C15,
 * then two xor-shift-multiply rounds), seeded 1000 + layer index, each 64-bit
 * output giving 8 bytes little-endian.  Three requests on a fixed block table.
 * Prints one line per listed position, "full <r> <k> <checksum>", then the
 * same for the TP shard of heads 1..2 numbered globally from 1 ("shard ...").
 * Exit status: 0 on success, 2 when no gfx950 device is present, 1 on any
 * other error.
 *
 *   kvck_demo --stream SEED N    prints the first N splitmix64 outputs of SEED
 *                                in hex and touches no device.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvck.h"

enum { LAYERS = 3, NB = 24, BS = 16, NH = 4, D = 64, ES = 2, R = 3, MAXB = 4 };

static uint64_t splitmix64(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

#define HIP_OK(x)                                                           \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                             \
    }                                                                       \
  } while (0)

static int run(const kvck_kv_layout* L, void* const* pools, const int32_t* layers, const int32_t* bases,
               int32_t head_begin, int32_t head_count, const int32_t* d_table, const int32_t* d_nb,
               const int64_t* d_start, const int64_t* d_tokens, uint64_t* d_out, void* d_ws, size_t ws_bytes,
               uint32_t* d_flags, const int32_t* nb, const char* tag) {
  uint64_t out[R * MAXB];
  uint32_t flags = 0;
  HIP_OK(hipMemset(d_flags, 0, sizeof(uint32_t)));
  kvck_status st = kvck_checksum_blocks(L, (const void* const*)pools, layers, bases, LAYERS, head_begin, head_count,
                                        d_table, MAXB, d_nb, d_start, d_tokens, R, MAXB, d_out, 1, 0, d_ws, ws_bytes,
                                        d_flags, NULL);
  if (st != KVCK_OK) {
    fprintf(stderr, "kvck_checksum_blocks: %s\n", kvck_status_string(st));
    return st == KVCK_ERR_NO_DEVICE ? 2 : 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, d_out, sizeof(out), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&flags, d_flags, sizeof(flags), hipMemcpyDeviceToHost));
  if (flags) {
    fprintf(stderr, "device flags 0x%x\n", flags);
    return 1;
  }
  for (int r = 0; r < R; ++r)
    for (int k = 0; k < nb[r]; ++k) printf("%s %d %d %llu\n", tag, r, k, (unsigned long long)out[r * MAXB + k]);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 4 && strcmp(argv[1], "--stream") == 0) {
    uint64_t state = strtoull(argv[2], NULL, 0);
    const long n = strtol(argv[3], NULL, 0);
    for (long i = 0; i < n; ++i) printf("%016llx\n", (unsigned long long)splitmix64(&state));
    return 0;
  }
  if (!kvck_platform_supported()) {
    fprintf(stderr, "no gfx950 device: %s\n", kvck_status_string(KVCK_ERR_NO_DEVICE));
    return 2;
  }
  const size_t pool_bytes = (size_t)2 * NB * BS * NH * D * ES;
  const int32_t layers[LAYERS] = {0, 7, 31};
  const int32_t bases_full[LAYERS] = {0, 0, 0};
  const int32_t bases_shard[LAYERS] = {1, 1, 1};
  const int32_t table[R * MAXB] = {5, 17, 2, 9, 11, 0, -1, -1, 21, 3, 14, -1};
  const int32_t nb[R] = {4, 2, 3};
  const int64_t start[R] = {0, 1, 0};
  const int64_t tokens[R] = {50, 40, 33};

  void* pools[LAYERS];
  uint8_t* host = (uint8_t*)malloc(pool_bytes);
  if (!host) return 1;
  for (int l = 0; l < LAYERS; ++l) {
    uint64_t state = 1000u + (uint64_t)l;
    for (size_t i = 0; i < pool_bytes; i += 8) {
      const uint64_t v = splitmix64(&state);
      for (int b = 0; b < 8; ++b) host[i + b] = (uint8_t)(v >> (8 * b));
    }
    HIP_OK(hipMalloc(&pools[l], pool_bytes));
    HIP_OK(hipMemcpy(pools[l], host, pool_bytes, hipMemcpyHostToDevice));
  }
  free(host);

  /* NHD: (2, NB, BS, NH, D) contiguous */
  kvck_kv_layout L;
  memset(&L, 0, sizeof(L));
  L.planes = 2;
  L.block_size = BS;
  L.num_heads = NH;
  L.row_bytes = D * ES;
  L.num_blocks = NB;
  L.head_stride = (int64_t)D * ES;
  L.slot_stride = L.head_stride * NH;
  L.block_stride = L.slot_stride * BS;
  L.plane_stride = L.block_stride * NB;

  int32_t *d_table, *d_nb;
  int64_t *d_start, *d_tokens;
  uint64_t* d_out;
  uint32_t* d_flags;
  void* d_ws;
  const size_t ws_bytes = kvck_blocks_workspace_bytes(LAYERS, R, MAXB);
  HIP_OK(hipMalloc((void**)&d_table, sizeof(table)));
  HIP_OK(hipMalloc((void**)&d_nb, sizeof(nb)));
  HIP_OK(hipMalloc((void**)&d_start, sizeof(start)));
  HIP_OK(hipMalloc((void**)&d_tokens, sizeof(tokens)));
  HIP_OK(hipMalloc((void**)&d_out, sizeof(uint64_t) * R * MAXB));
  HIP_OK(hipMalloc((void**)&d_flags, sizeof(uint32_t)));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMemcpy(d_table, table, sizeof(table), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_nb, nb, sizeof(nb), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_start, start, sizeof(start), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_tokens, tokens, sizeof(tokens), hipMemcpyHostToDevice));

  int rc = run(&L, pools, layers, bases_full, 0, NH, d_table, d_nb, d_start, d_tokens, d_out, d_ws, ws_bytes,
               d_flags, nb, "full");
  if (rc == 0)
    rc = run(&L, pools, layers, bases_shard, 1, 2, d_table, d_nb, d_start, d_tokens, d_out, d_ws, ws_bytes,
             d_flags, nb, "shard");

  for (int l = 0; l < LAYERS; ++l) (void)hipFree(pools[l]);
  (void)hipFree(d_table);
  (void)hipFree(d_nb);
  (void)hipFree(d_start);
  (void)hipFree(d_tokens);
  (void)hipFree(d_out);
  (void)hipFree(d_flags);
  (void)hipFree(d_ws);
  return rc;
}

// Plain streaming read of one large buffer: the HBM read bandwidth a trivial
// kernel reaches on this GPU, as context for the checksum main pass (which
// reads the same kind of bytes but through a block table).
//
//   paged_kv_cache_kvck_amd/hbm_read_probe [GiB]      (default 64)
//
// Each thread reads 16-byte chunks i, i+T, i+2T, .. (T = total threads) of the
// buffer with U independent loads in flight and XORs them (nothing is written
// unless the XOR hits a magic value), for several grid sizes, U and load kinds.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);        \
      std::exit(1);                                                                     \
    }                                                                                   \
  } while (0)

template <int U, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t n, uint32_t* out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 x = p[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

template <int U, bool NT>
void run(const u32x4* p, size_t n, uint32_t* out, int grid) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  for (int w = 0; w < 2; ++w) read_kernel<U, NT><<<grid, 256>>>(p, n, out);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  const int iters = 10;
  CHECK(hipEventRecord(a));
  for (int w = 0; w < iters; ++w) read_kernel<U, NT><<<grid, 256>>>(p, n, out);
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  std::printf("%-12s U=%2d grid=%6d : %8.1f GB/s\n", NT ? "non-temporal" : "plain", U, grid,
              (double)n * 16.0 * iters / (ms * 1e-3) / 1e9);
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
}

int main(int argc, char** argv) {
  const double gib = argc > 1 ? std::atof(argv[1]) : 64.0;
  const size_t bytes = (size_t)(gib * (double)(1ull << 30)) / 16 * 16;
  const size_t n = bytes / 16;
  u32x4* p = nullptr;
  uint32_t* out = nullptr;
  CHECK(hipMalloc(&p, bytes));
  CHECK(hipMalloc(&out, 4));
  CHECK(hipMemset(p, 1, bytes));
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  std::printf("buffer %.1f GiB, %d CUs\n", gib, cus);
  for (int m : {4, 8, 16, 32}) {
    run<8, true>(p, n, out, cus * m);
    run<16, true>(p, n, out, cus * m);
    run<16, false>(p, n, out, cus * m);
  }
  CHECK(hipFree(p));
  CHECK(hipFree(out));
  return 0;
}

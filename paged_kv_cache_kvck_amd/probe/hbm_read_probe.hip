// HBM read ceilings on this GPU, as context for the checksum main pass (which
// reads every valid cache byte once, through a block table).
//
//   paged_kv_cache_kvck_amd/hbm_read_probe [GiB]      (default 64)
//
// Access shapes over one large buffer (the read shapes write nothing unless an
// XOR of the data hits a magic value):
//   * grid-stride: thread i reads 16-byte chunks i, i+T, i+2T, .. (T = total
//     threads), U loads in flight, plain or non-temporal loads;
//   * runs: each wavefront reads whole contiguous runs of R bytes (R = 8, 32 or
//     64 KiB: one, four or eight 16-slot KV blocks of one head) with 16
//     non-temporal 1 KiB buffer loads per batch, the runs taken in address
//     order or in a scrambled order (odd multiplier modulo a power of two: a
//     permutation), which is the shape of a paged cache walked through a block
//     table.  "pipelined" keeps a second batch in flight while the first is used
//     (one or two workgroups per CU);
//   * copy: one half of the buffer to the other (read + write), by a streaming
//     kernel and by the runtime's device-to-device copy.
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

constexpr uint32_t kMagic = 0x9E3779B9u;

template <int U, bool NT>
__global__ __launch_bounds__(256) void stride_kernel(const u32x4* __restrict__ p, size_t n, uint32_t* out) {
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
  if (acc == kMagic) out[0] = acc;
}

// One wavefront per run.  Run r of nruns (a power of two) starts at byte
// r' * run, r' = r or (r * odd) mod nruns.  A batch is 16 loads of 64 lanes x
// 16 bytes; loads past the end of the run get an out-of-range buffer offset and
// read zeros.
template <bool SCRAMBLE, bool PIPE>
__global__ __launch_bounds__(256) void runs_kernel(const uint8_t* __restrict__ p, uint64_t nruns, uint32_t run,
                                                   uint32_t* out) {
  constexpr uint32_t kBatch = 16 * 1024;
  constexpr uint32_t kOutside = 0x80000000u;
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t wave = (uint64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t nwaves = (uint64_t)gridDim.x * 4;
  const int batches = (int)((run + kBatch - 1) / kBatch);
  uint32_t acc = 0;
  for (uint64_t r = wave; r < nruns; r += nwaves) {
    const uint64_t rr = SCRAMBLE ? ((r * 0x9E3779B97F4A7C15ull) & (nruns - 1)) : r;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p + rr * run), (short)0, 0x80000000, 0x00020000);
    u32x4 a[16], b[16];
    auto issue = [&](u32x4(&x)[16], int k) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t o = (uint32_t)k * kBatch + (uint32_t)i * 1024u;
        x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, o < run ? o + lane * 16u : kOutside, 0, 2);
      }
    };
    auto use = [&](const u32x4(&x)[16]) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc ^= x[i].x ^ x[i].y ^ x[i].z ^ x[i].w;
    };
    if constexpr (PIPE) {
      // both buffers issued at every step (batches past the run read nothing),
      // the empty asm keeps a buffer's reload after its last use: the waits
      // for one buffer leave the other's loads in flight
      issue(a, 0);
      for (int k = 0; k < batches; k += 2) {
        issue(b, k + 1);
        use(a);
        asm volatile("" ::"v"(acc) : "memory");
        issue(a, k + 2);
        use(b);
        asm volatile("" ::"v"(acc) : "memory");
      }
    } else {
      for (int k = 0; k < batches; ++k) {
        issue(a, k);
        use(a);
      }
    }
  }
  if (acc == kMagic) out[0] = acc;
}

// Streaming copy: thread i moves 16-byte chunks i, i+T, .. of src to dst with
// U loads in flight; non-temporal loads and stores.  The ceiling for a kernel
// that reads every byte once and writes it once (a fused copy).
template <int U>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

struct Timer {
  hipEvent_t a, b;
  Timer() {
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
  }
  ~Timer() {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
  }
};

template <class Launch>
double time_gbs(Launch launch, double bytes) {
  Timer t;
  for (int w = 0; w < 2; ++w) launch();
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  const int iters = 8;
  CHECK(hipEventRecord(t.a));
  for (int w = 0; w < iters; ++w) launch();
  CHECK(hipEventRecord(t.b));
  CHECK(hipEventSynchronize(t.b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, t.a, t.b));
  return bytes * iters / (ms * 1e-3) / 1e9;
}

int main(int argc, char** argv) {
  const double gib = argc > 1 ? std::atof(argv[1]) : 64.0;
  const size_t bytes = (size_t)(gib * (double)(1ull << 30)) / 65536 * 65536;
  if (bytes < 65536) {
    std::printf("buffer too small\n");
    return 1;
  }
  const size_t n = bytes / 16;
  uint8_t* p = nullptr;
  uint32_t* out = nullptr;
  CHECK(hipMalloc(&p, bytes));
  CHECK(hipMalloc(&out, 4));
  CHECK(hipMemset(p, 1, bytes));
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  std::printf("buffer %.1f GiB, %d CUs\n", bytes / (double)(1ull << 30), cus);
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  for (int m : {4, 16}) {
    const int grid = cus * m;
    std::printf("grid-stride non-temporal U= 8 grid=%6d : %8.1f GB/s\n", grid,
                time_gbs([&] { stride_kernel<8, true><<<grid, 256>>>(q, n, out); }, (double)bytes));
    std::printf("grid-stride non-temporal U=16 grid=%6d : %8.1f GB/s\n", grid,
                time_gbs([&] { stride_kernel<16, true><<<grid, 256>>>(q, n, out); }, (double)bytes));
    std::printf("grid-stride plain        U=16 grid=%6d : %8.1f GB/s\n", grid,
                time_gbs([&] { stride_kernel<16, false><<<grid, 256>>>(q, n, out); }, (double)bytes));
  }
  for (uint32_t run_kib : {8u, 32u, 64u}) {
    const uint32_t run = run_kib * 1024u;
    uint64_t nruns = 1;
    while (nruns * 2 * run <= bytes) nruns *= 2;   // power of two: the scramble is a permutation
    const double rb = (double)nruns * run;
    const int grid = cus * 4;
    std::printf("runs %2u KiB in order             grid=%6d : %8.1f GB/s\n", run_kib, grid,
                time_gbs([&] { runs_kernel<false, false><<<grid, 256>>>(p, nruns, run, out); }, rb));
    std::printf("runs %2u KiB scrambled            grid=%6d : %8.1f GB/s\n", run_kib, grid,
                time_gbs([&] { runs_kernel<true, false><<<grid, 256>>>(p, nruns, run, out); }, rb));
    for (int per_cu : {1, 2})
      std::printf("runs %2u KiB scrambled, pipelined grid=%6d : %8.1f GB/s\n", run_kib, cus * per_cu,
                  time_gbs([&] { runs_kernel<true, true><<<cus * per_cu, 256>>>(p, nruns, run, out); }, rb));
  }
  // copies between the two halves of the buffer (bytes read + bytes written)
  const size_t half = bytes / 2 / 16 * 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(p);
  u32x4* dst = reinterpret_cast<u32x4*>(p + half);
  for (int m : {4, 16}) {
    const int grid = cus * m;
    std::printf("copy kernel non-temporal U= 8 grid=%6d : %8.1f GB/s read+write\n", grid,
                time_gbs([&] { copy_kernel<8><<<grid, 256>>>(src, dst, half / 16); }, 2.0 * half));
  }
  std::printf("hipMemcpyAsync device to device        : %8.1f GB/s read+write\n",
              time_gbs([&] { CHECK(hipMemcpyAsync(dst, src, half, hipMemcpyDeviceToDevice, 0)); }, 2.0 * half));
  CHECK(hipFree(p));
  CHECK(hipFree(out));
  return 0;
}

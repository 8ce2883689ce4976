// Host-side checks of the libkvck C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
//
// Every entry point is called with arguments it must reject -- bad layouts,
// plane ranges, numbering, strides and extents at the edges of their integer
// types, undersized or misaligned workspaces -- and with valid arguments,
// which on a machine without a gfx950 device must report KVCK_ERR_NO_DEVICE.
// No device memory is ever touched: device pointers are fake addresses that
// validation never dereferences.  Any out-of-bounds host access, signed
// overflow or other undefined behaviour aborts the program.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "kvck.h"

namespace {

int g_failed = 0;
int g_checked = 0;

void expect_eq(long long got, long long want, const char* what, int line) {
  ++g_checked;
  if (got != want) {
    ++g_failed;
    std::printf("FAIL line %d: %s: got %lld, want %lld\n", line, what, got, want);
  }
}
#define EXPECT_EQ(got, want) expect_eq((long long)(got), (long long)(want), #got, __LINE__)

void* const kFake = reinterpret_cast<void*>(uintptr_t(0x7F0000001000));  // 256-byte aligned, never read
constexpr int32_t kI32Max = std::numeric_limits<int32_t>::max();
constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(kFake) + off); }

kvck_kv_layout hnd_layout() {
  kvck_kv_layout L;
  std::memset(&L, 0, sizeof(L));
  L.planes = 2;
  L.block_size = 16;
  L.num_heads = 8;
  L.row_bytes = 256;
  L.num_blocks = 100;
  L.plane_stride = 100 * 32768;
  L.block_stride = 32768;
  L.slot_stride = 256;
  L.head_stride = 4096;
  return L;
}

struct BlocksCall {
  kvck_kv_layout L = hnd_layout();
  std::vector<const void*> ptrs{kFake, kFake};
  std::vector<int32_t> layers{0, 1};
  std::vector<int32_t> bases{0, 0};
  int32_t head_begin = 0, head_count = 8;
  int32_t num_reqs = 4, max_blocks = 8;
  int64_t bt_stride = 8;
  void* out = kFake;
  int64_t out_stride = 1;
  void* ws = kFake;
  size_t ws_bytes = 0;  // 0: the size kvck_blocks_workspace_bytes gives
  int32_t direction = -1;  // -1: kvck_checksum_blocks; -2: kvck_checksum_blocks_noalloc; else the fused copy
  void* staging = kFake;
  int64_t staging_positions = 64;
  uintptr_t bt_off = 0, nb_off = 0, i64_off = 0;  // byte offsets of the request arrays (misalignment)

  int run() {
    const size_t need = ws_bytes ? ws_bytes
                                 : kvck_blocks_workspace_bytes((int32_t)ptrs.size(), num_reqs, max_blocks);
    const auto* bt = static_cast<const int32_t*>(fake(bt_off));
    const auto* nb = static_cast<const int32_t*>(fake(nb_off));
    const auto* i64 = static_cast<const int64_t*>(fake(i64_off));
    if (direction == -2)
      return kvck_checksum_blocks_noalloc(&L, ptrs.data(), layers.data(), bases.data(), (int32_t)ptrs.size(),
                                          head_begin, head_count, bt, bt_stride, nb, i64, i64, num_reqs, max_blocks,
                                          static_cast<uint64_t*>(out), out_stride, 0, nullptr, nullptr);
    if (direction < 0)
      return kvck_checksum_blocks(&L, ptrs.data(), layers.data(), bases.data(), (int32_t)ptrs.size(), head_begin,
                                  head_count, bt, bt_stride, nb, i64, i64, num_reqs, max_blocks,
                                  static_cast<uint64_t*>(out), out_stride, 0, ws, need, nullptr, nullptr);
    std::vector<void*> mptrs;
    for (const void* p : ptrs) mptrs.push_back(const_cast<void*>(p));
    return kvck_copy_checksum_blocks(direction, &L, mptrs.data(), layers.data(), bases.data(), (int32_t)ptrs.size(),
                                     head_begin, head_count, bt, bt_stride, nb, i64, i64, num_reqs, max_blocks,
                                     staging, staging_positions, static_cast<uint64_t*>(out), out_stride, 0, ws,
                                     need, nullptr, nullptr);
  }
};

void blocks_checks(bool have_device) {
  auto call = [](auto&& edit) {
    BlocksCall c;
    edit(c);
    return c.run();
  };
  EXPECT_EQ(call([](BlocksCall& c) { c.L.planes = 3; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.block_size = 0; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.row_bytes = 12; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.slot_stride = -256; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.num_blocks = -1; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.head_count = 0; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.head_begin = 7, c.head_count = 2; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.head_begin = kI32Max, c.head_count = kI32Max; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.bases = {0, 65535}; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.bases = {0, kI32Max}; }), KVCK_ERR_UNSUPPORTED);
  if (!have_device) EXPECT_EQ(call([](BlocksCall& c) { c.layers = {40000, kI32Max}; }), KVCK_ERR_NO_DEVICE);
  EXPECT_EQ(call([](BlocksCall& c) { c.layers = {0, -1}; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.ptrs[1] = nullptr; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.out = nullptr; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.bt_stride = 4; }), KVCK_ERR_INVALID_ARGUMENT);
  // output stride: one replica column of at most KVCK_MAX_OUT_STRIDE
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = 0; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = -3; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = KVCK_MAX_OUT_STRIDE + 1; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = kI64Max; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = 0, c.num_reqs = 0; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = 0, c.direction = KVCK_COPY_SAVE; }), KVCK_ERR_INVALID_ARGUMENT);
  if (!have_device) EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = KVCK_MAX_OUT_STRIDE; }), KVCK_ERR_NO_DEVICE);
  // request arrays and out aligned to their element size
  EXPECT_EQ(call([](BlocksCall& c) { c.bt_off = 2; }), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.nb_off = 2; }), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.i64_off = 4; }), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.out = fake(4); }), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.direction = KVCK_COPY_LOAD, c.bt_off = 1; }), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.ws_bytes = 64; }), KVCK_ERR_WORKSPACE);
  EXPECT_EQ(call([](BlocksCall& c) { c.ws = fake(8); }), KVCK_ERR_WORKSPACE);
  EXPECT_EQ(call([](BlocksCall& c) { c.ws = nullptr; }), KVCK_ERR_WORKSPACE);
  EXPECT_EQ(call([](BlocksCall& c) {
              c.ptrs = {fake(4), fake(4)};
              c.L.row_bytes = 8, c.L.slot_stride = 8, c.L.head_stride = 128, c.L.block_stride = 2048;
            }),
            KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.row_bytes = 16 * 1024 * 2; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) {
              c.ptrs.assign(KVCK_MAX_CACHES + 1, kFake);
              c.layers.assign(KVCK_MAX_CACHES + 1, 0);
              c.bases.assign(KVCK_MAX_CACHES + 1, 0);
            }),
            KVCK_ERR_UNSUPPORTED);
  // plane ranges at the edge of int32
  EXPECT_EQ(call([](BlocksCall& c) { c.L.plane_begin = kI32Max, c.L.plane_count = 1; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.plane_begin = 1, c.L.plane_count = kI32Max; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.plane_begin = -1; }), KVCK_ERR_INVALID_ARGUMENT);
  // strides and extents at the edge of int64
  EXPECT_EQ(call([](BlocksCall& c) { c.L.slot_stride = kI64Max / 2 / 16 * 16; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.block_stride = kI64Max / 16 * 16; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.num_blocks = kI64Max, c.L.block_stride = 32768; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.head_stride = (int64_t)1 << 62; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.plane_stride = (int64_t)1 << 50; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.chunk_bytes = 16, c.L.chunk_stride = kI64Max / 32 * 16; }),
            KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.L.chunk_bytes = 24; }), KVCK_ERR_UNSUPPORTED);  // 256 % 24 != 0
  // element-transposed planes (one-element runs): one plane per call, slots side by side
  auto trans = [](BlocksCall& c) {
    c.L.chunk_bytes = 2, c.L.chunk_stride = 16 * 2, c.L.slot_stride = 2, c.L.plane_begin = 1, c.L.plane_count = 1;
    c.L.head_stride = 128 * 16 * 2, c.L.block_stride = 8 * 128 * 16 * 2;
  };
  if (!have_device) EXPECT_EQ(call([&](BlocksCall& c) { trans(c); }), KVCK_ERR_NO_DEVICE);
  EXPECT_EQ(call([&](BlocksCall& c) { trans(c), c.L.chunk_stride = 16; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([&](BlocksCall& c) { trans(c), c.L.slot_stride = 4; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([&](BlocksCall& c) { trans(c), c.L.plane_begin = 0, c.L.plane_count = 0; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([&](BlocksCall& c) { trans(c), c.L.block_size = 2, c.L.chunk_stride = 4; }), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([&](BlocksCall& c) { trans(c), c.L.chunk_bytes = 3; }), KVCK_ERR_UNSUPPORTED);
  // the fused copy transposes whole N x N tiles: a tile row must fit one lane table (block_size <= 1024)
  if (!have_device) EXPECT_EQ(call([&](BlocksCall& c) { trans(c), c.direction = KVCK_COPY_SAVE; }), KVCK_ERR_NO_DEVICE);
  auto big = [&](BlocksCall& c) {
    trans(c), c.L.block_size = 2048, c.L.chunk_stride = 2048 * 2;
    c.L.head_stride = 128 * 2048 * 2, c.L.block_stride = 8 * c.L.head_stride;
  };
  if (!have_device) EXPECT_EQ(call([&](BlocksCall& c) { big(c); }), KVCK_ERR_NO_DEVICE);
  EXPECT_EQ(call([&](BlocksCall& c) { big(c), c.direction = KVCK_COPY_LOAD; }), KVCK_ERR_UNSUPPORTED);
  // batch sizes
  EXPECT_EQ(call([](BlocksCall& c) { c.num_reqs = kI32Max, c.max_blocks = kI32Max, c.bt_stride = kI32Max; }),
            KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.num_reqs = -1; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.num_reqs = 0; }), KVCK_OK);
  EXPECT_EQ(call([](BlocksCall& c) { c.max_blocks = 0; }), KVCK_OK);
  if (!have_device) EXPECT_EQ(call([](BlocksCall&) {}), KVCK_ERR_NO_DEVICE);

  // fused copy
  EXPECT_EQ(call([](BlocksCall& c) { c.direction = 2; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.direction = KVCK_COPY_SAVE, c.staging = nullptr; }),
            KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.direction = KVCK_COPY_LOAD, c.staging_positions = -1; }),
            KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.direction = KVCK_COPY_SAVE, c.staging_positions = kI64Max; }),
            KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call([](BlocksCall& c) { c.direction = KVCK_COPY_SAVE, c.staging = fake(4); }), KVCK_ERR_MISALIGNED);
  if (!have_device) EXPECT_EQ(call([](BlocksCall& c) { c.direction = KVCK_COPY_LOAD; }), KVCK_ERR_NO_DEVICE);

  // sizes
  EXPECT_EQ(kvck_blocks_workspace_bytes(0, 1, 1), 0);
  EXPECT_EQ(kvck_blocks_workspace_bytes(1, -1, 1), 0);
  EXPECT_EQ(kvck_blocks_workspace_bytes(4096, kI32Max, kI32Max), 0);
  const size_t one = kvck_blocks_workspace_bytes(1, 256, 512), many = kvck_blocks_workspace_bytes(32, 256, 512);
  EXPECT_EQ(one % 256, 0);
  EXPECT_EQ(many % 256, 0);
  EXPECT_EQ(many - one >= (size_t)32 * 256 * 512 * 8, 1);
  kvck_kv_layout L = hnd_layout();
  EXPECT_EQ(kvck_staging_bytes(nullptr, 1, 8), 0);
  EXPECT_EQ(kvck_staging_bytes(&L, 3, 8), (long long)3 * 2 * 8 * 16 * 256);
  EXPECT_EQ(kvck_staging_bytes(&L, 0, 8), 0);
  EXPECT_EQ(kvck_staging_bytes(&L, kI32Max, kI32Max), 0);  // 2^50 or more
  L.plane_begin = 1;
  EXPECT_EQ(kvck_staging_bytes(&L, 1, 8), (long long)1 * 8 * 16 * 256);
  L.plane_begin = kI32Max;
  L.plane_count = 1;
  EXPECT_EQ(kvck_staging_bytes(&L, 1, 8), 0);
  L.plane_begin = -5;
  L.plane_count = 0;
  EXPECT_EQ(kvck_staging_bytes(&L, 1, 8), 0);
  L = hnd_layout();
  L.planes = 3;
  EXPECT_EQ(kvck_staging_bytes(&L, 1, 8), 0);
}

void states_checks(bool have_device) {
  kvck_state_desc D[2];
  auto reset = [&] {
    D[0] = {64 * 8192, 8192, 2048, 4};
    D[1] = {64 * 2048, 2048, 1024, 2};
  };
  reset();
  const void* ptrs[4] = {kFake, kFake, kFake, kFake};
  const int32_t layers[2] = {1, 3}, base[2] = {0, 0};
  auto call = [&](int nstates = 2, int32_t nrows = 64, int32_t rb = 0, int32_t rc = 64, void* ws = kFake,
                  size_t ws_bytes = 1 << 20, int32_t num_reqs = 8, int32_t num_slots = 160,
                  int64_t out_stride = 1, void* out = kFake) {
    return kvck_checksum_states(D, nstates, ptrs, layers, base, 2, num_slots, nrows, rb, rc,
                                static_cast<const int32_t*>(kFake), num_reqs, static_cast<uint64_t*>(out), out_stride,
                                0, ws, ws_bytes, nullptr, nullptr);
  };
  D[1].elem_bytes = 1;
  EXPECT_EQ(call(), KVCK_ERR_UNSUPPORTED);
  D[1].elem_bytes = 8;
  EXPECT_EQ(call(), KVCK_ERR_UNSUPPORTED);
  reset();
  EXPECT_EQ(call(5), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call(0), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call(2, 64, 60, 8), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(2, 64, kI32Max, kI32Max), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(2, 64, 0, 64, kFake, 8), KVCK_ERR_WORKSPACE);
  EXPECT_EQ(call(2, 64, 0, 64, fake(8)), KVCK_ERR_WORKSPACE);
  EXPECT_EQ(call(2, 64, 0, 64, kFake, 1 << 20, 0), KVCK_OK);
  EXPECT_EQ(call(2, 64, 0, 64, kFake, 1 << 20, -1), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(2, 64, 0, 64, kFake, 1 << 20, 8, 160, 0), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(2, 64, 0, 64, kFake, 1 << 20, 8, 160, KVCK_MAX_OUT_STRIDE + 1), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(2, 64, 0, 64, kFake, 1 << 20, 8, 160, 1, fake(4)), KVCK_ERR_MISALIGNED);
  if (!have_device) EXPECT_EQ(call(2, 64, 0, 64, kFake, 1 << 20, 8, 160, KVCK_MAX_OUT_STRIDE), KVCK_ERR_NO_DEVICE);
  D[0].slot_stride = kI64Max / 16 * 16;
  EXPECT_EQ(call(), KVCK_ERR_UNSUPPORTED);
  reset();
  D[1].row_stride = (int64_t)1 << 49;
  EXPECT_EQ(call(), KVCK_ERR_UNSUPPORTED);
  reset();
  D[0].row_elems = kI32Max;  // 4-byte elements: row bytes not a multiple of 16
  EXPECT_EQ(call(), KVCK_ERR_UNSUPPORTED);
  D[0].row_elems = kI32Max - 7;
  D[0].row_stride = (int64_t)(kI32Max - 7) * 4;
  D[0].slot_stride = D[0].row_stride * 64;
  EXPECT_EQ(call(), KVCK_ERR_UNSUPPORTED);  // too many elements per slice
  reset();
  D[0].slot_stride = 8;
  EXPECT_EQ(call(), KVCK_ERR_MISALIGNED);
  reset();
  if (!have_device) EXPECT_EQ(call(), KVCK_ERR_NO_DEVICE);
  EXPECT_EQ(kvck_states_workspace_bytes(0, 64, 8), 0);
  EXPECT_EQ(kvck_states_workspace_bytes(kI32Max, kI32Max, kI32Max), 0);
  EXPECT_EQ(kvck_states_workspace_bytes(24, 64, 128) >= (size_t)24 * 8 * 128 * 8, 1);
}

void tags_checks(bool have_device) {
  auto call = [](const void* cs, const void* h, int64_t stride, int64_t n, const void* nbpr, int32_t mb,
                 void* tagged, const void* stored, void* mm, int32_t columns = 1) {
    return kvck_tag_checksums(static_cast<const uint64_t*>(cs), columns, static_cast<const uint8_t*>(h), stride,
                              0x1234, n,
                              static_cast<const int32_t*>(nbpr), nullptr, mb, 0, static_cast<uint64_t*>(tagged),
                              static_cast<const uint64_t*>(stored), static_cast<uint8_t*>(mm), nullptr, nullptr);
  };
  EXPECT_EQ(call(kFake, kFake, 32, 0, nullptr, 0, kFake, nullptr, nullptr), KVCK_OK);
  EXPECT_EQ(call(kFake, kFake, 32, -1, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(nullptr, kFake, 32, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, nullptr, nullptr, nullptr), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, kFake, nullptr, kFake), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 4, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 12, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call(kFake, fake(4), 32, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call(kFake, kFake, 32, 16, kFake, 5, kFake, nullptr, nullptr), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 32, kI64Max, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call(kFake, kFake, kI64Max / 8 * 8, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_UNSUPPORTED);
  // replica columns summed per entry; uint64 arrays 8-byte aligned
  EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, kFake, nullptr, nullptr, 0), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, kFake, nullptr, nullptr, KVCK_MAX_OUT_STRIDE + 1),
            KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call(kFake, kFake, 32, (int64_t)1 << 40, nullptr, 0, kFake, nullptr, nullptr, 4096),
            KVCK_ERR_UNSUPPORTED);
  EXPECT_EQ(call(fake(4), kFake, 32, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, fake(4), nullptr, nullptr), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, nullptr, fake(4), nullptr), KVCK_ERR_MISALIGNED);
  if (!have_device) EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, kFake, nullptr, nullptr), KVCK_ERR_NO_DEVICE);
  if (!have_device)
    EXPECT_EQ(call(kFake, kFake, 32, 16, nullptr, 0, kFake, nullptr, nullptr, KVCK_MAX_OUT_STRIDE), KVCK_ERR_NO_DEVICE);
}

void noalloc_checks(bool have_device) {
  auto call = [](auto&& edit) {
    BlocksCall c;
    c.direction = -2;
    edit(c);
    return c.run();
  };
  EXPECT_EQ(call([](BlocksCall& c) { c.num_reqs = 0; }), KVCK_OK);
  EXPECT_EQ(call([](BlocksCall& c) { c.out = nullptr; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.layers = {0, -1}; }), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(call([](BlocksCall& c) { c.bt_off = 2; }), KVCK_ERR_MISALIGNED);
  EXPECT_EQ(call([](BlocksCall& c) { c.out_stride = 0; }), KVCK_ERR_INVALID_ARGUMENT);
  // position records alone past the scratch: 32 bytes per request slot
  EXPECT_EQ(call([](BlocksCall& c) { c.num_reqs = 1100, c.max_blocks = 1024, c.bt_stride = 1024; }),
            KVCK_ERR_SCRATCH);
  EXPECT_EQ(call([](BlocksCall& c) { c.num_reqs = kI32Max, c.max_blocks = kI32Max, c.bt_stride = kI32Max; }),
            KVCK_ERR_UNSUPPORTED);
  if (!have_device) EXPECT_EQ(call([](BlocksCall&) {}), KVCK_ERR_NO_DEVICE);
}

void misc_checks() {
  EXPECT_EQ(kvck_abi_version(), 3);
  const int32_t codes[] = {KVCK_OK,           KVCK_ERR_INVALID_ARGUMENT, KVCK_ERR_UNSUPPORTED, KVCK_ERR_MISALIGNED,
                           KVCK_ERR_WORKSPACE, KVCK_ERR_HIP,             KVCK_ERR_NO_DEVICE,   KVCK_ERR_SCRATCH,
                           7,                 -1000,                     kI32Max};
  for (int32_t c : codes) EXPECT_EQ(kvck_status_string(c) != nullptr && kvck_status_string(c)[0] == 'K', 1);
  EXPECT_EQ(std::strcmp(kvck_status_string(KVCK_ERR_WORKSPACE), "KVCK_ERR_WORKSPACE"), 0);
  double ms = -1.0;
  int64_t calls = -1;
  EXPECT_EQ(kvck_instrument(1), KVCK_OK);
  EXPECT_EQ(kvck_instrument_read(&ms, &calls), KVCK_OK);
  EXPECT_EQ(calls, 0);
  EXPECT_EQ(kvck_instrument_read(nullptr, &calls), KVCK_ERR_INVALID_ARGUMENT);
  EXPECT_EQ(kvck_instrument(0), KVCK_OK);
}

}  // namespace

int main() {
  const bool have_device = kvck_platform_supported() != 0;
  blocks_checks(have_device);
  noalloc_checks(have_device);
  states_checks(have_device);
  tags_checks(have_device);
  misc_checks();
  std::printf("%d checks, %d failed (gfx950 device present: %d)\n", g_checked, g_failed, (int)have_device);
  if (g_failed == 0) std::printf("all checks passed\n");
  return g_failed == 0 ? 0 : 1;
}

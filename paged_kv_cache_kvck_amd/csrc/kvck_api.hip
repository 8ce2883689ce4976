// C ABI of libkvck: argument validation, launch shapes, workspace carving.
// Every check that can be made on the host is made before the first HIP call,
// so a rejected call touches no device state.
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <vector>

#include "kvck_internal.h"

#define KVCK_EXPORT extern "C" __attribute__((visibility("default")))

namespace kvck {
namespace {

constexpr int64_t kH = KVCK_MAX_KV_HEADS_PER_LAYER;

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)a) == 0; }

// Scratch of kvck_checksum_blocks_noalloc: one copy per device, held from the
// module's load until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[KVCK_SCRATCH_BYTES];

// Device address of `scratch` on device `dev` (current), or null if the
// runtime cannot give it.
void* scratch_address(int dev) {
  static std::mutex mu;
  static void* addr[64];
  std::lock_guard<std::mutex> g(mu);
  if (dev < 0 || dev >= 64) return nullptr;
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

// Largest byte extent of a tensor the kernels address (64-bit offsets with
// room to spare; far beyond any device memory).
constexpr int64_t kMaxExtent = (int64_t)1 << 50;

struct Dim {
  int64_t n, stride;  // extent along one axis, bytes between neighbours
};

// Byte extent of a strided tensor, sum of (n-1)*stride over its axes plus the
// bytes of its last element; false when that overflows or reaches kMaxExtent.
// Callers have checked n >= 0 and stride >= 0.
bool extent_ok(std::initializer_list<Dim> dims, int64_t tail) {
  int64_t total = tail;
  for (const Dim& d : dims) {
    if (d.n < 1) continue;
    int64_t t = 0;
    if (__builtin_mul_overflow(d.n - 1, d.stride, &t) || __builtin_add_overflow(total, t, &total)) return false;
  }
  return total < kMaxExtent;
}

// a * b * c < kMaxExtent for non-negative factors, without overflow
bool product_ok(int64_t a, int64_t b, int64_t c) {
  int64_t t = 0;
  return !__builtin_mul_overflow(a, b, &t) && !__builtin_mul_overflow(t, c, &t) && t < kMaxExtent;
}

// gfx950 check of the current device, cached per device id.
kvck_status current_device(int* dev_out) {
  static std::mutex mu;
  static int known[64];  // 0 unknown, 1 gfx950, -1 other
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return KVCK_ERR_NO_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVCK_ERR_NO_DEVICE;
  {
    std::lock_guard<std::mutex> g(mu);
    if (dev >= 0 && dev < 64 && known[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KVCK_ERR_HIP;
      known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (dev < 0 || dev >= 64 || known[dev] != 1) return KVCK_ERR_NO_DEVICE;
  }
  *dev_out = dev;
  return KVCK_OK;
}

// Lane-table shape: the smallest S whose 64*S lane-chunks cover a whole block
// row set of one (plane, head); larger row sets are split into groups of
// equal size, each at most the rows one table of 16 slots holds.
bool choose_shape(int32_t block_size, int32_t row_bytes, int chunk, int max_slots, BlocksShape* shp) {
  const int64_t cpr = row_bytes / chunk;
  const int64_t max_chunks = (int64_t)kWave * max_slots;
  if (cpr > max_chunks) return false;
  const int64_t rg_max = max_chunks / cpr;
  const int64_t groups = (block_size + rg_max - 1) / rg_max;
  const int64_t rg = (block_size + groups - 1) / groups;  // <= rg_max
  const int64_t need = (rg * cpr + kWave - 1) / kWave;    // <= max_slots
  int s = 1;
  while (s < need) s <<= 1;
  shp->chunk = chunk;
  shp->slots = s;
  shp->rows_per_group = (int)rg;
  shp->pipelined = false;
  shp->caches_per_task = 1;
  shp->planes_per_unit = 1;
  shp->merged = false;
  shp->copy_buffers = 1;
  shp->transposed = false;
  shp->elem_bytes = 0;
  shp->dense = false;
  shp->lds_transpose = false;
  return true;
}

// Heads side by side in a slot (head_stride == row_bytes) are read as one row
// per slot when one head's row is shorter than this: short rows would leave
// each load instruction with many short segments.
constexpr int32_t kMergeBelowRowBytes = 128;

// Schedule: with many tasks per resident wave, keep two unit buffers in
// flight and let one task cover several caches, so a wave's loads do not
// drain at every unit boundary and rarely at a task boundary (a boundary
// costs about one memory latency plus the reduction).  A task covers enough
// caches to stream about kPipeTaskBytes of a full block, capped at
// kPipeMaxCaches.  Small batches keep one cache per task and higher occupancy
// (their run time is dominated by ramp-up and tail).  Lane tables of more
// than 4 slots would need more than half the register file double-buffered:
// such blocks pipeline only in the narrow shape below (more row groups).
constexpr int64_t kPipeTaskBytes = 256 * 1024;
constexpr int kPipeMaxCaches = 16;
constexpr int64_t kPipeMinTasksPerWave = 32;
static_assert(kCachesPerLaunch % kPipeMaxCaches == 0, "launch groups must not straddle launches");

// `narrow` (or null) is the same rows split into lane tables of at most 4
// slots (8 for merged rows), the widest the pipelined kernel double-buffers:
// blocks whose rows need more slots per lane can still be pipelined, in more
// row groups.
//
// A call planned in place (`dense`) whose caches all fit one task's byte
// budget runs one pipelined task per position over every cache: a single
// launch with no second pass, where latency rather than lane use counts.
// KVCK_MERGED_PIPE=0 keeps merged rows on the unpipelined kernel (A/B switch;
// results are identical).
bool merged_pipe_off() {
  const char* e = getenv("KVCK_MERGED_PIPE");
  return e && e[0] == '0';
}

void choose_schedule(BlocksShape* shp, const BlocksShape* narrow, int32_t num_caches, int64_t max_items,
                     int64_t block_bytes, int planes, int heads, int cus, bool copy, bool dense, bool save) {
  const int64_t waves = (int64_t)cus * 4 * kMainWorkgroupsPerCU;  // resident waves of the main pass
  int lpt = 1;
  while (lpt < kPipeMaxCaches && (int64_t)(2 * lpt) * block_bytes <= kPipeTaskBytes) lpt *= 2;
  const int64_t tasks = max_items * ((num_caches + lpt - 1) / lpt);
  // A pipelined unit holds 16/S head slots (K and V can share one when heads
  // are few); with fewer heads than that its loads would be mostly masked.
  auto fills = [&](int slots) { return (int64_t)heads * (planes == 2 ? 2 : 1) * slots >= 16; };
  // Merged rows (a slot's heads as one row) fill their lanes by construction
  // and pipeline with up to 8 slots per lane (one plane per unit).
  const int max_pipe_slots = shp->merged ? 8 : 4;
  const BlocksShape* cand = shp->slots <= max_pipe_slots ? shp : narrow;
  const bool fits = cand != nullptr && (shp->merged || fills(cand->slots));
  const bool one_task = dense && !copy && cand != nullptr && num_caches <= lpt;
  bool pipe = (fits && num_caches > 1 && tasks >= kPipeMinTasksPerWave * waves) || one_task;
  if (!copy && !dense && shp->merged) {
    // The planned pipelined checksum of merged rows streams its units across
    // task boundaries (no drain between tasks), so a task may be as small as
    // one cache: halve the caches per task until every resident wave has
    // kPipeMinTasksPerWave tasks to balance the load, and pipeline whenever
    // the shape allows.
    while (lpt > 1 && max_items * ((num_caches + lpt - 1) / lpt) < kPipeMinTasksPerWave * waves) lpt /= 2;
    pipe = fits;
  }
  // KVCK_SCHEDULE=pipelined|simple overrides the choice (results are identical
  // either way)
  if (const char* force = getenv("KVCK_SCHEDULE")) {
    if (strcmp(force, "pipelined") == 0) pipe = true;
    if (strcmp(force, "simple") == 0) pipe = false;
  }
  if (merged_pipe_off() && shp->merged && !copy) pipe = false;
  if (copy) {
    // A load keeps one unit buffer per wave, as many waves as fit: its stores
    // into pool blocks gain from more waves in flight (same-box A/B, llama3-
    // shaped batch: the ping-pong kernel 23.8 -> 24.4 ms at all that fit, 26.2
    // at one workgroup per CU).  A save runs the ping-pong kernel at one
    // workgroup per CU (copy_grid): 22.66 -> 22.42 ms on the same batch, and
    // on 64-request batches +0.4 % (GPT-2-shaped fp16), +0.5 % (MLA) and
    // +8.3 % (fp8 64-byte merged rows).  KVCK_COPY_BUFFERS=1|2 forces one or
    // the other (results are identical).
    shp->copy_buffers = save ? 2 : 1;
    if (const char* b = getenv("KVCK_COPY_BUFFERS")) shp->copy_buffers = b[0] == '2' ? 2 : 1;
  }
  if (copy) pipe = true;  // the fused copy kernel always runs the pipelined structure
  if (pipe && !copy && shp->slots > max_pipe_slots && narrow && (shp->merged || fills(narrow->slots) || one_task)) {
    shp->slots = narrow->slots;
    shp->rows_per_group = narrow->rows_per_group;
  }
  if (!copy && shp->merged && shp->slots > 8) pipe = false;      // merged pipelined variants stop at 8 slots
  if (!copy && shp->transposed && shp->slots > 4) pipe = false;  // transposed ones at 4
  if (pipe) {
    shp->pipelined = true;
    shp->caches_per_task = lpt;
    // a unit holds 16/S head slots; with half of them or fewer used, carry K and V together
    const int hu = 16 / shp->slots;
    if (planes == 2 && shp->slots <= 4 && 2 * heads <= hu && !shp->merged) shp->planes_per_unit = 2;
  }
}

// Event pairs around main passes while instrumentation is on.
struct Instrument {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  size_t used = 0;
};
Instrument g_instr;

// Returns a (start, stop) pair to record, or nulls when instrumentation is off.
bool instrument_pair(hipEvent_t* s, hipEvent_t* e) {
  std::lock_guard<std::mutex> g(g_instr.mu);
  if (!g_instr.on) return false;
  if (g_instr.used == g_instr.start.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return false;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return false;
    }
    g_instr.start.push_back(a);
    g_instr.stop.push_back(b);
  }
  *s = g_instr.start[g_instr.used];
  *e = g_instr.stop[g_instr.used];
  ++g_instr.used;
  return true;
}

}  // namespace
}  // namespace kvck

using namespace kvck;

KVCK_EXPORT kvck_status kvck_instrument(int32_t enable) {
  std::lock_guard<std::mutex> g(g_instr.mu);
  g_instr.on = enable != 0;
  g_instr.used = 0;
  return KVCK_OK;
}

KVCK_EXPORT kvck_status kvck_instrument_read(double* total_ms, int64_t* calls) {
  if (!total_ms || !calls) return KVCK_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> g(g_instr.mu);
  double tot = 0.0;
  for (size_t i = 0; i < g_instr.used; ++i) {
    if (hipEventSynchronize(g_instr.stop[i]) != hipSuccess) return KVCK_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_instr.start[i], g_instr.stop[i]) != hipSuccess) return KVCK_ERR_HIP;
    tot += ms;
  }
  *total_ms = tot;
  *calls = (int64_t)g_instr.used;
  g_instr.used = 0;
  return KVCK_OK;
}

KVCK_EXPORT int32_t kvck_abi_version(void) { return KVCK_ABI_VERSION; }

KVCK_EXPORT const char* kvck_status_string(int32_t status) {
  switch (status) {
    case KVCK_OK: return "KVCK_OK";
    case KVCK_ERR_INVALID_ARGUMENT: return "KVCK_ERR_INVALID_ARGUMENT";
    case KVCK_ERR_UNSUPPORTED: return "KVCK_ERR_UNSUPPORTED";
    case KVCK_ERR_MISALIGNED: return "KVCK_ERR_MISALIGNED";
    case KVCK_ERR_WORKSPACE: return "KVCK_ERR_WORKSPACE";
    case KVCK_ERR_HIP: return "KVCK_ERR_HIP";
    case KVCK_ERR_NO_DEVICE: return "KVCK_ERR_NO_DEVICE";
    case KVCK_ERR_SCRATCH: return "KVCK_ERR_SCRATCH";
  }
  return "KVCK_UNKNOWN_STATUS";
}

KVCK_EXPORT int32_t kvck_platform_supported(void) {
  int dev = 0;
  return current_device(&dev) == KVCK_OK ? 1 : 0;
}

KVCK_EXPORT size_t kvck_blocks_workspace_bytes(int32_t num_caches, int32_t num_reqs, int32_t max_blocks) {
  if (num_caches < 1 || num_reqs < 0 || max_blocks < 0) return 0;
  if ((int64_t)num_reqs * max_blocks >= ((int64_t)1 << 31)) return 0;  // a batch the entry points reject
  return BlocksWorkspace::make(num_caches, num_reqs, max_blocks).total;
}

namespace {
// What the kernels need to know of a layout once it is checked.
struct LayoutInfo {
  int32_t run_bytes;  // bytes of one contiguous run of a row (the row itself unless x-split)
  int32_t runs;       // runs per row
  int32_t planes_cov; // planes the call covers
  bool transposed;    // runs shorter than a piece: rows stored element by element
};

// Layout checks of the blocks entry points: strides, runs, plane range and
// the extent every addressed byte lies in.
kvck_status check_layout(const kvck_kv_layout& L, LayoutInfo* li) {
  if (L.planes != 1 && L.planes != 2) return KVCK_ERR_INVALID_ARGUMENT;
  if (L.block_size < 1 || L.num_heads < 1 || L.row_bytes < 1 || L.num_blocks < 0) return KVCK_ERR_INVALID_ARGUMENT;
  if (L.plane_stride < 0 || L.block_stride < 0 || L.slot_stride < 0 || L.head_stride < 0)
    return KVCK_ERR_INVALID_ARGUMENT;
  if (L.row_bytes % 8 != 0) return KVCK_ERR_UNSUPPORTED;
  // rows stored as runs (x-split layouts) and plane subsets
  if (L.chunk_bytes < 0 || L.chunk_stride < 0 || L.plane_begin < 0 || L.plane_count < 0)
    return KVCK_ERR_INVALID_ARGUMENT;
  const int32_t run_bytes = L.chunk_bytes == 0 ? L.row_bytes : L.chunk_bytes;
  // runs shorter than a piece: rows stored element by element (element-transposed
  // planes); the elements of all slots of one index must sit side by side
  const bool transposed = run_bytes < 8;
  if (transposed) {
    if ((run_bytes != 1 && run_bytes != 2 && run_bytes != 4) || L.slot_stride != run_bytes)
      return KVCK_ERR_UNSUPPORTED;
    if (L.chunk_stride < (int64_t)L.block_size * run_bytes) return KVCK_ERR_INVALID_ARGUMENT;
    // an element row of the block must hold whole 8-byte loads
    if (((int64_t)L.block_size * run_bytes) % 8 != 0) return KVCK_ERR_UNSUPPORTED;
  } else if (run_bytes % 8 != 0 || L.row_bytes % run_bytes != 0) {
    return KVCK_ERR_UNSUPPORTED;
  }
  const int32_t runs = L.row_bytes / run_bytes;
  const int32_t planes_cov = L.plane_count == 0 ? L.planes - L.plane_begin : L.plane_count;
  if (planes_cov < 1 || (int64_t)L.plane_begin + planes_cov > L.planes) return KVCK_ERR_INVALID_ARGUMENT;
  if (transposed && planes_cov != 1) return KVCK_ERR_UNSUPPORTED;  // one plane per call
  // every byte the kernels may address lies within a 2^50-byte extent
  if (!extent_ok({{L.planes, L.plane_stride}, {L.num_blocks, L.block_stride}, {L.block_size, L.slot_stride},
                  {L.num_heads, L.head_stride}, {runs, L.chunk_stride}},
                 run_bytes))
    return KVCK_ERR_UNSUPPORTED;
  li->run_bytes = run_bytes;
  li->runs = runs;
  li->planes_cov = planes_cov;
  li->transposed = transposed;
  return KVCK_OK;
}

constexpr int kModeChecksum = -1;

// Smallest pool (bytes per cache) over which the fused copy sorts its positions by block id.
constexpr int64_t kOrderMinPoolBytes = (int64_t)2 << 30;  // kvck_checksum_blocks; otherwise a KVCK_COPY_* direction

// kvck_checksum_blocks and kvck_copy_checksum_blocks: validation, plan, main
// pass (checksum only, or fused copy), second pass.
kvck_status blocks_call(int mode, const kvck_kv_layout* layout, const void* const* cache_ptrs,
                        const int32_t* layer_numbers, const int32_t* global_head_base, int32_t num_caches,
                        int32_t head_begin, int32_t head_count, const int32_t* block_table,
                        int64_t block_table_row_stride, const int32_t* num_blocks_per_req, const int64_t* start_pos,
                        const int64_t* num_tokens, int32_t num_reqs, int32_t max_blocks, uint64_t* out,
                        int64_t out_stride, int32_t accumulate, void* workspace, size_t workspace_bytes, uint32_t* error_flags,
                        void* staging, int64_t staging_positions, kvck_stream_t stream, bool use_scratch = false) {
  if (mode != kModeChecksum && mode != KVCK_COPY_SAVE && mode != KVCK_COPY_LOAD) return KVCK_ERR_INVALID_ARGUMENT;
  if (use_scratch && mode != kModeChecksum) return KVCK_ERR_INVALID_ARGUMENT;
  // ---- layout
  if (!layout || !cache_ptrs || !layer_numbers || !global_head_base) return KVCK_ERR_INVALID_ARGUMENT;
  if (num_caches < 1 || num_caches > KVCK_MAX_CACHES) return KVCK_ERR_UNSUPPORTED;
  const kvck_kv_layout L = *layout;
  LayoutInfo li;
  const kvck_status ls = check_layout(L, &li);
  if (ls != KVCK_OK) return ls;
  const int32_t run_bytes = li.run_bytes, runs = li.runs, planes_cov = li.planes_cov;
  const bool transposed = li.transposed;
  if (head_begin < 0 || head_count < 1 || (int64_t)head_begin + head_count > L.num_heads)
    return KVCK_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < num_caches; ++i) {
    if (!cache_ptrs[i]) return KVCK_ERR_INVALID_ARGUMENT;
    if (layer_numbers[i] < 0 || global_head_base[i] < 0) return KVCK_ERR_INVALID_ARGUMENT;
    if ((int64_t)global_head_base[i] + head_count > kH) return KVCK_ERR_UNSUPPORTED;
  }
  // ---- requests
  if (num_reqs < 0 || max_blocks < 0) return KVCK_ERR_INVALID_ARGUMENT;
  if (out_stride < 1 || out_stride > KVCK_MAX_OUT_STRIDE) return KVCK_ERR_INVALID_ARGUMENT;
  if (num_reqs == 0 || max_blocks == 0) return KVCK_OK;
  if (!block_table || !num_blocks_per_req || !start_pos || !num_tokens || !out) return KVCK_ERR_INVALID_ARGUMENT;
  // arrays aligned to their element size (small calls read the request arrays with scalar loads)
  if (!aligned(block_table, 4) || !aligned(num_blocks_per_req, 4) || !aligned(start_pos, 8) ||
      !aligned(num_tokens, 8) || !aligned(out, 8) || (error_flags && !aligned(error_flags, 4)))
    return KVCK_ERR_MISALIGNED;
  if (block_table_row_stride < max_blocks) return KVCK_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_reqs * max_blocks >= (int64_t)1 << 31) return KVCK_ERR_UNSUPPORTED;
  // ---- alignment: 16-byte lane loads when everything allows, else 8-byte
  int chunk = 16;
  for (int pass = 0; pass < 2; ++pass) {
    // transposed rows: a chunk holds one element index of chunk/run_bytes slots
    // (and, for the fused copy, chunk/run_bytes elements of one staging row)
    const bool rows_ok = transposed ? ((int64_t)L.block_size * run_bytes) % chunk == 0 &&
                                          (mode == kModeChecksum || L.row_bytes % chunk == 0)
                                    : run_bytes % chunk == 0 && (L.block_size == 1 || L.slot_stride % chunk == 0);
    bool ok = rows_ok && L.block_stride % chunk == 0 && (planes_cov == 1 || L.plane_stride % chunk == 0) &&
              (L.num_heads == 1 || L.head_stride % chunk == 0) && (runs == 1 || L.chunk_stride % chunk == 0);
    for (int32_t i = 0; ok && i < num_caches; ++i) ok = aligned(cache_ptrs[i], chunk);
    if (mode != kModeChecksum) ok = ok && aligned(staging, chunk);
    if (ok) break;
    if (chunk == 8) return KVCK_ERR_MISALIGNED;
    chunk = 8;
  }
  // merged rows: the call's heads of one slot side by side, read (and, for the
  // fused copy, written on the pool side) as one row
  const int64_t wide = (int64_t)head_count * L.row_bytes;
  // (a merged copy's staging offsets are 32-bit across a plane's head images)
  const bool can_merge = !transposed && runs == 1 && (head_count == 1 || L.head_stride == L.row_bytes) &&
                         wide <= (int64_t)kWave * 16 * chunk &&
                         (mode == kModeChecksum || (int64_t)L.block_size * wide < ((int64_t)1 << 31));
  // (a single head, e.g. an MLA latent, is a merged row of one head: it then
  // pipelines with one head per unit instead of a unit of mostly masked heads)
  bool merged = can_merge && (L.row_bytes < kMergeBelowRowBytes || head_count == 1);
  // KVCK_MERGE_HEADS=0|1 overrides the choice where merging is possible (results are identical)
  if (const char* force = getenv("KVCK_MERGE_HEADS")) merged = can_merge && force[0] == '1';
  const int32_t lane_row_bytes = merged ? (int32_t)wide : L.row_bytes;
  BlocksShape shp, narrow;
  if (transposed) {
    // lane table over element rows of one (block, head): chunk f is element row
    // f / cpe, slots (f mod cpe) * chunk/run_bytes onward; rows split into groups
    // of at most what 16 slots per lane hold
    const int64_t cpe = (int64_t)L.block_size * run_bytes / chunk;
    // The fused copy transposes through LDS when chunks are 16 bytes (both
    // sides then move whole lines; same-box A/B against the register transpose:
    // 7-80 % faster, most for large blocks), with lane tables of at most 8
    // slots so a wave's LDS region stays within 8 KiB; 8-byte chunks (small
    // blocks) transpose in registers.  KVCK_TCOPY=regs|lds forces either where
    // possible (results are identical).
    bool lds_transpose = mode != kModeChecksum && chunk == 16;
    if (const char* t = getenv("KVCK_TCOPY")) lds_transpose = lds_transpose && strcmp(t, "regs") != 0;
    const int64_t D = L.row_bytes / run_bytes;
    // the fused copy transposes whole N x N tiles (N = chunk/run_bytes): groups of whole tile rows
    const int64_t unit = mode == kModeChecksum ? 1 : chunk / run_bytes;
    if (lds_transpose && (int64_t)kWave * 8 / cpe / unit < 1) lds_transpose = false;  // a tile row too wide
    const int64_t max_chunks = (int64_t)kWave * (lds_transpose ? 8 : 16);
    if (cpe > max_chunks) return KVCK_ERR_UNSUPPORTED;
    const int64_t rge_max = max_chunks / cpe / unit * unit;
    if (rge_max < 1) return KVCK_ERR_UNSUPPORTED;
    const int64_t groups = (D + rge_max - 1) / rge_max;
    const int64_t rge = ((D + groups - 1) / groups + unit - 1) / unit * unit;  // <= rge_max
    const int64_t need = (rge * cpe + kWave - 1) / kWave;
    int s = 1;
    while (s < need) s <<= 1;
    if (rge * L.chunk_stride + (int64_t)L.block_size * run_bytes >= ((int64_t)1 << 31)) return KVCK_ERR_UNSUPPORTED;
    memset(&shp, 0, sizeof(shp));
    shp.chunk = chunk;
    shp.slots = s;
    shp.rows_per_group = (int)rge;
    shp.caches_per_task = 1;
    shp.planes_per_unit = 1;
    shp.copy_buffers = 1;
    shp.transposed = true;
    shp.elem_bytes = run_bytes;
    shp.lds_transpose = lds_transpose;
  } else if (!choose_shape(L.block_size, lane_row_bytes, chunk, 16, &shp)) {
    return KVCK_ERR_UNSUPPORTED;
  }
  shp.merged = merged;
  const bool has_narrow = !transposed && choose_shape(L.block_size, lane_row_bytes, chunk, merged ? 8 : 4, &narrow);
  // lane-table offsets and piece terms are 32-bit
  if ((int64_t)shp.rows_per_group * L.slot_stride + (int64_t)(runs - 1) * L.chunk_stride +
          (merged ? lane_row_bytes : run_bytes) >=
      ((int64_t)1 << 31))
    return KVCK_ERR_UNSUPPORTED;
  const int64_t pieces = (int64_t)L.planes * L.row_bytes / 8;
  if (2 * (int64_t)shp.rows_per_group * pieces + 4 * (L.row_bytes / chunk) >= ((int64_t)1 << 32))
    return KVCK_ERR_UNSUPPORTED;
  // ---- staging (fused copy)
  const int64_t image_bytes = (int64_t)planes_cov * head_count * L.block_size * L.row_bytes;
  if (mode != kModeChecksum) {
    if (!staging || staging_positions < 0) return KVCK_ERR_INVALID_ARGUMENT;
    if ((int64_t)L.block_size * L.row_bytes >= ((int64_t)1 << 31)) return KVCK_ERR_UNSUPPORTED;
    if (!product_ok(staging_positions, num_caches, image_bytes)) return KVCK_ERR_UNSUPPORTED;
  }
  // ---- workspace (or, allocation-free, the library's scratch: at least the records must fit)
  const BlocksWorkspace w = BlocksWorkspace::make(num_caches, num_reqs, max_blocks);
  if (use_scratch) {
    if (w.partials_off > (size_t)KVCK_SCRATCH_BYTES) return KVCK_ERR_SCRATCH;
  } else if (!workspace || workspace_bytes < w.total || !aligned(workspace, (int64_t)kAlign)) {
    return KVCK_ERR_WORKSPACE;
  }

  int dev = 0;
  const kvck_status ds = current_device(&dev);
  if (ds != KVCK_OK) return ds;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int cus = device_cus(dev);
  const int64_t max_items = (int64_t)num_reqs * max_blocks;
  // Small checksum calls plan in place: one wave per (slot, cache group) task
  // reads its request's entries itself, which saves the plan launch; larger
  // ones list the positions first so no wave is spent on empty slots.
  // KVCK_PLAN=compact plans every call (results are identical).
  bool dense = mode == kModeChecksum && max_items * num_caches <= kDenseMaxTasks;
  if (const char* force = getenv("KVCK_PLAN"))
    if (strcmp(force, "compact") == 0) dense = false;
  choose_schedule(&shp, has_narrow ? &narrow : nullptr, num_caches, max_items, image_bytes, planes_cov, head_count,
                  cus, mode != kModeChecksum, dense, mode == KVCK_COPY_SAVE);
  shp.dense = dense;
  const int32_t lpt = shp.caches_per_task;
  const int32_t total_groups = (num_caches + lpt - 1) / lpt;
  const int64_t max_start = INT64_MAX / L.block_size - max_blocks;  // keeps (start + k) * block_size exact
  if (use_scratch) {
    // records, then partials of the task groups the schedule forms (none for one group)
    const size_t need = w.partials_off + (total_groups > 1 ? align_up(sizeof(uint64_t) * (size_t)max_items *
                                                                       (size_t)total_groups)
                                                           : 0);
    if (need > (size_t)KVCK_SCRATCH_BYTES) return KVCK_ERR_SCRATCH;
    workspace = scratch_address(dev);
    if (!workspace) return KVCK_ERR_HIP;
  }

  if (!dense && launch_plan(block_table, block_table_row_stride, num_blocks_per_req, start_pos, num_tokens,
                            num_reqs, max_blocks, L.block_size, L.num_blocks, out_stride, workspace, error_flags,
                            st) != hipSuccess)
    return KVCK_ERR_HIP;
  // The fused copy visits positions grouped by block id when each cache's pool spans at least
  // kOrderMinPoolBytes: random blocks over a large pool are what the order recovers.  Same-box
  // A/B, whole calls with the sort: llama3-shaped pools (4.8 GB per layer) save 23.27 -> 22.73 ms,
  // load 24.38 -> 23.93; GPT-2-shaped (0.9 GB), fp8 (0.45 GB) and MLA (90 MB) pools lost 0.9-3.0 %
  // on the save and within +-0.7 % on the load.  KVCK_COPY_ORDER=listing|grouped forces either
  // (results are identical).
  int32_t* order = nullptr;
  if (mode != kModeChecksum && !transposed) {
    const char* o = getenv("KVCK_COPY_ORDER");
    const int64_t pool_span = L.num_blocks * L.block_stride + (int64_t)(L.planes - 1) * L.plane_stride;
    const bool grouped = o ? strcmp(o, "listing") != 0 : pool_span >= kOrderMinPoolBytes;
    if (grouped) {
      order = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + w.order_off);
      const PosRecord* recs = reinterpret_cast<const PosRecord*>(static_cast<uint8_t*>(workspace) + w.recs_off);
      if (launch_order(recs, static_cast<const uint32_t*>(workspace), L.num_blocks, order, st) != hipSuccess)
        return KVCK_ERR_HIP;
    }
  }

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  BlocksArgs a;
  memset(&a, 0, sizeof(a));
  a.plane_stride = L.plane_stride;
  a.block_stride = L.block_stride;
  a.slot_stride = L.slot_stride;
  a.head_stride = L.head_stride;
  a.recs = reinterpret_cast<const PosRecord*>(ws + w.recs_off);
  a.n_items = reinterpret_cast<const uint32_t*>(ws);
  a.partials = reinterpret_cast<uint64_t*>(ws + w.partials_off);
  a.out = out;
  a.out_stride = out_stride;
  a.max_items = max_items;
  a.chunk_stride = L.chunk_stride;
  a.piece_base = 2ull * (uint64_t)L.plane_begin * (uint64_t)(pieces / L.planes);
  a.planes = planes_cov;
  a.planes_total = L.planes;
  a.chunks_per_run = (merged ? lane_row_bytes : run_bytes) / chunk;
  a.run_major = runs > 1 ? 1 : 0;
  a.heads = merged ? 1 : head_count;  // a merged row is one unit-level head
  a.row_bytes = L.row_bytes;
  a.pieces = (int32_t)pieces;
  a.rows_per_group = shp.rows_per_group;
  a.chunks_per_row = transposed ? (int32_t)((int64_t)L.block_size * run_bytes / chunk) : lane_row_bytes / chunk;
  a.chunks_per_head = L.row_bytes / chunk;
  a.caches_per_task = lpt;
  a.direct = total_groups == 1;
  a.accumulate = accumulate != 0;
  a.max_blocks = max_blocks;
  a.block_size = L.block_size;
  a.bt_stride = block_table_row_stride;
  a.num_blocks = L.num_blocks;
  a.max_start = max_start;
  a.block_table = block_table;
  a.nbpr = num_blocks_per_req;
  a.start_pos = start_pos;
  a.num_tokens = num_tokens;
  a.req_flags = error_flags;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = !use_scratch && instrument_pair(&ev0, &ev1);  // (an allocation-free call creates no events)
  if (timed && hipEventRecord(ev0, st) != hipSuccess) return KVCK_ERR_HIP;
  for (int32_t c0 = 0; c0 < num_caches; c0 += kCachesPerLaunch) {
    const int32_t n = num_caches - c0 < kCachesPerLaunch ? num_caches - c0 : kCachesPerLaunch;
    a.num_caches = n;
    a.group_offset = c0 / lpt;
    for (int32_t i = 0; i < n; ++i) {
      a.base[i] = static_cast<const uint8_t*>(cache_ptrs[c0 + i]) + (int64_t)head_begin * L.head_stride;
      a.mbase[i] = (uint64_t)(2 * ((int64_t)layer_numbers[c0 + i] * kH + global_head_base[c0 + i]) + 1);
    }
    const int64_t tasks = max_items * ((n + lpt - 1) / lpt);
    if (mode == kModeChecksum) {
      const int grid = transposed ? tblocks_grid(shp, dev, tasks) : blocks_grid(shp, dev, tasks);
      if (dense && (int64_t)grid * (kBlockThreads / kWave) < tasks) return KVCK_ERR_HIP;  // one wave per task
      if ((transposed ? launch_tblocks(a, shp, grid, st) : launch_blocks(a, shp, grid, st)) != hipSuccess)
        return KVCK_ERR_HIP;
    } else {
      CopyArgs ca;
      memset(&ca, 0, sizeof(ca));
      ca.b = a;
      ca.staging = static_cast<uint8_t*>(staging);
      ca.staging_positions = staging_positions;
      ca.image_bytes = image_bytes;
      ca.error_flags = error_flags;
      ca.num_caches_total = num_caches;
      ca.cache_offset = c0;
      ca.block_size = L.block_size;
      ca.order = order;
      if (transposed) {
        const int grid = tcopy_grid(shp, mode, dev, tasks, L.block_size);
        if (launch_tcopy(ca, shp, mode, grid, st) != hipSuccess) return KVCK_ERR_HIP;
      } else {
        const int grid = copy_grid(shp, mode, dev, tasks);
        if (launch_copy(ca, shp, mode, grid, st) != hipSuccess) return KVCK_ERR_HIP;
      }
    }
  }
  if (timed && hipEventRecord(ev1, st) != hipSuccess) return KVCK_ERR_HIP;
  if (total_groups > 1) {
    const hipError_t e = dense ? launch_reduce_dense(a.partials, max_items, total_groups, num_blocks_per_req,
                                                     start_pos, max_blocks, max_start, out, out_stride,
                                                     a.accumulate, st)
                               : launch_reduce(a.partials, max_items, total_groups, a.n_items, 0, a.recs, out,
                                               out_stride, a.accumulate, st);
    if (e != hipSuccess) return KVCK_ERR_HIP;
  }
  return KVCK_OK;
}
}  // namespace

KVCK_EXPORT kvck_status kvck_checksum_blocks(const kvck_kv_layout* layout, const void* const* cache_ptrs,
                                             const int32_t* layer_numbers, const int32_t* global_head_base,
                                             int32_t num_caches, int32_t head_begin, int32_t head_count,
                                             const int32_t* block_table, int64_t block_table_row_stride,
                                             const int32_t* num_blocks_per_req, const int64_t* start_pos,
                                             const int64_t* num_tokens, int32_t num_reqs, int32_t max_blocks,
                                             uint64_t* out, int64_t out_stride, int32_t accumulate,
                                             void* workspace, size_t workspace_bytes, uint32_t* error_flags,
                                             kvck_stream_t stream) {
  return blocks_call(kModeChecksum, layout, cache_ptrs, layer_numbers, global_head_base, num_caches, head_begin,
                     head_count, block_table, block_table_row_stride, num_blocks_per_req, start_pos, num_tokens,
                     num_reqs, max_blocks, out, out_stride, accumulate, workspace, workspace_bytes, error_flags,
                     nullptr, 0, stream);
}

KVCK_EXPORT kvck_status kvck_checksum_blocks_noalloc(
    const kvck_kv_layout* layout, const void* const* cache_ptrs, const int32_t* layer_numbers,
    const int32_t* global_head_base, int32_t num_caches, int32_t head_begin, int32_t head_count,
    const int32_t* block_table, int64_t block_table_row_stride, const int32_t* num_blocks_per_req,
    const int64_t* start_pos, const int64_t* num_tokens, int32_t num_reqs, int32_t max_blocks, uint64_t* out,
    int64_t out_stride, int32_t accumulate, uint32_t* error_flags, kvck_stream_t stream) {
  return blocks_call(kModeChecksum, layout, cache_ptrs, layer_numbers, global_head_base, num_caches, head_begin,
                     head_count, block_table, block_table_row_stride, num_blocks_per_req, start_pos, num_tokens,
                     num_reqs, max_blocks, out, out_stride, accumulate, nullptr, 0, error_flags, nullptr, 0, stream,
                     /*use_scratch=*/true);
}

KVCK_EXPORT kvck_status kvck_copy_checksum_blocks(int32_t direction, const kvck_kv_layout* layout,
                                                  void* const* cache_ptrs, const int32_t* layer_numbers,
                                                  const int32_t* global_head_base, int32_t num_caches,
                                                  int32_t head_begin, int32_t head_count,
                                                  const int32_t* block_table, int64_t block_table_row_stride,
                                                  const int32_t* num_blocks_per_req, const int64_t* start_pos,
                                                  const int64_t* num_tokens, int32_t num_reqs, int32_t max_blocks,
                                                  void* staging, int64_t staging_positions, uint64_t* out,
                                                  int64_t out_stride, int32_t accumulate, void* workspace,
                                                  size_t workspace_bytes, uint32_t* error_flags,
                                                  kvck_stream_t stream) {
  if (direction != KVCK_COPY_SAVE && direction != KVCK_COPY_LOAD) return KVCK_ERR_INVALID_ARGUMENT;
  return blocks_call(direction, layout, cache_ptrs, layer_numbers, global_head_base, num_caches, head_begin,
                     head_count, block_table, block_table_row_stride, num_blocks_per_req, start_pos, num_tokens,
                     num_reqs, max_blocks, out, out_stride, accumulate, workspace, workspace_bytes, error_flags,
                     staging, staging_positions, stream);
}

KVCK_EXPORT size_t kvck_staging_bytes(const kvck_kv_layout* layout, int32_t num_caches, int32_t head_count) {
  if (!layout || num_caches < 1 || head_count < 1 || (layout->planes != 1 && layout->planes != 2) ||
      layout->block_size < 1 || layout->row_bytes < 1 || layout->plane_begin < 0 || layout->plane_count < 0)
    return 0;
  const int64_t planes =
      layout->plane_count > 0 ? layout->plane_count : (int64_t)layout->planes - layout->plane_begin;
  if (planes < 1 || (int64_t)layout->plane_begin + planes > layout->planes) return 0;
  const int64_t image = planes * head_count * (int64_t)layout->block_size;  // < 2^2 * 2^31 * 2^31
  if (!product_ok(image, layout->row_bytes, num_caches)) return 0;
  return (size_t)(image * layout->row_bytes * num_caches);
}

namespace {
constexpr int32_t kRowsPerTask = 8;
int32_t row_groups(int32_t row_count) { return (int32_t)(((int64_t)row_count + kRowsPerTask - 1) / kRowsPerTask); }
}  // namespace

KVCK_EXPORT size_t kvck_states_workspace_bytes(int32_t num_layers, int32_t row_count, int32_t num_reqs) {
  if (num_layers < 1 || row_count < 1 || num_reqs < 0) return 0;
  const int64_t splits = (int64_t)num_layers * row_groups(row_count);
  int64_t items = 0;  // a batch the entry point rejects
  if (__builtin_mul_overflow(splits, (int64_t)num_reqs, &items) || items >= ((int64_t)1 << 40)) return 0;
  return kAlign + (splits > 1 ? align_up(sizeof(uint64_t) * (size_t)splits * (size_t)num_reqs) : 0);
}

KVCK_EXPORT kvck_status kvck_checksum_states(const kvck_state_desc* states, int32_t states_per_layer,
                                             const void* const* state_ptrs, const int32_t* layer_numbers,
                                             const int32_t* global_row_base, int32_t num_layers, int32_t num_slots,
                                             int32_t num_rows, int32_t row_begin, int32_t row_count,
                                             const int32_t* slot_ids, int32_t num_reqs, uint64_t* out,
                                             int64_t out_stride, int32_t accumulate, void* workspace,
                                             size_t workspace_bytes, uint32_t* error_flags, kvck_stream_t stream) {
  if (!states || !state_ptrs || !layer_numbers || !global_row_base) return KVCK_ERR_INVALID_ARGUMENT;
  if (states_per_layer < 1 || states_per_layer > KVCK_MAX_STATES_PER_LAYER) return KVCK_ERR_UNSUPPORTED;
  if (num_layers < 1 || num_layers > KVCK_MAX_CACHES) return KVCK_ERR_UNSUPPORTED;
  if (num_slots < 1 || num_rows < 1 || row_begin < 0 || row_count < 1 || (int64_t)row_begin + row_count > num_rows)
    return KVCK_ERR_INVALID_ARGUMENT;
  int64_t elems = 0;
  for (int32_t i = 0; i < states_per_layer; ++i) {
    const kvck_state_desc& d = states[i];
    if (d.row_elems < 1 || d.slot_stride < 0 || d.row_stride < 0) return KVCK_ERR_INVALID_ARGUMENT;
    if (d.elem_bytes != 2 && d.elem_bytes != 4) return KVCK_ERR_UNSUPPORTED;
    if (((int64_t)d.row_elems * d.elem_bytes) % 16 != 0) return KVCK_ERR_UNSUPPORTED;
    if (d.slot_stride % 16 != 0 || d.row_stride % 16 != 0) return KVCK_ERR_MISALIGNED;
    if (!extent_ok({{num_slots, d.slot_stride}, {num_rows, d.row_stride}}, (int64_t)d.row_elems * d.elem_bytes))
      return KVCK_ERR_UNSUPPORTED;
    elems += d.row_elems;
  }
  if (elems >= ((int64_t)1 << 31) - 8) return KVCK_ERR_UNSUPPORTED;
  for (int32_t l = 0; l < num_layers; ++l) {
    if (layer_numbers[l] < 0 || global_row_base[l] < 0) return KVCK_ERR_INVALID_ARGUMENT;
    if ((int64_t)global_row_base[l] + row_count > kH) return KVCK_ERR_UNSUPPORTED;
    for (int32_t i = 0; i < states_per_layer; ++i) {
      const void* p = state_ptrs[(int64_t)l * states_per_layer + i];
      if (!p) return KVCK_ERR_INVALID_ARGUMENT;
      if (!aligned(p, 16)) return KVCK_ERR_MISALIGNED;
    }
  }
  if (num_reqs < 0) return KVCK_ERR_INVALID_ARGUMENT;
  if (out_stride < 1 || out_stride > KVCK_MAX_OUT_STRIDE) return KVCK_ERR_INVALID_ARGUMENT;
  if (num_reqs == 0) return KVCK_OK;
  if (!slot_ids || !out) return KVCK_ERR_INVALID_ARGUMENT;
  if (!aligned(slot_ids, 4) || !aligned(out, 8) || (error_flags && !aligned(error_flags, 4)))
    return KVCK_ERR_MISALIGNED;
  const int32_t groups = row_groups(row_count);
  const int64_t splits = (int64_t)num_layers * groups;
  int64_t items = 0;
  if (__builtin_mul_overflow(splits, (int64_t)num_reqs, &items) || items >= ((int64_t)1 << 40))
    return KVCK_ERR_UNSUPPORTED;
  const size_t need = kvck_states_workspace_bytes(num_layers, row_count, num_reqs);
  if (splits > 1 && (!workspace || workspace_bytes < need || !aligned(workspace, (int64_t)kAlign)))
    return KVCK_ERR_WORKSPACE;

  int dev = 0;
  const kvck_status ds = current_device(&dev);
  if (ds != KVCK_OK) return ds;
  hipStream_t st = static_cast<hipStream_t>(stream);

  StatesArgs a;
  memset(&a, 0, sizeof(a));
  int32_t eoff = 0;
  for (int32_t i = 0; i < states_per_layer; ++i) {
    a.slot_stride[i] = states[i].slot_stride;
    a.row_stride[i] = states[i].row_stride;
    a.row_chunks[i] = (int32_t)((int64_t)states[i].row_elems * states[i].elem_bytes / 16);
    a.elem_bytes[i] = states[i].elem_bytes;
    a.elem_off[i] = eoff;
    eoff += states[i].row_elems;
  }
  a.slot_ids = slot_ids;
  a.partials = splits > 1 ? reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) + kAlign) : nullptr;
  a.out = out;
  a.out_stride = out_stride;
  a.error_flags = error_flags;
  a.nstates = states_per_layer;
  a.num_slots = num_slots;
  a.num_reqs = num_reqs;
  a.row_begin = row_begin;
  a.row_count = row_count;
  a.rows_per_task = kRowsPerTask;
  a.groups_per_layer = groups;
  a.direct = splits == 1;
  a.accumulate = accumulate != 0;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const bool timed = instrument_pair(&ev0, &ev1);
  if (timed && hipEventRecord(ev0, st) != hipSuccess) return KVCK_ERR_HIP;
  for (int32_t l0 = 0; l0 < num_layers; l0 += kLayersPerStatesLaunch) {
    const int32_t n = num_layers - l0 < kLayersPerStatesLaunch ? num_layers - l0 : kLayersPerStatesLaunch;
    a.num_layers = n;
    a.split_offset = l0 * groups;
    for (int32_t l = 0; l < n; ++l) {
      for (int32_t i = 0; i < states_per_layer; ++i)
        a.ptr[l][i] = static_cast<const uint8_t*>(state_ptrs[(int64_t)(l0 + l) * states_per_layer + i]);
      a.mbase[l] = (uint64_t)(2 * ((int64_t)layer_numbers[l0 + l] * kH + global_row_base[l0 + l]) + 1);
    }
    const int grid = states_grid(dev, (int64_t)n * groups * num_reqs);
    if (launch_states(a, grid, st) != hipSuccess) return KVCK_ERR_HIP;
  }
  if (timed && hipEventRecord(ev1, st) != hipSuccess) return KVCK_ERR_HIP;
  if (splits > 1) {
    if (launch_reduce(a.partials, num_reqs, (int32_t)splits, nullptr, num_reqs, nullptr, out, out_stride,
                      a.accumulate, st) != hipSuccess)
      return KVCK_ERR_HIP;
  }
  return KVCK_OK;
}

KVCK_EXPORT kvck_status kvck_tag_checksums(const uint64_t* checksums, int32_t columns, const uint8_t* block_hashes,
                                           int64_t hash_stride, uint64_t fingerprint, int64_t n,
                                           const int32_t* num_blocks_per_req,
                                           const int64_t* start_pos, int32_t max_blocks, int32_t block_size,
                                           uint64_t* tagged, const uint64_t* stored, uint8_t* mismatch,
                                           uint32_t* mismatch_count, kvck_stream_t stream) {
  if (n < 0) return KVCK_ERR_INVALID_ARGUMENT;
  if (n == 0) return KVCK_OK;
  if (!checksums || !block_hashes) return KVCK_ERR_INVALID_ARGUMENT;
  if (columns < 1 || columns > KVCK_MAX_OUT_STRIDE) return KVCK_ERR_INVALID_ARGUMENT;
  if (!tagged && !stored) return KVCK_ERR_INVALID_ARGUMENT;       // nothing to do
  if ((mismatch || mismatch_count) && !stored) return KVCK_ERR_INVALID_ARGUMENT;
  if (hash_stride < 8) return KVCK_ERR_INVALID_ARGUMENT;
  if (hash_stride % 8 != 0 || !aligned(block_hashes, 8) || !aligned(checksums, 8) || !aligned(tagged, 8) ||
      !aligned(stored, 8) || !aligned(mismatch_count, 4))
    return KVCK_ERR_MISALIGNED;
  if (!extent_ok({{n, hash_stride}}, 8) || !extent_ok({{n, (int64_t)columns * 8}}, 8)) return KVCK_ERR_UNSUPPORTED;
  if (num_blocks_per_req && (max_blocks < 1 || n % max_blocks != 0)) return KVCK_ERR_INVALID_ARGUMENT;
  if (start_pos && (!num_blocks_per_req || block_size < 1)) return KVCK_ERR_INVALID_ARGUMENT;
  if ((num_blocks_per_req && !aligned(num_blocks_per_req, 4)) || (start_pos && !aligned(start_pos, 8)))
    return KVCK_ERR_MISALIGNED;
  // the start positions kvck_checksum_blocks accepts: (start + k) * block_size stays exact
  const int64_t max_start = start_pos ? INT64_MAX / block_size - max_blocks : INT64_MAX;
  int dev = 0;
  const kvck_status ds = current_device(&dev);
  if (ds != KVCK_OK) return ds;
  if (launch_tags(checksums, columns, block_hashes, hash_stride, fingerprint, n, num_blocks_per_req, start_pos,
                  max_blocks, max_start, tagged, stored, mismatch, mismatch_count,
                  static_cast<hipStream_t>(stream)) != hipSuccess)
    return KVCK_ERR_HIP;
  return KVCK_OK;
}

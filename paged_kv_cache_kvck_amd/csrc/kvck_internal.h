// Internal declarations of libkvck: kernel argument blocks, workspace layout
// and launchers.  Not part of the ABI (see include/kvck.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvck.h"

namespace kvck {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;          // 4 independent waves per workgroup
constexpr int kCachesPerLaunch = 64;        // caches carried in one argument block
// Workgroups per CU of a planned checksum main pass (fewer than fit): one
// wave per SIMD, each with two units of loads in flight.  Against full
// occupancy, interleaved on one GPU over every pool shape measured: never
// slower, 1-1.5 points of 8 TB/s faster on the large pools; fewer streams
// read faster once each one is double-buffered.
constexpr int kMainWorkgroupsPerCU = 1;
constexpr int kAllThatFit = 1 << 20;  // workgroups_per_cu: as many as fit
constexpr int kLayersPerStatesLaunch = 32;  // Mamba layers carried in one argument block
constexpr size_t kAlign = 256;
// Checksum calls of at most this many (slot, cache) tasks plan in place: the
// dense kernel variants run one task per wave, in grids of at most
// kDenseMaxTasks / 4 workgroups.
constexpr int64_t kDenseMaxTasks = 8192;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// One listed block position, built on the device from the request arrays.
struct alignas(16) PosRecord {
  int64_t t0;       // first token the position holds: pos * block_size
  int64_t out_idx;  // (r * max_blocks + k) * out_stride: the position's output element
  int32_t block;    // physical block id
  int32_t valid;    // slots to checksum (0: none, or a bad id)
  int64_t pad;
};
static_assert(sizeof(PosRecord) == 32, "record is 32 bytes");

// Workspace of kvck_checksum_blocks:
//   [header 256 B: uint32 n_items] [prefix int32 x (R+1)] [records] [partials] [order int32 x R*max_blocks]
struct BlocksWorkspace {
  size_t prefix_off, recs_off, partials_off, order_off, total;
  static BlocksWorkspace make(int32_t num_caches, int32_t num_reqs, int32_t max_blocks) {
    BlocksWorkspace w;
    const size_t items = (size_t)num_reqs * (size_t)max_blocks;
    w.prefix_off = kAlign;
    w.recs_off = w.prefix_off + align_up(sizeof(int32_t) * ((size_t)num_reqs + 1));
    w.partials_off = w.recs_off + align_up(sizeof(PosRecord) * items);
    w.order_off = w.partials_off + (num_caches > 1 ? align_up(sizeof(uint64_t) * items * (size_t)num_caches) : 0);
    w.total = w.order_off + align_up(sizeof(int32_t) * items);  // the fused copy's visiting order
    return w;
  }
};

// Per-launch arguments of the paged K/V kernel (passed by value).
struct BlocksArgs {
  int64_t plane_stride, block_stride, slot_stride, head_stride;  // bytes
  const PosRecord* recs;
  const uint32_t* n_items;   // device: listed positions
  uint64_t* partials;        // [num_caches][max_items] when not direct
  uint64_t* out;
  int64_t out_stride;                        // elements between consecutive slots' outputs
  int64_t max_items;
  int64_t chunk_stride;                      // bytes between a row's contiguous runs
  uint64_t piece_base;                       // 2 * (first covered plane) * pieces per plane
  int32_t planes, heads, row_bytes, pieces;  // planes covered by the call; pieces = P per token
  int32_t planes_total;                      // planes of the slice
  int32_t rows_per_group;                    // rows covered by one lane table
  int32_t chunks_per_row;
  int32_t chunks_per_head;                   // chunks of one head's row (< chunks_per_row: merged heads)
  int32_t chunks_per_run;                    // lane chunks in one contiguous run of a row
  int32_t run_major;                         // rows stored as several runs: lanes walk [run][row]
  int32_t num_caches;                        // caches in this launch
  int32_t caches_per_task;                   // caches one task covers (a partial's group)
  int32_t group_offset;                      // partial row of this launch's first group
  int32_t direct;                            // write out[] directly (one group overall)
  int32_t accumulate;
  const uint8_t* base[kCachesPerLaunch];     // pool base + head_begin*head_stride
  uint64_t mbase[kCachesPerLaunch];          // 2*(layer*H + global_head_base) + 1 (< 2^48)
  // Calls planned in place (the dense kernel variants): tasks index every
  // (r, k) slot, item = r*max_blocks + k, and read the request arrays
  // themselves; recs and n_items are then unused.
  int32_t max_blocks, block_size;
  int64_t bt_stride, num_blocks, max_start;
  const int32_t* block_table;
  const int32_t* nbpr;
  const int64_t* start_pos;
  const int64_t* num_tokens;
  uint32_t* req_flags;                       // error word for bad requests and ids (may be null)
};

// Arguments of the fused copy + checksum kernel.
struct CopyArgs {
  BlocksArgs b;              // pool side, records, caches, outputs
  uint8_t* staging;          // device: entries x caches x block images
  int64_t staging_positions; // capacity in entries (listed positions)
  int64_t image_bytes;       // planes * heads * block_size * row_bytes
  uint32_t* error_flags;
  int32_t num_caches_total;  // caches of the call (images per entry)
  int32_t cache_offset;      // global index of this launch's first cache
  int32_t block_size;
  const int32_t* order;      // listed positions in visiting order (null: listing order)
};

struct StatesArgs {
  int64_t slot_stride[KVCK_MAX_STATES_PER_LAYER];
  int64_t row_stride[KVCK_MAX_STATES_PER_LAYER];
  int32_t row_chunks[KVCK_MAX_STATES_PER_LAYER];  // 16-byte chunks per row
  int32_t elem_bytes[KVCK_MAX_STATES_PER_LAYER];
  int32_t elem_off[KVCK_MAX_STATES_PER_LAYER];    // element number of the row's first element
  const int32_t* slot_ids;
  uint64_t* partials;  // [splits][num_reqs]
  uint64_t* out;
  int64_t out_stride;  // elements between consecutive requests' outputs
  uint32_t* error_flags;
  int32_t nstates, num_layers, num_slots, num_reqs;
  int32_t row_begin, row_count, rows_per_task, groups_per_layer;
  int32_t split_offset;  // split index of this launch's first (layer, group)
  int32_t direct, accumulate;
  const uint8_t* ptr[kLayersPerStatesLaunch][KVCK_MAX_STATES_PER_LAYER];
  uint64_t mbase[kLayersPerStatesLaunch];  // 2*(layer*H + global_row_base) + 1 (< 2^48)
};

// Kernel shape chosen on the host for one kvck_checksum_blocks call.
struct BlocksShape {
  int chunk;      // 16 or 8 bytes per lane load
  int slots;      // lane-table slots S (1, 2, 4, 8, 16)
  int rows_per_group;
  bool pipelined; // two unit buffers in flight, several caches per task
  int caches_per_task;
  int planes_per_unit;  // 1, or 2 (K and V in one unit) when heads are few
  bool merged;          // a lane-table row is a slot's adjacent heads (NHD-like pools)
  int copy_buffers;     // fused copy: 1 = one unit buffer (more resident waves), 2 = ping-pong
  bool transposed;      // rows stored element by element (elements of a row elem_stride apart)
  int elem_bytes;       // element size of transposed rows (1, 2 or 4)
  bool dense;           // planned in place: tasks read the request arrays (kernel variant)
  bool lds_transpose;   // fused copy of transposed planes: transpose staged through LDS
};

// launchers (return hipSuccess or the first HIP error)
hipError_t launch_plan(const int32_t* block_table, int64_t bt_stride, const int32_t* nbpr,
                       const int64_t* start_pos, const int64_t* num_tokens, int32_t num_reqs,
                       int32_t max_blocks, int32_t block_size, int64_t num_blocks, int64_t out_stride,
                       void* workspace, uint32_t* error_flags, hipStream_t stream);
hipError_t launch_blocks(const BlocksArgs& a, const BlocksShape& shp, int grid, hipStream_t stream);
int blocks_grid(const BlocksShape& shp, int device, int64_t max_tasks);
hipError_t launch_reduce(const uint64_t* partials, int64_t stride, int32_t splits, const uint32_t* n_items,
                         int64_t n_fixed, const PosRecord* recs, uint64_t* out, int64_t out_stride,
                         int32_t accumulate, hipStream_t stream);
hipError_t launch_reduce_dense(const uint64_t* partials, int64_t stride, int32_t splits, const int32_t* nbpr,
                               const int64_t* start_pos, int32_t max_blocks, int64_t max_start, uint64_t* out,
                               int64_t out_stride, int32_t accumulate, hipStream_t stream);
hipError_t launch_states(const StatesArgs& a, int grid, hipStream_t stream);
hipError_t launch_tblocks(const BlocksArgs& a, const BlocksShape& shp, int grid, hipStream_t stream);
int tblocks_grid(const BlocksShape& shp, int device, int64_t max_tasks);
hipError_t launch_copy(const CopyArgs& a, const BlocksShape& shp, int direction, int grid, hipStream_t stream);
hipError_t launch_order(const PosRecord* recs, const uint32_t* n_items, int64_t num_blocks, int32_t* order,
                        hipStream_t stream);
int copy_grid(const BlocksShape& shp, int direction, int device, int64_t max_tasks);
hipError_t launch_tcopy(const CopyArgs& a, const BlocksShape& shp, int direction, int grid, hipStream_t stream);
int tcopy_grid(const BlocksShape& shp, int direction, int device, int64_t max_tasks, int32_t block_size);
hipError_t launch_tags(const uint64_t* checksums, int32_t columns, const uint8_t* hashes, int64_t hash_stride,
                       uint64_t fingerprint, int64_t n, const int32_t* nbpr, const int64_t* start_pos, int32_t max_blocks,
                       int64_t max_start, uint64_t* tagged, const uint64_t* stored, uint8_t* mismatch,
                       uint32_t* count, hipStream_t stream);
int states_grid(int device, int64_t tasks);
int device_cus(int device);                                   // cached per device
int kernel_occupancy(const void* fn, int device, int fallback);  // workgroups per CU, cached
int workgroups_per_cu(int fits, int preferred);                  // what a launch uses of `fits`

}  // namespace kvck

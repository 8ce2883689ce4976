/*
 * kvck.h -- C ABI of libkvck: connector-agnostic checksums of paged KV-cache
 * blocks on AMD Instinct MI355X (gfx950).
 *
 * The checksum is the one defined on the vLLM API page
 * "vllm.distributed.kv_transfer.kv_checksum.checksum" (module docstring):
 *
 *   item 1  For each (layer, KV head) of a block, the K bytes then the V bytes
 *           of every token, in token order, form a slice; it is read as
 *           little-endian uint64 pieces x_j, j = t*P + p for the p-th piece
 *           of the token at request position t (P pieces per token), and
 *               s(layer, head) = sum over j of x_j (2j + 1)        mod 2^64
 *   item 2  The block position's checksum weighs each slice by an odd factor:
 *               c = sum over (layer, head) of m s(layer, head)     mod 2^64
 *               m = 2 (layer * 65536 + global head) + 1
 *   Mamba   For a Mamba group the request's running state takes the place of
 *           its blocks (position 0); each global row of the layer's states is
 *           a slice, its pieces the 2- or 4-byte elements as unsigned ints.
 *
 * Conventions shared by every entry point:
 *  - Pointers marked "device" are HIP device pointers on the current device;
 *    pointers marked "host" are read during the call only.  The library
 *    allocates no memory and keeps no pointer after it returns; the caller
 *    owns every buffer.
 *  - Calls are asynchronous and ordered on `stream`.  Results are valid once
 *    the stream has reached the call; the cache bytes must not change until
 *    then (a checksum only means something once the KV is complete).
 *  - A negative return value means the call launched nothing.  Errors found
 *    only on the device (a bad block id, a bad request entry, a bad state
 *    slot) are reported by OR-ing KVCK_FLAG_* bits into *error_flags (if not
 *    NULL); the library never clears that word.
 *  - All checksum arithmetic is unsigned 64-bit integer arithmetic; results
 *    are bit-exact and independent of launch shape and scheduling.
 *  - Thread-safe; calls that share a workspace must be stream-ordered.
 */
#ifndef KVCK_H_
#define KVCK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVCK_ABI_VERSION 3

/* The page attribute MAX_KV_HEADS_PER_LAYER (2^16): H of the slice factor and
 * a bound on a layer's KV heads (or Mamba rows); calls beyond it are refused. */
#define KVCK_MAX_KV_HEADS_PER_LAYER 65536
/* Largest accepted layer number: any non-negative int32.  The page numbers a
 * layer by the number in its name, with no bound; the factor
 * m = 2(layer*H + head) + 1 stays below 2^48 and is carried in 64 bits. */
#define KVCK_MAX_LAYER_NUMBER 2147483647
/* Caches (layers) per kvck_checksum_blocks call and Mamba layers per
 * kvck_checksum_states call. */
#define KVCK_MAX_CACHES 4096
/* States per Mamba layer. */
#define KVCK_MAX_STATES_PER_LAYER 4
/* Largest out_stride of the checksum entry points and `columns` of
 * kvck_tag_checksums: the number of replica-key columns a partial result may
 * have (see "Replica columns" below). */
#define KVCK_MAX_OUT_STRIDE 65536

/*
 * Replica columns.  The checksum page (module docstring; attribute ReplicaKey;
 * class KVChecksumGroup) keys a worker's partial checksums by the
 * (replicas, replica_index) of the layers they cover, so that replicated KV
 * (MLA, or GQA on more TP ranks than KV heads) is compared replica by
 * replica: a group's values are (num_positions, len(replica_keys)), one column
 * per key, and what is offloaded with a block is its row summed.  Every
 * checksum entry point writes its results out_stride elements apart, so with
 * out_stride = C and out at element c of a row-major [..., C] array a call
 * fills column c; a worker makes one call per replica key, over that key's
 * caches, each into its own column.  out_stride = 1 is a dense array.
 */

typedef enum kvck_status {
  KVCK_OK = 0,
  KVCK_ERR_INVALID_ARGUMENT = -1, /* null pointer, negative size, bad stride */
  KVCK_ERR_UNSUPPORTED = -2,      /* > H heads/rows, row bytes not a multiple of 8, element
                                     width not 2 or 4, too many caches, a
                                     tensor whose strided byte extent reaches
                                     2^50 (pool, state, staging, hashes) */
  KVCK_ERR_MISALIGNED = -3,       /* base pointer or stride not 8-byte aligned, or an array
                                     not aligned to its element size */
  KVCK_ERR_WORKSPACE = -4,        /* workspace missing or too small */
  KVCK_ERR_HIP = -5,              /* a HIP runtime call failed */
  KVCK_ERR_NO_DEVICE = -6,        /* no gfx950 device is current */
  KVCK_ERR_SCRATCH = -7           /* an allocation-free call needs more than
                                     KVCK_SCRATCH_BYTES of scratch */
} kvck_status;

/* Bits OR-ed into *error_flags by the kernels. */
#define KVCK_FLAG_BAD_BLOCK_ID 1u   /* a position with valid slots names a block
                                       outside [0, num_blocks); it contributes 0 */
#define KVCK_FLAG_BAD_REQUEST 2u    /* num_blocks_per_req outside [0, max_blocks]
                                       or start_pos < 0; the request is skipped */
#define KVCK_FLAG_BAD_STATE_SLOT 4u /* a Mamba slot id outside [0, num_slots);
                                       the request's value is 0 */
#define KVCK_FLAG_STAGING_FULL 8u   /* a listed position past the staging capacity:
                                       neither copied nor checksummed (value 0) */

/* Directions of kvck_copy_checksum_blocks. */
#define KVCK_COPY_SAVE 0 /* paged pool -> staging buffer */
#define KVCK_COPY_LOAD 1 /* staging buffer -> paged pool */

/* A hipStream_t; NULL is the null stream. */
typedef void* kvck_stream_t;

/*
 * Byte layout of one layer's paged KV pool, shared by every cache of a call.
 * A row is the head_size elements of one (plane, block, slot, head) and must
 * be contiguous; its address is
 *   base + plane*plane_stride + block*block_stride + slot*slot_stride + head*head_stride.
 * vLLM NHD pool (2, num_blocks, block_size, num_heads, head_size) (page
 * "[vLLM 源码解析] KV Cache", section "reshape kv_cache") and the head-major HND
 * pool (2, num_blocks, num_heads, block_size, head_size) are two stride sets
 * of this struct; an MLA latent pool (num_blocks, block_size, head_size) has
 * planes = 1, num_heads = 1.
 */
typedef struct kvck_kv_layout {
  int32_t planes;       /* planes of a token's slice: 2 = K then V; 1 = one latent plane */
  int32_t block_size;   /* slots per block, >= 1 */
  int32_t num_heads;    /* KV heads held by the pool tensor, >= 1 */
  int32_t row_bytes;    /* head_size * element bytes; multiple of 8 */
  int64_t num_blocks;   /* blocks in the pool; valid ids are [0, num_blocks) */
  int64_t plane_stride; /* bytes between the planes the call covers */
  int64_t block_stride; /* bytes */
  int64_t slot_stride;  /* bytes */
  int64_t head_stride;  /* bytes; ignored when num_heads == 1 */
  /* Optional (0 = default).  A row stored as contiguous runs of chunk_bytes
   * (a multiple of 8 dividing row_bytes), consecutive runs chunk_stride bytes
   * apart -- e.g. the x-split K layout [num_blocks, num_heads, head_size/x,
   * block_size, x] (page "[vLLM 源码解析] KV Cache", the reshape_and_cache
   * section): chunk_bytes = x*element bytes, chunk_stride = block_size*x*
   * element bytes, slot_stride = x*element bytes.  0: the row is contiguous.
   * chunk_bytes of 1, 2 or 4 (one element per run) describes an
   * element-transposed plane [num_blocks, num_heads, head_size, block_size]
   * (the V layout of ROCm's paged-attention kernels): chunk_stride =
   * block_size*element bytes, slot_stride = chunk_bytes.  Such calls cover one
   * plane (plane_count 1) and need block_size*element bytes to be a multiple
   * of 8; kvck_copy_checksum_blocks also needs block_size <= 1024
   * (KVCK_ERR_UNSUPPORTED otherwise). */
  int32_t chunk_bytes;
  int32_t reserved0;
  int64_t chunk_stride;
  /* Optional: the call covers planes plane_begin .. plane_begin+plane_count-1
   * of the slice (plane_count 0 = all planes).  Pieces keep their numbering
   * in the whole slice, so calls over K and over V (e.g. separate K and V
   * tensors, each its own cache_ptrs) add up to the checksum of both; the
   * cache pointers address the call's first plane. */
  int32_t plane_begin;
  int32_t plane_count;
} kvck_kv_layout;

/*
 * kvck_checksum_blocks -- per block position checksums of paged K/V.
 *
 * A token's slice bytes are its K row then its V row (planes == 2) or its
 * latent row (planes == 1); P = planes*row_bytes/8.  Request r lists
 * num_blocks_per_req[r] blocks, block_table[r*block_table_row_stride + k]
 * at block position start_pos[r] + k (as the page's KVChecksumBlocks gives a
 * start position and then one block id per following position); position pos
 * holds tokens pos*block_size .. +block_size-1 of the request, and slots at
 * or past num_tokens[r] are not checksummed.
 *
 * Caches: cache_ptrs[i] (host array of device pointers) is layer
 * layer_numbers[i]; the call covers its local heads head_begin ..
 * head_begin+head_count-1, and local head head_begin+k is global head
 * global_head_base[i]+k (TP shard: a subset of heads with global numbering;
 * PP stage: a subset of layers -- partial results sum to the full value).
 *
 * Output: out[(r*max_blocks + k)*out_stride] (device, uint64) for every
 * listed position k < num_blocks_per_req[r]; other entries are not written.
 * out_stride is 1..KVCK_MAX_OUT_STRIDE (one replica column of C: C).  With
 * accumulate != 0 the checksum is added (mod 2^64) to what out holds.
 *
 * Workspace: device, at least kvck_blocks_workspace_bytes(num_caches,
 * num_reqs, max_blocks) bytes, 256-byte aligned; its contents on entry are
 * ignored.  kvck_blocks_workspace_bytes returns 0 for arguments the entry
 * points reject (num_caches < 1, negative sizes, num_reqs*max_blocks >= 2^31).
 *
 * Schedule: pools of rows run one workgroup of four wavefronts per compute
 * unit (element-transposed planes: as many as fit).  Large batches (many
 * tasks per resident wavefront) keep two load batches in flight per
 * wavefront and give each task several layers; small ones use one layer per
 * task.  The environment variable KVCK_SCHEDULE =
 * "pipelined" or "simple" forces one of the two; results are bit-identical.
 * Calls of at most 8192 (request slot, cache) pairs read the request arrays
 * in the main pass itself (no separate planning launch; the smallest run as a
 * single launch); KVCK_PLAN = "compact" turns this off, with identical
 * results and error bits.  Either way block_table entries k < max_blocks of
 * every row may be read, and only listed, valid ones are used.
 *
 * Other switches, read at each call, that change how the work is done but
 * never the results: KVCK_MERGE_HEADS = "0" / "1" (read a slot's heads as one
 * row: automatic for rows under 128 bytes and single heads), KVCK_MERGED_PIPE
 * = "0" (merged rows unpipelined), KVCK_COPY_BUFFERS = "1" / "2" (fused copy
 * with one or two load buffers per wave; the default is two for a save, one
 * for a load), KVCK_TCOPY = "regs" (fused copy of
 * element-transposed planes transposed in registers instead of through LDS),
 * KVCK_COPY_ORDER = "listing" / "grouped" (fused copy of row layouts visits
 * positions in listing order, or grouped by block id; by default grouped when
 * each cache's pool spans at least 2 GiB), KVCK_GRID_PER_CU = n
 * (workgroups per compute unit of every launch, up to what fits).
 */
kvck_status kvck_checksum_blocks(
    const kvck_kv_layout* layout,          /* host */
    const void* const* cache_ptrs,         /* host [num_caches] of device pointers */
    const int32_t* layer_numbers,          /* host [num_caches], 0..KVCK_MAX_LAYER_NUMBER */
    const int32_t* global_head_base,       /* host [num_caches] */
    int32_t num_caches,                    /* 1..KVCK_MAX_CACHES */
    int32_t head_begin, int32_t head_count,
    const int32_t* block_table,            /* device [num_reqs, block_table_row_stride] */
    int64_t block_table_row_stride,        /* elements, >= max_blocks */
    const int32_t* num_blocks_per_req,     /* device [num_reqs] */
    const int64_t* start_pos,              /* device [num_reqs] */
    const int64_t* num_tokens,             /* device [num_reqs] */
    int32_t num_reqs, int32_t max_blocks,
    uint64_t* out,                         /* device [num_reqs * max_blocks * out_stride] */
    int64_t out_stride,                    /* elements, 1..KVCK_MAX_OUT_STRIDE */
    int32_t accumulate,
    void* workspace, size_t workspace_bytes,
    uint32_t* error_flags,                 /* device, optional */
    kvck_stream_t stream);

size_t kvck_blocks_workspace_bytes(int32_t num_caches, int32_t num_reqs, int32_t max_blocks);

/*
 * kvck_checksum_blocks_noalloc -- kvck_checksum_blocks for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments and results, without
 * the workspace.  In its place the call uses a scratch array of
 * KVCK_SCRATCH_BYTES that the library holds on each device it runs on, from
 * the first such call until the process ends.  The call allocates nothing
 * and records no events (instrumentation does not time it).  Its first call
 * on a device also looks up that array's device address (a runtime query,
 * no allocation): make one call on the device before capturing the call
 * into a HIP graph.
 *
 * It needs the plan's position records (32 bytes per num_reqs*max_blocks
 * slot, plus a few KiB) and, when its caches form more than one task group
 * (one group covers one to sixteen caches, whichever the schedule picks), 8
 * bytes per slot and group; a call that would need more than
 * KVCK_SCRATCH_BYTES returns KVCK_ERR_SCRATCH and launches nothing.  Any call
 * with kvck_blocks_workspace_bytes(num_caches, num_reqs, max_blocks) <=
 * KVCK_SCRATCH_BYTES fits.  Nothing in the scratch has to start at any
 * value: every call writes what it later reads.
 *
 * All such calls on one device share its scratch array, so calls that
 * overlap on one device -- on different streams, or from different host
 * threads without ordering them on one stream -- race and give wrong
 * results; calls ordered on one stream do not.
 */
#define KVCK_SCRATCH_BYTES (32u << 20)
kvck_status kvck_checksum_blocks_noalloc(
    const kvck_kv_layout* layout, const void* const* cache_ptrs, const int32_t* layer_numbers,
    const int32_t* global_head_base, int32_t num_caches, int32_t head_begin, int32_t head_count,
    const int32_t* block_table, int64_t block_table_row_stride, const int32_t* num_blocks_per_req,
    const int64_t* start_pos, const int64_t* num_tokens, int32_t num_reqs, int32_t max_blocks,
    uint64_t* out, int64_t out_stride, int32_t accumulate, uint32_t* error_flags, kvck_stream_t stream);

/*
 * Shape of one Mamba state, shared by every Mamba layer of a call.  A state
 * tensor is (num_slots, num_rows, ...); the row is the TP-split dimension and
 * its row_elems elements must be contiguous.
 */
typedef struct kvck_state_desc {
  int64_t slot_stride;  /* bytes between state slots */
  int64_t row_stride;   /* bytes between rows */
  int32_t row_elems;    /* elements per row */
  int32_t elem_bytes;   /* 2 or 4 (read unsigned) */
} kvck_state_desc;

/*
 * kvck_checksum_states -- Mamba running-state checksums (position 0).
 *
 * Slice g of a Mamba layer is local row row_begin+g (global row
 * global_row_base[l]+g) of every state of the layer, concatenated in the
 * order of `states`, elements numbered from 0 across the concatenation:
 *   s = sum_e x_e (2e + 1),  c = sum_{layer, g} m * s,  m = 2(layer*H + g_global) + 1.
 * Request r's state slot is slot_ids[r]; out[r*out_stride] receives its
 * checksum (added to what it holds when accumulate != 0).
 *
 * state_ptrs holds num_layers*states_per_layer device pointers, layer-major
 * (state_ptrs[l*states_per_layer + i] is state i of layer l).
 * Workspace: device, kvck_states_workspace_bytes(num_layers, row_count,
 * num_reqs) bytes, 256-byte aligned (that function returns 0 for arguments
 * the entry point rejects).
 */
kvck_status kvck_checksum_states(
    const kvck_state_desc* states, int32_t states_per_layer,  /* host [states_per_layer], 1..4 */
    const void* const* state_ptrs,         /* host [num_layers*states_per_layer] of device pointers */
    const int32_t* layer_numbers,          /* host [num_layers] */
    const int32_t* global_row_base,        /* host [num_layers] */
    int32_t num_layers,
    int32_t num_slots, int32_t num_rows,   /* extent of every state tensor */
    int32_t row_begin, int32_t row_count,
    const int32_t* slot_ids,               /* device [num_reqs] */
    int32_t num_reqs,
    uint64_t* out,                         /* device [num_reqs * out_stride] */
    int64_t out_stride,                    /* elements, 1..KVCK_MAX_OUT_STRIDE */
    int32_t accumulate,
    void* workspace, size_t workspace_bytes,
    uint32_t* error_flags,                 /* device, optional */
    kvck_stream_t stream);

size_t kvck_states_workspace_bytes(int32_t num_layers, int32_t row_count, int32_t num_reqs);

/*
 * kvck_copy_checksum_blocks -- a connector's save or load of paged K/V fused
 * with the checksum: every valid row is read once and written once, and the
 * checksums of kvck_checksum_blocks come out of the same pass (all its
 * arguments mean the same; on a load the pool is written).
 *
 * The two directions are the worker-side connector calls of the page
 * "Connector.md", section 2.1 (worker side): save_kv_layer, which after a
 * layer's attention writes that layer's paged KV out to the connector's side,
 * and start_load_kv, which before the model's forward pass writes KV held
 * outside into vLLM's paged KV buffer.  The staging buffer stands for the
 * connector's side; the checksum is the one of the checksum page above, taken
 * on the bytes as they pass (a save is checksummed once the KV is final, a
 * load once its data have arrived).
 *
 * Staging layout (device, owned by the caller): entries are the listed
 * positions in request order -- entry e of request r's k-th listed position is
 * sum_{r'<r} num_blocks_per_req[r'] + k -- and each entry holds one block
 * image per cache, in cache order.  An image is [plane][head][slot][row_bytes]
 * over planes x head_count x block_size rows (kvck_staging_bytes(...) bytes
 * per entry); only the valid slots of the position are copied, in either
 * direction, and the rest of the image and of the pool block is left as is.
 * Entries past staging_positions are flagged KVCK_FLAG_STAGING_FULL and
 * skipped.  A load needs the same planes, heads and request structure as the
 * save that filled the staging buffer; the image does not depend on the pool
 * layout, so a block saved from one layout (say an element-transposed V plane)
 * loads into another (an HND V plane).
 */
kvck_status kvck_copy_checksum_blocks(
    int32_t direction,                     /* KVCK_COPY_SAVE or KVCK_COPY_LOAD */
    const kvck_kv_layout* layout,
    void* const* cache_ptrs,               /* host [num_caches] of device pointers */
    const int32_t* layer_numbers, const int32_t* global_head_base, int32_t num_caches,
    int32_t head_begin, int32_t head_count,
    const int32_t* block_table, int64_t block_table_row_stride,
    const int32_t* num_blocks_per_req, const int64_t* start_pos, const int64_t* num_tokens,
    int32_t num_reqs, int32_t max_blocks,
    void* staging, int64_t staging_positions,  /* device */
    uint64_t* out, int64_t out_stride, int32_t accumulate,
    void* workspace, size_t workspace_bytes,
    uint32_t* error_flags,
    kvck_stream_t stream);

/* Staging bytes of one entry (listed position) for kvck_copy_checksum_blocks;
 * 0 for an invalid layout or plane range, or a size of 2^50 bytes or more. */
size_t kvck_staging_bytes(const kvck_kv_layout* layout, int32_t num_caches, int32_t head_count);

/*
 * kvck_tag_checksums -- tags of offloaded checksums and the load-time check.
 *
 * The page's function block_checksum_tags: a block's tag is the little-endian
 * value of its hash's leading 8 bytes, XOR the group's fingerprint; the
 * checksum offloaded with a block (one uint64, the page's BLOCK_CHECKSUM_BYTES)
 * is XORed with the tag, which ties it to that block hash and group of layers.
 * A position's checksum is its row of `columns` replica columns summed
 * (class KVChecksumGroup: the stored value is the row's partials summed when
 * the KV was offloaded; columns = 1 for one column).  For every entry i (only
 * listed positions i = r*max_blocks + k, k < num_blocks_per_req[r], when
 * num_blocks_per_req is given):
 *   c_i = sum over col < columns of checksums[i*columns + col]
 *   t_i = c_i ^ LE64(block_hashes + i*hash_stride) ^ fingerprint
 *   tagged[i] = t_i                               (if tagged: the value to offload)
 *   mismatch[i] = (t_i != stored[i])              (if stored: a load of offloaded KV)
 *   *mismatch_count += number of mismatches       (if mismatch_count)
 * Other entries are not written.  A request lists nothing when its count is
 * outside [0, max_blocks] or, with start_pos given, its start position is
 * negative or too large for block_size (the rule under which
 * kvck_checksum_blocks skips a request and leaves its entries unwritten), so
 * a rejected request is neither tagged nor compared.  All pointers are device
 * pointers; the uint64 arrays and block_hashes must be 8-byte aligned, with
 * hash_stride a multiple of 8 (vLLM block hashes are 32 bytes).  At least one
 * of tagged / stored.
 */
kvck_status kvck_tag_checksums(
    const uint64_t* checksums,             /* device [n][columns] */
    int32_t columns,                       /* 1..KVCK_MAX_OUT_STRIDE */
    const uint8_t* block_hashes,           /* device [n][hash_stride] */
    int64_t hash_stride,                   /* bytes, >= 8, multiple of 8 */
    uint64_t fingerprint,
    int64_t n,
    const int32_t* num_blocks_per_req,     /* device [n/max_blocks], optional */
    const int64_t* start_pos,              /* device [n/max_blocks], optional, needs num_blocks_per_req */
    int32_t max_blocks,
    int32_t block_size,                    /* >= 1 when start_pos is given */
    uint64_t* tagged,                      /* device [n], optional */
    const uint64_t* stored,                /* device [n], optional */
    uint8_t* mismatch,                     /* device [n], optional, needs stored */
    uint32_t* mismatch_count,              /* device, optional, needs stored; incremented */
    kvck_stream_t stream);

/*
 * Instrumentation (optional, process-wide).  While enabled, every
 * kvck_checksum_blocks, kvck_copy_checksum_blocks and kvck_checksum_states
 * call records one pair of HIP events on its stream around its main pass --
 * the kernel launches that stream the cache bytes (not the plan, the copy's
 * visiting order or the second pass) -- so a benchmark can time that kernel
 * alone.  kvck_checksum_blocks_noalloc records none.
 * kvck_instrument_read waits for the recorded events, returns the summed
 * elapsed milliseconds and the number of calls timed, and starts a new tally.
 */
kvck_status kvck_instrument(int32_t enable);
kvck_status kvck_instrument_read(double* total_ms, int64_t* calls);

/* Human-readable name of a kvck_status value (static storage). */
const char* kvck_status_string(int32_t status);

/* Whether this platform can run the checksum kernels: 1 if the current HIP
 * device is a gfx950 GPU, else 0.  The library's counterpart of the checksum
 * page's helper kv_checksum_platform_supported (section "helper functions"),
 * which gates the page's Triton kernel on CUDA-like or XPU platforms. */
int32_t kvck_platform_supported(void);

/* KVCK_ABI_VERSION of the loaded library. */
int32_t kvck_abi_version(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* KVCK_H_ */

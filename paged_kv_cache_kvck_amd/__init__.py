"""KV-cache block checksums on MI355X (gfx950).

The checksum of the vLLM API page
"vllm.distributed.kv_transfer.kv_checksum.checksum", computed by hand-written
HIP kernels in ``libkvck.so`` behind a C ABI (include/kvck.h).  The names
below are the C entry points, taking torch tensors; the library is loaded on
first use and its absence is an error, never a fallback.
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    KVCK_FLAG_BAD_BLOCK_ID,
    KVCK_FLAG_BAD_REQUEST,
    KVCK_COPY_LOAD,
    KVCK_COPY_SAVE,
    KVCK_FLAG_BAD_STATE_SLOT,
    KVCK_FLAG_STAGING_FULL,
    KVCK_ABI_VERSION,
    KVCK_MAX_CACHES,
    KVCK_MAX_OUT_STRIDE,
    KVCK_SCRATCH_BYTES,
    KvckDeviceError,
    KvckError,
    LAYOUT_NAMES,
    PreparedCall,
    PreparedCaches,
    kv_layout,
    kvck_abi_version,
    kvck_blocks_workspace_bytes,
    kvck_checksum_blocks,
    kvck_checksum_blocks_noalloc,
    kvck_checksum_states,
    kvck_copy_checksum_blocks,
    kvck_instrument,
    kvck_instrument_read,
    kvck_platform_supported,
    kvck_staging_bytes,
    kvck_states_workspace_bytes,
    kvck_status_string,
    kvck_tag_checksums,
    load_library,
    prepare_call,
    prepare_caches,
    state_desc,
)

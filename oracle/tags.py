"""Oracle of the offloaded-checksum tags (test infrastructure only).

vLLM API page "vllm.distributed.kv_transfer.kv_checksum.checksum":

* function ``block_checksum_tags(block_hashes, fingerprint)``: the uint64 an
  offloaded block checksum is XORed with, so that it matches only the block it
  was stored for -- the first 8 bytes of the block's hash read little-endian,
  XOR the group's fingerprint;
* attribute ``BLOCK_CHECKSUM_BYTES``: one int64 is stored per block;
* ``KVChecksumGroup.stored`` / ``KVChecksumScheduled.reqs_to_load``: a load of
  offloaded KV is checked against the checksums offloaded with it.

Reading: what is offloaded with block i is ``c_i XOR tag_i``; a load of block
i is consistent when its fresh checksum XOR its tag equals what was stored.
"""

from __future__ import annotations

import numpy as np


def block_checksum_tags(block_hashes, fingerprint: int) -> np.ndarray:
    """uint64 tag per block: little-endian value of hash[:8] XOR fingerprint."""
    tags = [int.from_bytes(bytes(h[:8]), "little") for h in block_hashes]
    return np.array(tags, dtype=np.uint64) ^ np.uint64(fingerprint)


def tag_checksums(checksums, block_hashes, fingerprint: int) -> np.ndarray:
    """The values to offload with the blocks: checksum XOR tag."""
    return np.asarray(checksums, dtype=np.uint64) ^ block_checksum_tags(block_hashes, fingerprint)


def offload_mismatches(checksums, block_hashes, fingerprint: int, stored) -> np.ndarray:
    """True where a loaded block's checksum does not match what was offloaded."""
    return tag_checksums(checksums, block_hashes, fingerprint) != np.asarray(stored, dtype=np.uint64)

"""Oracle of the offloaded-checksum tags (test infrastructure only).

vLLM API page "vllm.distributed.kv_transfer.kv_checksum.checksum":

* function ``block_checksum_tags(block_hashes, fingerprint)``: a per-block
  uint64 built from the block's hash (its leading 8 bytes as a little-endian
  integer) and the group's fingerprint (XOR), used to bind an offloaded
  checksum to the one block and group of layers it belongs to;
* attribute ``BLOCK_CHECKSUM_BYTES``: 8 bytes are kept per offloaded block;
* ``KVChecksumGroup.stored`` / ``KVChecksumScheduled.reqs_to_load``: a load of
  offloaded KV is checked against the checksums offloaded with it;
* ``KVChecksumGroup.values`` / attribute ``ReplicaKey``: a worker's partial
  checksums have one column per replica key, and what was offloaded for a
  position is its row of partials summed.

Reading: what is offloaded with block i is ``c_i XOR tag_i``; a load of block
i is consistent when its fresh checksum XOR its tag equals what was stored.
"""

from __future__ import annotations

import numpy as np


def _le64(digest) -> int:
    """Integer whose little-endian byte string is the digest's first 8 bytes."""
    value = 0
    for i, byte in enumerate(bytes(digest)[:8]):
        value |= byte << (8 * i)
    return value


def block_checksum_tags(block_hashes, fingerprint: int) -> np.ndarray:
    """One uint64 tag per block hash: _le64(hash) XOR fingerprint."""
    fp = int(fingerprint) & ((1 << 64) - 1)
    return np.array([_le64(h) ^ fp for h in block_hashes], dtype=np.uint64)


def offloaded_value(values) -> np.ndarray:
    """The value a position contributes to ``stored``: its row of partial
    checksums (the last axis, one column per replica key) summed mod 2^64."""
    v = np.asarray(values, dtype=np.uint64)
    return v.sum(axis=-1, dtype=np.uint64)


def tag_checksums(checksums, block_hashes, fingerprint: int) -> np.ndarray:
    """The values to offload with the blocks: checksum XOR tag."""
    return np.asarray(checksums, dtype=np.uint64) ^ block_checksum_tags(block_hashes, fingerprint)


def offload_mismatches(checksums, block_hashes, fingerprint: int, stored) -> np.ndarray:
    """True where a loaded block's checksum does not match what was offloaded."""
    return tag_checksums(checksums, block_hashes, fingerprint) != np.asarray(stored, dtype=np.uint64)

"""Pins of the offloaded-checksum tag oracle (CPU only).

Page function ``block_checksum_tags``: first 8 bytes of the block hash read
little-endian, XOR the fingerprint (one uint64 per block, BLOCK_CHECKSUM_BYTES).
"""

import numpy as np

from oracle import tags


def test_little_endian_first_eight_bytes():
    h = bytes(range(1, 33))                      # 32-byte hash 01 02 .. 20
    assert tags.block_checksum_tags([h], 0)[0] == 0x0807060504030201
    assert tags.block_checksum_tags([b"\xff" * 8 + b"\x00" * 24], 0)[0] == 0xFFFFFFFFFFFFFFFF
    # bytes past the eighth never matter
    assert tags.block_checksum_tags([h[:8] + b"\xaa" * 24], 7)[0] == tags.block_checksum_tags([h], 7)[0]


def test_fingerprint_xor():
    h = [bytes([0] * 32), bytes([0x80] + [0] * 31)]
    t = tags.block_checksum_tags(h, 0x0123456789ABCDEF)
    assert t[0] == 0x0123456789ABCDEF
    assert t[1] == 0x0123456789ABCDEF ^ 0x80


def test_tag_is_an_involution_and_detects_wrong_blocks():
    rng = np.random.default_rng(0)
    hashes = [rng.bytes(32) for _ in range(64)]
    c = rng.integers(0, 2**63, size=64, dtype=np.int64).astype(np.uint64) * np.uint64(2)
    fp = 0x5EED5EED5EED5EED
    stored = tags.tag_checksums(c, hashes, fp)
    assert np.array_equal(stored ^ tags.block_checksum_tags(hashes, fp), c)
    assert not tags.offload_mismatches(c, hashes, fp, stored).any()
    # a block loaded for the wrong hash, a wrong fingerprint, a changed checksum: all mismatch
    swapped = hashes[1:] + hashes[:1]
    assert tags.offload_mismatches(c, swapped, fp, stored).all()
    assert tags.offload_mismatches(c, hashes, fp ^ 1, stored).all()
    c2 = c.copy()
    c2[5] ^= np.uint64(1 << 40)
    assert tags.offload_mismatches(c2, hashes, fp, stored).tolist() == [i == 5 for i in range(64)]

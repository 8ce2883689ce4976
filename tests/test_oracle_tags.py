"""Pins of the offloaded-checksum tag oracle (CPU only).

Page function ``block_checksum_tags``: first 8 bytes of the block hash read
little-endian, XOR the fingerprint (one uint64 per block, BLOCK_CHECKSUM_BYTES).
Each pin takes the tags module, so the same pins also run against planted
mistakes in copies of it (each must be caught).
"""

import os
import types

import numpy as np
import pytest

from oracle import tags


def pin_little_endian_first_eight_bytes(t):
    h = bytes(range(1, 33))                      # 32-byte hash 01 02 .. 20
    assert t.block_checksum_tags([h], 0)[0] == 0x0807060504030201
    assert t.block_checksum_tags([b"\xff" * 8 + b"\x00" * 24], 0)[0] == 0xFFFFFFFFFFFFFFFF
    # bytes past the eighth never matter
    assert t.block_checksum_tags([h[:8] + b"\xaa" * 24], 7)[0] == t.block_checksum_tags([h], 7)[0]


def pin_fingerprint_xor(t):
    h = [bytes([0] * 32), bytes([0x80] + [0] * 31)]
    tg = t.block_checksum_tags(h, 0x0123456789ABCDEF)
    assert tg[0] == 0x0123456789ABCDEF
    assert tg[1] == 0x0123456789ABCDEF ^ 0x80
    # a fingerprint with the top bit set keeps all 64 bits
    assert t.block_checksum_tags(h[:1], 0xF000000000000001)[0] == 0xF000000000000001


def pin_involution_and_detection(t):
    rng = np.random.default_rng(0)
    hashes = [rng.bytes(32) for _ in range(64)]
    c = rng.integers(0, 2**63, size=64, dtype=np.int64).astype(np.uint64) * np.uint64(2)
    fp = 0x5EED5EED5EED5EED
    stored = t.tag_checksums(c, hashes, fp)
    assert np.array_equal(stored ^ t.block_checksum_tags(hashes, fp), c)
    assert not t.offload_mismatches(c, hashes, fp, stored).any()
    # a block loaded for the wrong hash, a wrong fingerprint, a changed checksum: all mismatch
    swapped = hashes[1:] + hashes[:1]
    assert t.offload_mismatches(c, swapped, fp, stored).all()
    assert t.offload_mismatches(c, hashes, fp ^ 1, stored).all()
    c2 = c.copy()
    c2[5] ^= np.uint64(1 << 40)
    assert t.offload_mismatches(c2, hashes, fp, stored).tolist() == [i == 5 for i in range(64)]


TAG_PINS = [pin_little_endian_first_eight_bytes, pin_fingerprint_xor, pin_involution_and_detection]


@pytest.mark.parametrize("pin", TAG_PINS, ids=lambda f: f.__name__)
def test_tag_pin(pin):
    pin(tags)


SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "tags.py")

MUTATIONS = {
    "hash read big-endian": ("value |= byte << (8 * i)", "value |= byte << (8 * (7 - i))"),
    "hash bytes 1..8": ("bytes(digest)[:8]", "bytes(digest)[1:9]"),
    "hash bytes 0..7 of 7": ("bytes(digest)[:8]", "bytes(digest)[:7]"),
    "fingerprint dropped": ("_le64(h) ^ fp for h", "_le64(h) for h"),
    "fingerprint added": ("_le64(h) ^ fp for h", "(_le64(h) + fp) & ((1 << 64) - 1) for h"),
    "fingerprint cut to 32 bits": ("fp = int(fingerprint) & ((1 << 64) - 1)", "fp = int(fingerprint) & 0xFFFFFFFF"),
    "stored value is the tag alone": ("np.asarray(checksums, dtype=np.uint64) ^ block_checksum_tags",
                                      "0 * np.asarray(checksums, dtype=np.uint64) ^ block_checksum_tags"),
    "mismatch test inverted": ("!= np.asarray(stored, dtype=np.uint64)", "== np.asarray(stored, dtype=np.uint64)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_tag_mutant_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("tags_mutant")
    exec(compile(src.replace(old, new), SRC + f" [{name}]", "exec"), mod.__dict__)
    caught = False
    for pin in TAG_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError or a crash: either way the pin rejects it
            caught = True
            break
    assert caught, f"no tag pin catches the mutant {name!r}"

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

import oracle
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


def pin_offloaded_row_sum(t):
    # one column is the value itself; columns add modulo 2^64 over the last axis
    assert t.offloaded_value(np.array([[5], [2**64 - 1]], np.uint64)).tolist() == [5, 2**64 - 1]
    assert t.offloaded_value(np.array([[2**63, 2**63, 7], [1, 2, 3]], np.uint64)).tolist() == [7, 6]
    x = np.arange(24, dtype=np.uint64).reshape(2, 3, 4)
    assert t.offloaded_value(x).tolist() == [[6, 22, 38], [54, 70, 86]]


def pin_offloaded_columns_are_partials_of_one_checksum(t):
    """Columns over disjoint sets of a group's layers (each set with its own
    replica key) are partial checksums, which the page says sum to the
    group's checksum c: their row sum equals the checksum over all layers."""
    rng = np.random.default_rng(5)
    bs, heads, hd, nb = 4, 2, 8, 6
    pools = [rng.integers(0, 2**16, size=(2, nb, bs, heads, hd), dtype=np.uint16) for _ in range(3)]
    bt = np.array([[3, 1, 4], [0, 5, 2]], np.int32)
    nblk, sp, nt = np.array([3, 2], np.int32), np.array([0, 7], np.int64), np.array([11, 37], np.int64)
    layers = [0, 4, 9]
    full = oracle.checksum_blocks(pools, "NHD", layers, [0] * 3, bt, nblk, sp, nt)
    cols = [oracle.checksum_blocks(pools[:1], "NHD", layers[:1], [0], bt, nblk, sp, nt),
            oracle.checksum_blocks(pools[1:], "NHD", layers[1:], [0] * 2, bt, nblk, sp, nt)]
    got = t.offloaded_value(np.stack(cols, axis=-1))
    for r in range(2):
        assert got[r, :nblk[r]].tolist() == full[r, :nblk[r]].tolist()
        assert got[r, :nblk[r]].tolist() != cols[0][r, :nblk[r]].tolist()


TAG_PINS = [pin_little_endian_first_eight_bytes, pin_fingerprint_xor, pin_involution_and_detection,
            pin_offloaded_row_sum, pin_offloaded_columns_are_partials_of_one_checksum]


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
    "row sum over the first axis": ("v.sum(axis=-1, dtype=np.uint64)", "v.sum(axis=0, dtype=np.uint64)"),
    "first replica column only": ("v.sum(axis=-1, dtype=np.uint64)", "v[..., 0]"),
    "row sum cut to 32 bits": ("v.sum(axis=-1, dtype=np.uint64)", "v.sum(axis=-1, dtype=np.uint64) & np.uint64(0xFFFFFFFF)"),
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

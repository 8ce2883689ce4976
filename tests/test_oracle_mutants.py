"""Planted mistakes: each mutated copy of the oracle must fail at least one pin.

The mutations are textual edits of a copy of ``oracle/kv_checksum.py`` made on
the CPU (a dropped term, a wrong index, a transposed operand, a wrong byte
order, ...).  A pin set that passed a mutant would not be strong enough to
trust the oracle.
"""

import importlib.util
import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kv_checksum.py")

MUTATIONS = {
    "dropped +1 in 2j+1": ("odd = _U64(2) * j + _U64(1)", "odd = _U64(2) * j"),
    "2j+3 instead of 2j+1": ("odd = _U64(2) * j + _U64(1)", "odd = _U64(2) * j + _U64(3)"),
    "token numbered from the block": ("t = _U64(position * bs) + np.arange(v, dtype=_U64)",
                                      "t = np.arange(v, dtype=_U64)"),
    "piece stride P-1": ("j = t[:, None] * _U64(P) + np.arange(P, dtype=_U64)[None, :]",
                         "j = t[:, None] * _U64(P - 1) + np.arange(P, dtype=_U64)[None, :]"),
    "V before K (NHD)": ("planes = [cache[p, b, :v, h0:h0 + n, :] for p in (0, 1)]",
                         "planes = [cache[p, b, :v, h0:h0 + n, :] for p in (1, 0)]"),
    "V before K (HND)": ("np.swapaxes(cache[p, b, h0:h0 + n, :v, :], 0, 1) for p in (0, 1)]",
                         "np.swapaxes(cache[p, b, h0:h0 + n, :v, :], 0, 1) for p in (1, 0)]"),
    "big-endian pieces": ('x = rows.view("<u8")', 'x = rows.view(">u8")'),
    "m without +1": ("m = _U64(2) * (_U64(layer) * _U64(MAX_KV_HEADS_PER_LAYER) + heads) + _U64(1)",
                     "m = _U64(2) * (_U64(layer) * _U64(MAX_KV_HEADS_PER_LAYER) + heads)"),
    "layer ignored in m": ("m = _U64(2) * (_U64(layer) * _U64(MAX_KV_HEADS_PER_LAYER) + heads)",
                           "m = _U64(2) * (_U64(0) * _U64(MAX_KV_HEADS_PER_LAYER) + heads)"),
    "local head numbering": ("heads = _U64(g0) + np.arange(n, dtype=_U64)", "heads = np.arange(n, dtype=_U64)"),
    "H = 1 << 15": ("MAX_KV_HEADS_PER_LAYER = 1 << 16", "MAX_KV_HEADS_PER_LAYER = 1 << 15"),
    "num_valid_tokens off by one": ("last = min(first + block_size, num_tokens)",
                                    "last = min(first + block_size, num_tokens + 1)"),
    "no exclusion of slots": ("v = num_valid_tokens(position, bs, num_tokens)\n", "v = bs\n"),
    "token index kept in 32 bits": ("t = _U64(position * bs) + np.arange(v, dtype=_U64)",
                                    "t = _U64((position * bs) & 0xFFFFFFFF) + np.arange(v, dtype=_U64)"),
    "piece index kept in 32 bits": ("odd = _U64(2) * j + _U64(1)", "odd = _U64(2) * (j & _U64(0xFFFFFFFF)) + _U64(1)"),
    "slice factor kept in 31 bits": ("c = c + (m * s).sum(dtype=_U64)",
                                     "c = c + ((m & _U64(0x7FFFFFFF)) * s).sum(dtype=_U64)"),
    "slice factor kept in 32 bits": ("c = c + (m * s).sum(dtype=_U64)",
                                     "c = c + ((m & _U64(0xFFFFFFFF)) * s).sum(dtype=_U64)"),
    "layer number kept in 16 bits": ("m = _U64(2) * (_U64(layer) * _U64(MAX_KV_HEADS_PER_LAYER) + heads)",
                                     "m = _U64(2) * (_U64(layer & 0xFFFF) * _U64(MAX_KV_HEADS_PER_LAYER) + heads)"),
    "Mamba elements numbered from 1": ("e = np.arange(x.size, dtype=_U64)", "e = np.arange(x.size, dtype=_U64) + _U64(1)"),
    "Mamba local row numbering": ("m = _U64(slice_factor(layer, g0 + g))", "m = _U64(slice_factor(layer, g))"),
    "Mamba states reversed": ("for st in states])", "for st in states[::-1]])"),
    "Mamba elements read signed": ("return state.view(np.uint16)", "return state.view(np.int16)"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{abs(hash(name))}")
    mod.__file__ = SRC
    exec(compile(src, SRC + f" [{name}]", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name, *MUTATIONS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError or a crash: either way the pin rejects it
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin catches the mutant {name!r}"

"""The oracle against what the pages and mathematics fix (CPU only)."""

import pytest

import pins
from oracle import kv_checksum as o


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(o)


def test_single_piece_detection_exhaustive():
    """Every one of the tiny config's 6,400 pieces, flipped, changes c."""
    pins.pin_detection(o, exhaustive=True)


def test_more_heads_than_bound_not_checksummed():
    import numpy as np
    rng = np.random.default_rng(0)
    case, _ = pins.make_case(rng, layout="NHD", layers=(0,), nh=2, bases=((1 << 16) - 1,))
    with pytest.raises(ValueError):
        o.checksum_blocks(**case)

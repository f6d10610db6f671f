"""The parity tests' acceptance bound against FP32 arithmetic and the values
worked out by hand (no GPU needed); the pins are in tests/bound_pins.py."""
import pytest

import oracle
from tests import bound_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_BOUND_PINS, ids=lambda p: p.__name__)
def test_bound_pin(pin):
    pin(oracle.error_bound)


def test_round_mantissa_helper():
    """The reduced-precision rounding the pins use, on known values."""
    import numpy as np
    r = pins.round_mantissa
    assert r(np.float32(1 + 2 ** -11 - 2 ** -23), 10) == 1.0
    assert r(np.float32(1 + 2 ** -11), 10) == 1.0            # tie: even mantissa
    assert r(np.float32(1 + 3 * 2 ** -11), 10) == np.float32(1 + 2 ** -9)  # tie: up to even
    assert r(np.float32(1 + 2 ** -10), 10) == np.float32(1 + 2 ** -10)
    assert r(np.float32(-1.5), 7) == np.float32(-1.5)

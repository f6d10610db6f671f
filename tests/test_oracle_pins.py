"""The oracle against mathematics (no GPU needed)."""
import pytest

from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_f32_rounding_helper():
    """The exact FP32 rounding used by the brute-force pin, on known values."""
    from fractions import Fraction
    import numpy as np
    # 1 + 2^-24 is a tie between 1 and 1 + 2^-23: even mantissa wins (1).
    assert pins.f32_of_fraction(1 + Fraction(1, 2 ** 24)) == np.float32(1.0)
    # 1 + 3 * 2^-24 is a tie between 1 + 2^-23 and 1 + 2^-22: even wins.
    assert pins.f32_of_fraction(1 + Fraction(3, 2 ** 24)) == np.float32(1 + 2 ** -22)
    # just above a tie rounds up
    assert pins.f32_of_fraction(1 + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 60)) == \
        np.float32(1 + 2 ** -23)
    assert pins.f32_of_fraction(Fraction(-1, 3)) == np.float32(-1 / 3)
    assert pins.f32_of_fraction(Fraction(0)) == np.float32(0)

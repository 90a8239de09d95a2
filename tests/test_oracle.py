"""The oracle against its pins (CPU only)."""

import numpy as np
import pytest

from oracle import ref
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x3EAB],
                    dtype=np.uint16)
    got = ref.bf16_bits_to_f64(bits)
    exp = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127,
           (1 + 0x2B / 128) * 2.0 ** -2]
    assert np.array_equal(got, np.array(exp))
    assert np.signbit(got[3]) and not np.signbit(got[2])
    assert np.isnan(ref.bf16_bits_to_f64(np.array([0x7FC1], dtype=np.uint16)))[0]

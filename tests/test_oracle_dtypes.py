"""Pins of the exact storage decode with bit patterns of known value."""

from __future__ import annotations

import numpy as np

from oracle.dtypes import decode


def test_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, np.inf, 2.0 ** -133, 3.140625]
    got = decode(bits, "bf16")
    assert got.dtype == np.float64
    assert list(got) == want
    assert np.signbit(got[4])


def test_fp16_bit_patterns():
    bits = np.array([0x3C00, 0xC000, 0x3C01, 0x0001, 0x7BFF], dtype=np.uint16)
    got = decode(bits.view(np.float16), "f16")
    assert list(got) == [1.0, -2.0, 1.0 + 2.0 ** -10, 2.0 ** -24, 65504.0]


def test_fp32_widening_is_exact():
    x = np.array([1.0 + 2.0 ** -23, -3.5e-40, 1.0e38], dtype=np.float32)
    got = decode(x, "f32")
    assert got[0] == 1.0 + 2.0 ** -23
    assert got[2] == float(np.float32(1.0e38))

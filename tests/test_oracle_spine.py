"""Pins for the oracle's row-scaled int8 dequantisation (CPU only).

Checked against exact rational arithmetic (every int8 value times scales
spread over the float32 range, rounded to nearest-even by hand), powers of
two (exact), the row orientation (one-hot scales), and IEEE special values.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import spine as S


def _f32_rne(fr):
    """Nearest float32 to the rational fr, ties to even, by bisection over
    the float32 bit patterns (finite values only)."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    lo, hi = 0, 0x7F7FFFFF  # +0 .. largest finite, ordered as integers
    val = lambda b: Fraction(struct.unpack("<f", struct.pack("<I", b))[0])
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if val(mid) <= a:
            lo = mid
        else:
            hi = mid
    dl, dh = a - val(lo), val(hi) - a
    b = lo if dl < dh or (dl == dh and lo % 2 == 0) else hi
    out = struct.unpack("<f", struct.pack("<I", b))[0]
    return -out if neg else out


def test_every_int8_times_sampled_scales_is_the_rounded_exact_product():
    rng = np.random.default_rng(0)
    # scales with full 24-bit significands over a wide exponent range
    scales = (rng.standard_normal(12) * np.exp2(rng.integers(-60, 60, 12))).astype(np.float32)
    q = np.tile(np.arange(-128, 128, dtype=np.int16).astype(np.int8), (12, 1))
    out = S.int8_row_dequant(q, scales)
    for r in range(12):
        for c in range(0, 256, 7):
            want = _f32_rne(Fraction(int(q[r, c])) * Fraction(float(scales[r])))
            assert out[r, c] == np.float32(want), (r, c)
    # the products that need rounding do occur (else this pin is empty)
    assert any(abs(int(v)) % 2 == 1 and int(v) not in (1, -1) for v in q[0])


def test_power_of_two_scales_are_exact_and_rows_are_not_transposed():
    R, C = 5, 9
    q = (np.arange(R * C) % 255 - 127).astype(np.int8).reshape(R, C)
    scale = np.exp2(np.arange(R, dtype=np.float32) - 2).astype(np.float32)
    out = S.int8_row_dequant(q, scale)
    for r in range(R):
        assert np.array_equal(out[r], q[r].astype(np.float32) * np.float32(2.0 ** (r - 2)))
    one_hot = np.zeros(R, dtype=np.float32)
    one_hot[3] = 1.0
    out = S.int8_row_dequant(q, one_hot)
    assert np.array_equal(out[3], q[3].astype(np.float32))
    assert not np.any(np.delete(out, 3, axis=0))


def test_special_values():
    q = np.array([[0, 1, -1, 127, -128]], dtype=np.int8)
    out = S.int8_row_dequant(q, np.array([-2.0], dtype=np.float32))
    assert np.signbit(out[0, 0]) and out[0, 0] == 0.0          # 0 * -2 = -0
    assert out[0].tolist()[1:] == [-2.0, 2.0, -254.0, 256.0]
    big = S.int8_row_dequant(q, np.array([3.0e38], dtype=np.float32))
    assert np.isinf(big[0, 3]) and np.isinf(big[0, 4])        # overflow to +-inf
    inf = S.int8_row_dequant(q, np.array([np.inf], dtype=np.float32))
    assert np.isnan(inf[0, 0]) and inf[0, 1] == np.inf        # 0 * inf = NaN
    nan = S.int8_row_dequant(q, np.array([np.nan], dtype=np.float32))
    assert np.isnan(nan).all()
    with pytest.raises(ValueError):
        S.int8_row_dequant(q, np.ones(2, dtype=np.float32))

"""Host logic of the MXFP8 code checker that the GPU tests apply to the
layer's h codes (CPU only): the oracle's own codes pass; a code one step
off far from a rounding midpoint, a truncating quantiser and an unreachable
block exponent are rejected; legitimate neighbours at a midpoint or a
power-of-two block maximum pass and report their exact value change."""

import numpy as np
import pytest

from oracle import formats as F
from tests._gpu import check_h_block_codes, gamma, h_error_bound, scale_pos


def _h(seed, n=6, I=64):
    return np.random.default_rng(seed).standard_normal((n, I)) * 3.0


def test_oracle_codes_pass():
    h = _h(0)
    c, s = F.mxfp8_quantize(h)
    delta, nd = check_h_block_codes(h, 1e-6 * np.abs(h), c, s)
    assert nd == 0 and not delta.any()


def test_one_step_off_far_from_a_midpoint_fails():
    h = _h(1)
    c, s = F.mxfp8_quantize(h)
    c = c.copy()
    q = F.e4m3_decode(c)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    frac = np.abs(h / sc - q) / np.maximum(np.abs(q), 1e-30)
    i = np.unravel_index(np.argmin(frac + (np.abs(q) < 1) * 9), h.shape)  # a value on a code
    c[i] = c[i] + 1 if (c[i] & 0x7F) < 0x7E else c[i] - 1
    with pytest.raises(AssertionError, match="outside the fp32 bound"):
        check_h_block_codes(h, 1e-6 * np.abs(h), c, s)


def test_truncating_quantiser_fails():
    h = _h(2, n=16)
    c, s = F.mxfp8_quantize(h)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    v = h / sc
    # toward zero instead of to nearest: one code lower wherever RNE rounded up
    up = np.abs(F.e4m3_decode(c)) > np.abs(v)
    lower = np.where(up, c - 1, c).astype(np.uint8)  # magnitude one step lower (same sign)
    with pytest.raises(AssertionError):
        check_h_block_codes(h, 1e-6 * np.abs(h), lower, s)


def test_neighbour_code_at_a_midpoint_passes_with_its_exact_delta():
    h = _h(3)
    c, s = F.mxfp8_quantize(h)
    E = int(s[0, 0]) - 127
    # element 5 of row 0 placed exactly between the codes for 1.5 and 1.625
    h[0, 5] = np.ldexp(1.5625, E) * np.sign(h[0, 5] or 1.0)
    c, s = F.mxfp8_quantize(h)
    alt = c.copy()
    alt[0, 5] = c[0, 5] ^ 1  # the other neighbour (mantissa LSB)
    dh = 1e-9 * np.abs(h)
    delta, nd = check_h_block_codes(h, dh, alt, s)
    assert nd == 1
    expect = (F.e4m3_decode(alt[0, 5]) - F.e4m3_decode(c[0, 5])) * 2.0 ** E
    assert delta[0, 5] == expect and np.count_nonzero(delta) == 1


def test_block_exponent_near_a_power_of_two():
    h = _h(4)
    h[1, :32] *= 0.5
    h[1, 7] = 8.0  # block max exactly a power of two: exponent 3 - 8 = -5
    c, s = F.mxfp8_quantize(h)
    assert s[1, 0] == 127 - 5
    # the kernel saw 8 - tiny: exponent -6, every code of the block recomputed
    alt_s = s.copy()
    alt_s[1, 0] -= 1
    alt_c = c.copy()
    alt_c[1, :32] = F.e4m3_encode_rne_sat(np.ldexp(np.minimum(np.abs(h[1, :32]), 8 - 1e-9)
                                                   * np.sign(h[1, :32]), 6))
    dh = 1e-7 * np.abs(h).max() * np.ones_like(h)
    delta, nd = check_h_block_codes(h, dh, alt_c, alt_s)
    assert nd >= 1
    # far from a power of two the same change is rejected
    h2 = h.copy()
    h2[1, 7] = 7.0
    c2, s2 = F.mxfp8_quantize(h2)
    bad_s = s2.copy()
    bad_s[1, 0] -= 1
    with pytest.raises(AssertionError, match="block exponents"):
        check_h_block_codes(h2, dh, c2, bad_s)


def test_error_bound_covers_fp32_evaluations():
    """float32 evaluations of g, u and SiLU(g) u (in two summation orders)
    stay within h_error_bound's dh of the float64 h."""
    rng = np.random.default_rng(5)
    H, I = 1024, 64
    x = F.mxfp8_roundtrip(rng.standard_normal((4, H)))
    wg = F.e2m1_decode(rng.integers(0, 16, (I, H))) * 2.0 ** -6
    wu = F.e2m1_decode(rng.integers(0, 16, (I, H))) * 2.0 ** -6
    h, dh = h_error_bound(x, wg, wu)
    for order in (slice(None), slice(None, None, -1)):
        x32, g32, u32 = x.astype(np.float32), wg.astype(np.float32), wu.astype(np.float32)
        g = np.zeros((4, I), np.float32)
        u = np.zeros((4, I), np.float32)
        for kk in range(H)[order]:
            g += x32[:, kk:kk + 1] * g32[:, kk][None, :]
            u += x32[:, kk:kk + 1] * u32[:, kk][None, :]
        h32 = (g / (np.float32(1) + np.exp(-g))) * u
        assert (np.abs(h32.astype(np.float64) - h) <= dh).all()
    assert gamma(7168) < 1e-3


def test_scale_positions_permute_each_group_of_16():
    p = scale_pos(np.arange(64))
    for g in range(4):
        assert sorted(p[16 * g:16 * g + 16].tolist()) == list(range(16 * g, 16 * g + 16))
    assert p[1] == 4 and p[4] == 1 and p[5] == 5


def test_e2m1_codes_oracle_pass_and_one_step_off_fails():
    """The same checks on MXFP4 (E2M1) codes."""
    h = _h(6, n=8)
    c, s = F.mxfp4_quantize(h)
    delta, nd = check_h_block_codes(h, 1e-9 * np.abs(h), c, s, "e2m1")
    assert nd == 0 and not delta.any()
    q = F.e2m1_decode(c)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    on_code = np.isclose(h / sc, q, rtol=0, atol=1e-3) & (np.abs(q) >= 1) & (np.abs(q) < 6)
    if not on_code.any():  # make one element sit exactly on a code
        h[0, 3] = np.sign(h[0, 3] or 1.0) * 2.0 * sc[0, 3]
        c, s = F.mxfp4_quantize(h)
        on_code = np.zeros_like(h, bool)
        on_code[0, 3] = True
    i = np.argwhere(on_code)[0]
    bad = c.copy()
    bad[tuple(i)] = c[tuple(i)] + 1 if (c[tuple(i)] & 7) < 7 else c[tuple(i)] - 1
    with pytest.raises(AssertionError, match="outside the fp32 bound"):
        check_h_block_codes(h, 1e-9 * np.abs(h), bad, s, "e2m1")


def test_unpack_nibbles_low_first():
    from tests._gpu import unpack_nibbles
    assert unpack_nibbles(np.array([[0x21, 0xF0]], np.uint8)).tolist() == [[1, 2, 0, 15]]

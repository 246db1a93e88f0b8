"""Pins for the oracle's number formats (CPU only).

Each check compares the oracle against something other than itself: the
formats' closed forms, ROCm's host-side FP4 decode, torch's float8 and
bfloat16 casts, brute-force nearest-value search, and the byte counts the
pages print (kimi-k3-in-c note, byte accounting; Deltafin README, "How it
works").
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import record as R

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- E2M1 -----

def test_e2m1_closed_form_table():
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = F.e2m1_decode(np.arange(16))
    assert list(got[:8]) == pos
    assert list(-got[8:]) == pos
    assert np.signbit(got[8]) and got[8] == 0.0  # code 8 is -0
    assert not np.signbit(got[0])


@pytest.fixture(scope="module")
def rocm_fp4_table(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("fp4") / "fp4host"
    src = os.path.join(HERE, "golden", "rocm_fp4_host.hip")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o", str(out)],
                   check=True, capture_output=True)
    lines = subprocess.run([str(out)], check=True, capture_output=True, text=True).stdout.split("\n")
    rows = [l.split() for l in lines if l.strip()]
    return {int(b): (float(a), float(c), a.startswith("-"), c.startswith("-")) for b, a, c in rows}


def test_e2m1_and_nibble_order_match_rocm_host_decode(rocm_fp4_table):
    """ROCm's packed FP4 pair puts element 0 in the low nibble."""
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)  # 16 rows of K=32
    scales = np.full((16, 1), 127, dtype=np.uint8)
    w = F.mxfp4_dequant(codes, scales).reshape(-1)
    for b in range(256):
        lo, hi, lo_neg, hi_neg = rocm_fp4_table[b]
        assert w[2 * b] == lo and bool(np.signbit(w[2 * b])) == lo_neg
        assert w[2 * b + 1] == hi and bool(np.signbit(w[2 * b + 1])) == hi_neg


# ---------------------------------------------------------------- E8M0 -----

def test_e8m0_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_decode(b)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert got[0] == 2.0 ** -127
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[126] == 0.5


# ---------------------------------------------------------------- E4M3 -----

def _e4m3_grid():
    """All finite non-negative E4M3 values with their codes (torch decode)."""
    codes = np.arange(128, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    keep = ~np.isnan(vals)
    return vals[keep], codes[keep]


def test_e4m3_decode_all_codes_match_torch():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(c)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert F.e4m3_decode(0x7E) == 448.0


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.uniform(-448, 448, 20000),
        g.standard_normal(20000) * 3,
        g.standard_normal(20000) * 1e-3,  # subnormal range
        np.ldexp(g.uniform(1, 2, 2000), g.integers(-12, 8, 2000)),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_rne_sat(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def _brute_nearest_e4m3(a):
    """Nearest grid value to |a| with ties to the even code; clamp at 448."""
    vals, codes = _e4m3_grid()
    order = np.argsort(vals)
    vals, codes = vals[order], codes[order]
    a = np.minimum(np.abs(a), 448.0)
    idx = np.searchsorted(vals, a)
    lo = np.clip(idx - 1, 0, len(vals) - 1)
    hi = np.clip(idx, 0, len(vals) - 1)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0) & (codes[lo] % 2 == 1))
    return np.where(pick_hi, codes[hi], codes[lo])


def test_e4m3_encode_brute_force_all_bf16_magnitudes():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # all finite non-negative bf16
    v = F.bf16_decode(bits)
    for shift in (-12, -4, 0):
        x = np.ldexp(v, shift)
        x = x[x <= 1e4]
        got = F.e4m3_encode_rne_sat(x)
        exp = _brute_nearest_e4m3(x).astype(np.uint8)
        np.testing.assert_array_equal(got, exp)
        neg = F.e4m3_encode_rne_sat(-x)
        np.testing.assert_array_equal(neg, exp | 0x80)


def test_e4m3_saturates():
    got = F.e4m3_encode_rne_sat(np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf, -1e9]))
    assert list(F.e4m3_decode(got)) == [448.0] * 7 + [-448.0]


# ---------------------------------------------------------------- bf16 -----

def test_bf16_encode_matches_torch_on_float32():
    g = np.random.default_rng(3)
    v = np.concatenate([
        g.standard_normal(50000),
        g.standard_normal(5000) * 1e-39,  # float32 subnormals
        g.uniform(-3.3e38, 3.3e38, 5000),
        [0.0, -0.0, 1.0, -1.0],
    ]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.bf16_encode_rne(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_encode_float64_ties_and_no_double_rounding():
    # halfway between 1 and 1 + 2**-7 -> even (1.0); between 1+2**-7 and 1+2**-6 -> 1+2**-6
    assert F.bf16_encode_rne(1.0 + 2.0 ** -8) == 0x3F80
    assert F.bf16_encode_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the halfway point by less than float32 can hold: must round up
    assert F.bf16_encode_rne(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    # brute force on random float64: nearest of the two bf16 neighbours
    g = np.random.default_rng(5)
    v = g.standard_normal(20000) * np.exp(g.uniform(-20, 20, 20000))
    got = F.bf16_decode(F.bf16_encode_rne(v))
    lo = F.bf16_decode((np.abs(v).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    hi = F.bf16_decode(((np.abs(v).astype(np.float32).view(np.uint32) >> 16) + 1).astype(np.uint16))
    # float32 truncation may land one step above |v|; widen the candidate set
    lo2 = F.bf16_decode(((np.abs(v).astype(np.float32).view(np.uint32) >> 16) - 1).astype(np.uint16))
    cands = np.stack([lo2, lo, hi], axis=1)
    d = np.abs(cands - np.abs(v)[:, None])
    best = d.min(axis=1)
    assert np.all(np.abs(np.abs(got) - np.abs(v)) == best)


# ---------------------------------------------------------------- MXFP4 ----

def test_mxfp4_single_nibble_placement_and_block_scale():
    n, k = 3, 96
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.full((n, k // 32), 127, dtype=np.uint8)
    codes[1, 20] = 0x70  # element 41 (odd -> high nibble) = 6.0
    codes[2, 33] = 0x05  # element 66 (even -> low nibble) = 3.0
    scales[1, 1] = 130  # block 1 (elements 32..63) of row 1: x8
    scales[2, 2] = 120  # block 2 (elements 64..95) of row 2: x2**-7
    w = F.mxfp4_dequant(codes, scales)
    expect = np.zeros((n, k))
    expect[1, 41] = 6.0 * 8
    expect[2, 66] = 3.0 * 2.0 ** -7
    np.testing.assert_array_equal(w, expect)


def test_mxfp4_extreme_scales():
    codes = np.full((1, 16), 0x21, dtype=np.uint8)  # elements 0.5, 1.0 alternating
    for b, mult in ((0, 2.0 ** -127), (1, 2.0 ** -126), (254, 2.0 ** 127)):
        w = F.mxfp4_dequant(codes, np.array([[b]], dtype=np.uint8))
        np.testing.assert_array_equal(w[0, 0::2], 0.5 * mult)
        np.testing.assert_array_equal(w[0, 1::2], 1.0 * mult)
        # exactly representable in float32 (subnormals for b <= 1)
        assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
    w = F.mxfp4_dequant(codes, np.array([[255]], dtype=np.uint8))
    assert np.all(np.isnan(w))


def test_record_bytes_match_pages():
    # kimi-k3-in-c note, byte accounting: 17,547,264 bytes per expert,
    # 0.53125 bytes per MXFP4 weight
    assert R.record_bytes(7168, 1536) == 17_547_264
    assert R.record_bytes(7168, 1536) / (3 * 7168 * 1536) == 0.53125
    # Deltafin README "How it works": 16 experts x 92 MoE layers ~ 25.8 GB/token
    assert round(16 * 92 * R.record_bytes(7168, 1536) / 1e9, 1) == 25.8
    assert R.record_bytes(256, 64) == 26_112


def test_record_split_puts_each_matrix_in_its_section():
    h, i = 64, 32
    rec = np.zeros(R.record_bytes(h, i), dtype=np.uint8)
    views = R.split(rec, h, i)
    for m, code in enumerate((0x22, 0x44, 0x66)):  # 1.0, 2.0, 4.0
        views[2 * m][...] = code
        views[2 * m + 1][...] = 127 + m
    wg, wu, wd = R.dequant_expert(rec, h, i)
    assert wg.shape == (i, h) and wu.shape == (i, h) and wd.shape == (h, i)
    assert np.all(wg == 1.0) and np.all(wu == 4.0) and np.all(wd == 16.0)


# ---------------------------------------------------------------- MXFP8 ----

def test_mxfp8_scale_rule_and_saturation():
    blk = np.zeros((1, 32))
    blk[0, 0] = 1.0  # amax = 2**0 -> E = -8
    blk[0, 1] = 1.0 / 3
    c, s = F.mxfp8_quantize(blk)
    assert s[0, 0] == 127 - 8
    assert F.e4m3_decode(c[0, 0]) == 256.0
    blk[0, 0] = 1.99  # amax in [1, 2): E = -8, 1.99 * 256 = 509 -> saturates to 448
    c, s = F.mxfp8_quantize(blk)
    assert s[0, 0] == 119 and F.e4m3_decode(c[0, 0]) == 448.0
    c, s = F.mxfp8_quantize(np.zeros((2, 64)))
    assert np.all(s == 0) and np.all(c == 0)
    c, s = F.mxfp8_quantize(np.full((1, 32), 2.0 ** 140))
    assert s[0, 0] == 127 + 127  # clamped exponent


def test_mxfp8_brute_force_over_all_bf16():
    """Every finite bf16 value, placed in a block whose max is 2**3."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    v = F.bf16_decode(bits)
    v = v[v <= 8.0]
    pad = (-len(v)) % 31
    v = np.concatenate([v, np.zeros(pad)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((v.shape[0], 1), 8.0), v], axis=1)  # E = 3 - 8 = -5
    sign = np.where(np.arange(blocks.size).reshape(blocks.shape) % 2 == 0, 1.0, -1.0)
    blocks = blocks * sign
    c, s = F.mxfp8_quantize(blocks)
    assert np.all(s == 127 - 5)
    exp = _brute_nearest_e4m3(np.ldexp(np.abs(blocks), 5)).astype(np.uint8)
    exp = np.where(np.signbit(blocks), exp | 0x80, exp)
    np.testing.assert_array_equal(c, exp)


# ------------------------------------------------- MXFP4 activations ----

def _brute_nearest_e2m1(a):
    """Nearest E2M1 magnitude code (0..7) to each non-negative a, ties to the
    code with its mantissa bit clear, above 6 saturating -- by enumerating
    the eight magnitudes from the closed form."""
    mags = F.e2m1_decode(np.arange(8))
    a = np.minimum(np.asarray(a, dtype=np.float64), 6.0)
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    return np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))


def test_e2m1_encode_brute_force_dense_grid():
    """Every multiple of 1/64 in [0, 8] (all midpoints and ties included) and
    every finite bf16 value up to 8, both signs, against the brute force."""
    grid = np.arange(0, 8 * 64 + 1) / 64.0
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    bf = F.bf16_decode(bits)
    for v in (grid, bf[bf <= 8.0]):
        got = F.e2m1_encode_rne_sat(v)
        exp = _brute_nearest_e2m1(v).astype(np.uint8)
        np.testing.assert_array_equal(got, exp)
        np.testing.assert_array_equal(F.e2m1_encode_rne_sat(-v), exp | 8)


def test_e2m1_ties_and_saturation_by_hand():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 1e30, -0.25])
    assert F.e2m1_decode(F.e2m1_encode_rne_sat(v)).tolist() == \
        [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 6.0, -0.0]
    assert F.e2m1_encode_rne_sat(np.array([-0.25]))[0] == 8  # -0 keeps its sign
    c = np.arange(16, dtype=np.uint8)
    np.testing.assert_array_equal(F.e2m1_encode_rne_sat(F.e2m1_decode(c)), c)


def test_mxfp4_scale_rule_and_saturation():
    blk = np.zeros((1, 32))
    blk[0, 0] = 4.0  # amax = 2**2 -> E = 0
    blk[0, 1] = 1.0 / 3
    c, s = F.mxfp4_quantize(blk)
    assert s[0, 0] == 127 and F.e2m1_decode(c[0, 0]) == 4.0 and F.e2m1_decode(c[0, 1]) == 0.5
    blk[0, 0] = 7.9  # amax in [4, 8): E = 0, 7.9 saturates to 6
    c, s = F.mxfp4_quantize(blk)
    assert s[0, 0] == 127 and F.e2m1_decode(c[0, 0]) == 6.0
    blk[0, 0] = 1.0  # amax 1 -> E = -2: scaled values x4
    c, s = F.mxfp4_quantize(blk)
    assert s[0, 0] == 125 and F.e2m1_decode(c[0, 0]) == 4.0
    c, s = F.mxfp4_quantize(np.zeros((2, 64)))
    assert np.all(s == 0) and np.all(c == 0)
    c, s = F.mxfp4_quantize(np.full((1, 32), 2.0 ** 140))
    assert s[0, 0] == 127 + 127


def test_mxfp4_brute_force_blocks():
    """Blocks of grid values under a block maximum of 2**3: E = 1, each
    element's code the brute-force nearest of v / 2."""
    v = np.arange(0, 8 * 64) / 64.0
    pad = (-len(v)) % 31
    v = np.concatenate([v, np.zeros(pad)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((v.shape[0], 1), 8.0), v], axis=1)
    sign = np.where(np.arange(blocks.size).reshape(blocks.shape) % 3 == 0, -1.0, 1.0)
    blocks = blocks * sign
    c, s = F.mxfp4_quantize(blocks)
    assert np.all(s == 128)
    exp = _brute_nearest_e2m1((np.abs(blocks) / 2).ravel()).reshape(blocks.shape).astype(np.uint8)
    exp = np.where(np.signbit(blocks), exp | 8, exp)
    np.testing.assert_array_equal(c, exp)
    # the dequantised value is the code's E2M1 value times 2**E
    np.testing.assert_array_equal(F.mxfp4_act_dequant(c, s), F.e2m1_decode(c) * 2.0)

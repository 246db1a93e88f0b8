"""Number formats used by the layer, decoded/encoded in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

MXFP4 (kimi-k3-in-c note, byte accounting; Deltafin explainer section 2.1):
every weight is a 4-bit E2M1 element, and each run of 32 consecutive
elements along the input dimension shares one 8-bit E8M0 power-of-two
exponent, so a weight costs 0.5 + 1/32 = 0.53125 bytes.

The element and scale encodings below are the OCP microscaling (MX) formats
as this oracle reads them (the pages do not spell them out):
  E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
  E8M0: unsigned exponent byte b, value 2**(b-127); b == 255 is NaN.
  E4M3 (FN variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
        largest finite 448, S.1111.111 is NaN, no infinities.
"""

import numpy as np

# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------


def e2m1_decode(codes):
    """Value of 4-bit E2M1 codes (int array, 0..15) as float64.

    Closed form: s = bit 3, e = bits 2..1, m = bit 0;
    e > 0: (-1)^s * 2^(e-1) * (1 + m/2);  e == 0: (-1)^s * m/2.
    Code 8 decodes to -0.0.
    """
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp(1.0 + m / 2.0, np.maximum(e - 1, 0))
    mag = np.where(e == 0, m * 0.5, normal)
    return np.where(s == 1, -mag, mag)


# ----------------------------------------------------------------------------
# E8M0
# ----------------------------------------------------------------------------


def e8m0_decode(b):
    """Value of E8M0 scale bytes as float64: 2**(b-127); 255 -> NaN."""
    bb = np.asarray(b).astype(np.int64)
    if np.any((bb < 0) | (bb > 255)):
        raise ValueError("E8M0 scales are bytes")
    v = np.ldexp(1.0, np.minimum(bb, 254) - 127)
    return np.where(bb == 255, np.nan, v)


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def bf16_decode(bits):
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_encode_rne(v):
    """float64 -> bfloat16 bit patterns, round to nearest, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range; its
    subnormal spacing is 2**-133.  Values whose rounded magnitude reaches
    2**128 become infinity.  NaN maps to the canonical quiet NaN 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat_v = v.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_v)
    a = np.abs(flat_v)
    neg = np.signbit(flat_v)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        _, ex = np.frexp(a)  # a = f * 2**ex, f in [0.5, 1)
        lead = ex - 1  # exponent of the leading bit
        ulp_exp = np.where(lead >= -126, lead - 7, -133)
        q = np.rint(np.ldexp(a, -ulp_exp))  # rint rounds half to even
        r = np.ldexp(q, ulp_exp)
        r = np.where(np.isinf(a), np.inf, r)
        r = np.where(r >= 2.0 ** 128, np.inf, r)
        r = np.where(a == 0, 0.0, r)
    r32 = r.astype(np.float32)  # exact: r is on the bfloat16 grid
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(neg, bits | np.uint16(0x8000), bits)
    bits = np.where(nan, np.uint16(0x7FC0), bits)
    flat_o[:] = bits
    return out


# ----------------------------------------------------------------------------
# E4M3 (FN)
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the largest normal, 448 = 1.75 * 2**8


def e4m3_decode(codes):
    """Value of E4M3FN byte codes as float64 (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    sub = m / 8.0 * 2.0 ** -6
    nor = np.ldexp(1.0 + m / 8.0, e - 7)
    mag = np.where(e == 0, sub, nor)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode_rne_sat(v):
    """float64 -> E4M3FN codes, round to nearest even, saturating to +-448.

    Normal spacing in binade [2**p, 2**(p+1)) is 2**(p-3) for p >= -6;
    below 2**-6 the subnormal spacing is 2**-9.  A magnitude that rounds
    above 448 is clamped to 448 (the MX conversion saturates).  The sign
    of zero is kept.  NaN inputs are rejected (they never reach this
    quantiser in the layer).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN input to E4M3 quantiser")
    a = np.abs(v)
    neg = np.signbit(v)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        _, ex = np.frexp(a)
        lead = ex - 1
        ulp_exp = np.where(lead >= -6, lead - 3, -9)
        q = np.ldexp(np.rint(np.ldexp(a, -ulp_exp)), ulp_exp)
        q = np.where(np.isinf(a), E4M3_MAX, q)
        q = np.minimum(q, E4M3_MAX)
        q = np.where(a == 0, 0.0, q)
        _, qex = np.frexp(q)
        qlead = qex - 1
        is_norm = q >= 2.0 ** -6
        efield = np.where(is_norm, qlead + 7, 0)
        mant = np.where(is_norm, np.ldexp(q, -qlead) - 1.0, np.ldexp(q, 9))
        mant = np.where(is_norm, mant * 8.0, mant)
    code = (efield.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------
# MXFP4 weights
# ----------------------------------------------------------------------------

MX_BLOCK = 32


def mxfp4_dequant(codes, scales):
    """Dequantise one MXFP4 matrix to float64.

    codes:  uint8 [N, K/2]; element k of a row sits in byte k // 2, even k in
            the low nibble, odd k in the high nibble.
    scales: uint8 [N, K/32]; byte j scales elements 32*j .. 32*j+31 of the row.
    Returns W[n, k] = E2M1(nibble(n, k)) * 2**(scale[n, k // 32] - 127).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, kh = codes.shape
    k = 2 * kh
    if scales.shape != (n, k // MX_BLOCK) or k % MX_BLOCK:
        raise ValueError("scale shape does not match codes")
    nib = np.empty((n, k), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    elem = e2m1_decode(nib)
    sc = e8m0_decode(scales)
    return elem * np.repeat(sc, MX_BLOCK, axis=1)


# ----------------------------------------------------------------------------
# MXFP8 activations
# ----------------------------------------------------------------------------


def mxfp8_quantize(v):
    """Quantise rows of v (float64 [..., K], K % 32 == 0) to MXFP8 E4M3.

    Per block of 32 consecutive elements along the last axis:
      a = max |v_i|;  E = clamp(floor(log2 a) - 8, -127, 127), E = -127 when
      a == 0;  q_i = RNE_E4M3(v_i / 2**E) saturated to +-448.
    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32] = E + 127).
    The quantised value is e4m3_decode(code) * 2**E.
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    if k % MX_BLOCK:
        raise ValueError("MXFP8 blocks need K % 32 == 0")
    blocks = v.reshape(v.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(amax)
    floor_log2 = ex - 1
    e = np.where(amax == 0, -127, np.clip(floor_log2 - E4M3_EMAX, -127, 127))
    scaled = np.ldexp(blocks, -e[..., None])
    codes = e4m3_encode_rne_sat(scaled).reshape(v.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequant(codes, scales):
    """Inverse of mxfp8_quantize: e4m3 value * 2**(scale - 127)."""
    codes = np.asarray(codes)
    k = codes.shape[-1]
    vals = e4m3_decode(codes)
    sc = e8m0_decode(scales)
    return vals * np.repeat(sc, MX_BLOCK, axis=-1).reshape(vals.shape[:-1] + (k,))


def mxfp8_roundtrip(v):
    """Value after MXFP8 quantisation (float64)."""
    c, s = mxfp8_quantize(v)
    return mxfp8_dequant(c, s)


# ----------------------------------------------------------------------------
# MXFP4 activations (the prefill path's FP4 x FP4 variant)
# ----------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_EMAX = 2  # exponent of the largest normal, 6 = 1.5 * 2**2


def e2m1_encode_rne_sat(v):
    """float64 -> E2M1 codes (0..15), round to nearest, ties to even, saturating to +-6.

    Magnitude spacing: 0.5 on [0, 2) (the subnormal 0.5 and the binade
    [1, 2)), 1 on [2, 4), 2 on [4, 6]; "even" is the code whose mantissa bit
    (bit 0) is clear.  A magnitude above 6 becomes 6 (the MX conversion
    saturates).  The sign of zero is kept (code 8 is -0).  NaN inputs are
    rejected.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN input to E2M1 quantiser")
    a = np.minimum(np.abs(v), E2M1_MAX)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.rint(a / step) * step  # numpy's rint rounds half to even
    # a tie at a binade edge rounds onto the edge from below (1.75 -> 2, 3.5 -> 4)
    # with the next binade's code; the even choice inside a binade is rint's
    q = np.minimum(q, E2M1_MAX)
    # codes 0..7 are the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 in increasing order
    code = np.searchsorted(e2m1_decode(np.arange(8)), q).astype(np.int64)
    code = np.where(np.signbit(v), code | 8, code)
    return code.astype(np.uint8)


def mxfp4_quantize(v):
    """Quantise rows of v (float64 [..., K], K % 32 == 0) to MXFP4: per block
    of 32 consecutive elements along the last axis, a = max |v_i|,
    E = clamp(floor(log2 a) - 2, -127, 127) (E = -127 when a == 0) and
    q_i = RNE_E2M1(v_i / 2**E) saturated to +-6 -- the MXFP8 rule with E2M1's
    largest normal exponent (2) in place of E4M3's (8).
    Returns (codes uint8 [..., K], one E2M1 code per element; scale bytes
    uint8 [..., K/32] = E + 127).  The value is e2m1_decode(code) * 2**E.
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    if k % MX_BLOCK:
        raise ValueError("MXFP4 blocks need K % 32 == 0")
    blocks = v.reshape(v.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(amax)
    e = np.where(amax == 0, -127, np.clip(ex - 1 - E2M1_EMAX, -127, 127))
    scaled = np.ldexp(blocks, -e[..., None])
    codes = e2m1_encode_rne_sat(scaled).reshape(v.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp4_act_dequant(codes, scales):
    """Inverse of mxfp4_quantize: e2m1 value * 2**(scale - 127)."""
    codes = np.asarray(codes)
    k = codes.shape[-1]
    vals = e2m1_decode(codes)
    sc = e8m0_decode(scales)
    return vals * np.repeat(sc, MX_BLOCK, axis=-1).reshape(vals.shape[:-1] + (k,))


def mxfp4_roundtrip(v):
    """Value after MXFP4 quantisation (float64)."""
    c, s = mxfp4_quantize(v)
    return mxfp4_act_dequant(c, s)

"""Shared helpers of the GPU parity tests (not collected by pytest)."""

import numpy as np
import torch

import synth
import synth.device as SD
from oracle import formats as F
from oracle import moe as M
from oracle.record import dequant_expert

REL_TOL = 2e-3   # max over tokens of ||y_gpu - y_oracle||_2 / ||y_oracle||_2
TIE_EPS = 1e-6   # scores within this of the k-th score may go either way


def to_np_u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def rel_l2_per_token(y_bits, y_ref):
    y = F.bf16_decode(y_bits)
    num = np.linalg.norm(y - y_ref, axis=-1)
    den = np.linalg.norm(y_ref, axis=-1)
    return num / den


class Built:
    """One synthetic layer on the device plus its oracle description.

    dev holds the canonical device tensors (mutable by tests); lib is the
    library's layer over their packed copies -- call repack() after changing
    dev["experts"] or the shared matrices.
    """

    def __init__(self, cfg, seed=0, layer=0, bias=False, bias_mode="logits", routed_scale=1.0):
        self.cfg = cfg
        self.seed, self.layer_idx = seed, layer
        self.bias_mode, self.routed_scale = bias_mode, routed_scale
        d = SD.upload_layer(cfg, seed, layer, bias=bias)
        self.dev = d
        self.repack()
        H, I = cfg["hidden"], cfg["inter"]
        self.oracle = M.Layer(H, I, cfg["n_experts"], cfg["top_k"], d["host_router_w"],
                              expert_record=lambda e: synth.expert_record(seed, layer, e, H, I),
                              shared=d["host_shared"], router_bias=d["host_bias"],
                              bias_mode=bias_mode, routed_scale=routed_scale)

    def repack(self):
        from mxfp4_routed_expert_x896_amd import binding
        c, d = self.cfg, self.dev
        mode = binding.ROUTER_BIAS_SELECT if self.bias_mode == "select" else binding.ROUTER_BIAS_LOGITS
        self.lib = binding.Layer.from_canonical(
            c["hidden"], c["inter"], c["n_experts"], c["top_k"], d["router_w"], d["experts"],
            d["shared_gate"], d["shared_up"], d["shared_down"], d["router_bias"],
            router_mode=mode, routed_scale=self.routed_scale)
        torch.cuda.synchronize()


def check_routing(gpu_ids, gpu_w, scores, k, eps=TIE_EPS):
    """Selection parity with near-tie exclusion at the k-th score.

    Experts whose oracle score is above tau + eps must be selected, those
    below tau - eps must not be; the ones in between may go either way.
    The GPU's ids must be distinct, ordered by score (up to eps), and its
    weights must sum to one.
    """
    T, E = scores.shape
    n_ambiguous = 0
    for t in range(T):
        ids = gpu_ids[t]
        assert len(set(ids.tolist())) == k, f"token {t}: repeated ids {ids}"
        assert np.all((ids >= 0) & (ids < E))
        s = scores[t]
        tau = np.sort(s)[::-1][k - 1]
        must = set(np.nonzero(s > tau + eps)[0].tolist())
        never = set(np.nonzero(s < tau - eps)[0].tolist())
        got = set(ids.tolist())
        assert must <= got, f"token {t}: missing {must - got}"
        assert not (got & never), f"token {t}: selected {got & never}"
        if len(got ^ set(np.argsort(-s, kind='stable')[:k].tolist())):
            n_ambiguous += 1
        assert np.all(np.diff(s[ids]) <= eps), f"token {t}: ids not ordered by score"
        np.testing.assert_allclose(gpu_w[t].sum(), 1.0, rtol=0, atol=1e-6)
    return n_ambiguous


def topk_candidates(keys, k):
    """Number of experts at or above the selection's candidate threshold for
    one token's keys: the k-th largest of the 64 per-lane maxima, lane l
    holding experts l, l + 64, ...  (the top-k routine's first step, as the
    library's router header describes it).  Above 256 the routine abandons
    its candidate list and runs its exact k-round path."""
    keys = np.asarray(keys)
    lane_max = np.array([keys[l::64].max() for l in range(min(64, keys.size))])
    m = np.sort(lane_max)[::-1][k - 1]
    return int((keys >= m).sum())


def threaded_map(fn, items, what, threads=16):
    """[fn(i) for i in items] on a thread pool (numpy releases the interpreter
    lock in its array loops, so the items run side by side on the host's
    cores), with BLAS held to one thread per call so the pool does not
    oversubscribe the host.  Prints a line each time another eighth of the
    items is done, so long host-side checks show their progress."""
    import concurrent.futures as cf
    import sys
    import time
    from threadpoolctl import threadpool_limits
    items = list(items)
    out = [None] * len(items)
    t0, step = time.time(), max(1, len(items) // 8)
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(min(threads, max(1, len(items)))) as ex:
        futs = {ex.submit(fn, it): i for i, it in enumerate(items)}
        for n, f in enumerate(cf.as_completed(futs), 1):
            out[futs[f]] = f.result()
            if n % step == 0 or n == len(items):
                print(f"  [{what}] {n}/{len(items)} done ({time.time() - t0:.0f} s)", flush=True,
                      file=sys.stderr)
    return out


def oracle_rows(x_bits, orc, ids, w, tokens, **kw):
    """The oracle's moe_forward for each token of `tokens` on its own (rows in
    that order), run side by side (threaded_map)."""
    rows = threaded_map(lambda t: M.moe_forward(x_bits, orc, ids, w, tokens=[t], **kw)[0],
                        [int(t) for t in tokens], "oracle rows")
    return np.stack(rows)


def oracle_weights(scores, ids):
    sel = np.take_along_axis(scores, ids.astype(np.int64), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


# ---- MXFP8 path: the layer's own activation codes against the oracle

U32 = 2.0 ** -23  # a faithfully rounded fp32 operation errs by less than this, relative


def gamma(n):
    """Bound on the relative error of an n-term fp32 sum of exact products in
    any order, as a fraction of the sum of the magnitudes: n u / (1 - n u)."""
    return n * U32 / (1.0 - n * U32)


def scale_pos(blk):
    """Position of block blk's scale byte in an MFMA-ordered scale row (the
    order the library's header gives for its workspace regions)."""
    blk = np.asarray(blk)
    return (blk & ~15) | ((blk & 3) << 2) | ((blk & 15) >> 2)


def _region(b, lay, T, ws, region, dtype):
    return b.workspace_region(lay, T, region, ws).cpu().numpy().view(dtype)


# the two MX activation formats: element encoder, decoder, quantiser, and the
# largest normal exponent that the block-exponent rule subtracts
MX_FORMATS = {
    "e4m3": (F.e4m3_encode_rne_sat, F.e4m3_decode, F.mxfp8_quantize, F.mxfp8_dequant,
             F.E4M3_EMAX),
    "e2m1": (F.e2m1_encode_rne_sat, F.e2m1_decode, F.mxfp4_quantize, F.mxfp4_act_dequant,
             F.E2M1_EMAX),
}


def _between(v_lo, v_hi, fmt):
    """Decoded values that RNE-with-saturation gives to v_lo and v_hi (every
    value in between rounds to a code between them)."""
    enc, dec = MX_FORMATS[fmt][:2]
    return dec(enc(v_lo)), dec(enc(v_hi))


def _block_exp(amax, fmt):
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(np.maximum(amax, 0.0))
    return np.where(amax <= 0, -127, np.clip(ex - 1 - MX_FORMATS[fmt][4], -127, 127))


def unpack_nibbles(packed):
    """uint8 [..., n] of two E2M1 codes per byte -> uint8 [..., 2 n], the even
    element from the low nibble."""
    packed = np.asarray(packed, np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def h_error_bound(xin, wg, wu):
    """(h, dh): the float64 h = SiLU(g) u of the MXFP8 rows xin and a bound on
    how far a fp32 evaluation can land from it.  g and u are fp32 sums of H
    exact products (E2M1 x E4M3 times powers of two), so each errs by at
    most gamma(H) sum|x_k w_k| (Bg, Bu) in any summation order; SiLU's slope
    is below 1.1 everywhere; the SiLU evaluation and the product add a few
    ulp (16 2^-24 relative is taken)."""
    g = xin @ wg.T
    u = xin @ wu.T
    gm = gamma(xin.shape[-1])
    Bg = gm * (np.abs(xin) @ np.abs(wg).T)
    Bu = gm * (np.abs(xin) @ np.abs(wu).T)
    sg = np.abs(M.silu(g))
    au = np.abs(u) + Bu
    dh = 1.1 * Bg * au + sg * Bu + 16 * 2.0 ** -24 * (sg + 1.1 * Bg) * au
    return M.silu(g) * u, dh


def check_h_block_codes(h, dh, codes_g, scales_g, fmt="e4m3"):
    """Element-by-element check of a kernel's MX codes of h (MXFP8 for fmt
    "e4m3", MXFP4 for "e2m1"; rows of I values, codes uint8 [n, I], scale
    bytes [n, I/32] in plain order) against the oracle's quantisation of the
    float64 h.  Equal values pass.
    A differing block exponent must be reachable from some block maximum
    within the fp32 bound dh of the float64 one; a differing code must be
    the rounding of some value within dh of h under the kernel's exponent.
    Returns (delta, n_diff): the kernel's value minus the oracle's per
    element, and how many elements differ.  Raises AssertionError on a code
    no fp32 evaluation of h could produce."""
    n, I = h.shape
    _, dec, quant, dequant, _ = MX_FORMATS[fmt]
    co, so = quant(h)
    vg = dequant(codes_g, scales_g)
    vo = dequant(co, so)
    diff = vg != vo
    if not diff.any():
        return np.zeros_like(h), 0
    Eg = scales_g.astype(np.int64) - 127
    Eo = so.astype(np.int64) - 127
    hb = h.reshape(n, -1, 32)
    db = dh.reshape(n, -1, 32)
    amax = np.abs(hb).max(axis=-1)
    dmax = db.max(axis=-1)
    lo_e, hi_e = _block_exp(amax - dmax, fmt), _block_exp(amax + dmax, fmt)
    bad_exp = (Eg != Eo) & ((Eg < lo_e) | (Eg > hi_e))
    assert not bad_exp.any(), (f"{bad_exp.sum()} block exponents no fp32 h reaches: "
                               f"kernel {Eg[bad_exp][:4]}, oracle {Eo[bad_exp][:4]}")
    sc = np.repeat(np.ldexp(1.0, Eg), 32, axis=-1)
    qg = dec(codes_g)
    lo, hi = _between((h - dh) / sc, (h + dh) / sc, fmt)
    ok = (qg >= np.minimum(lo, hi)) & (qg <= np.maximum(lo, hi))
    bad = diff & ~ok
    assert not bad.any(), (f"{bad.sum()} h codes outside the fp32 bound: kernel "
                           f"{qg[bad][:4]}, allowed [{lo[bad][:4]}, {hi[bad][:4]}], "
                           f"h {h[bad][:4]}")
    return vg - vo, int(diff.sum())


MAX_FLIP_RATE = 1e-2  # far above the observed rate; a wrong rounding rule flips ~1/4 or more


def check_mxfp8_workspace(b, lay, ws, T, x_bits, ids, w, orc, tokens=None, experts=None,
                          x_rows=None, fmt="e4m3"):
    """Checks of an MFMA-path call's intermediate values in its workspace
    (fmt "e4m3": the MXFP8 path; "e2m1": the MXFP4 path, whose code rows
    hold two codes per byte):
      * x codes and block exponents of rows x_rows (default all) bit-exact
        against the oracle's quantiser (x is exact bf16 on both sides),
        zero codes and exponent 127 in the padding past H;
      * the plan: every pair at exactly one position, grouped by expert in
        ascending order;
      * the h codes of every pair of the given experts (default: every expert
        that a token in `tokens` uses; all tokens if None), element by element
        (check_h_block_codes), with zero codes / exponent 127 past I.
    Returns the exact change of each token in `tokens` (rows in that order)
    that the kernel's legitimately different h codes make, w_j Wd (dv) summed
    over its pairs, for check_parity's effect argument."""
    H, I, k = orc.hidden, orc.inter, orc.top_k
    Kq, Iq = -(-H // 512) * 512, -(-I // 512) * 512
    x_bits = np.asarray(x_bits, np.uint16)
    ids = np.asarray(ids, np.int64)
    w = np.asarray(w, np.float64)
    rows = np.arange(T) if x_rows is None else np.asarray(x_rows)
    quant = MX_FORMATS[fmt][2]
    fp4 = fmt == "e2m1"
    xq = _region(b, lay, T, ws, b.WS_X_CODES, np.uint8)
    xq = unpack_nibbles(xq[:T * Kq // 2].reshape(T, Kq // 2)) if fp4 else xq.reshape(T, Kq)
    xs = _region(b, lay, T, ws, b.WS_X_SCALES, np.uint8).reshape(T, Kq // 32)
    rc, rs = quant(F.bf16_decode(x_bits[rows]))
    np.testing.assert_array_equal(xq[rows, :H], rc)
    np.testing.assert_array_equal(xs[rows][:, scale_pos(np.arange(H // 32))], rs)
    assert not xq[rows, H:].any()
    assert (xs[rows][:, scale_pos(np.arange(H // 32, Kq // 32))] == 127).all()
    pairs = _region(b, lay, T, ws, b.WS_PAIRS, np.int32)[:T * k].astype(np.int64)
    assert np.array_equal(np.sort(pairs), np.arange(T * k)), "plan is not a permutation"
    pe = ids.reshape(-1)[pairs]
    assert (np.diff(pe) >= 0).all(), "plan positions not grouped by ascending expert"
    pos_of = np.empty(T * k, np.int64)
    pos_of[pairs] = np.arange(T * k)
    hq = _region(b, lay, T, ws, b.WS_H_CODES, np.uint8)
    hq = (unpack_nibbles(hq[:T * k * Iq // 2].reshape(T * k, Iq // 2)) if fp4
          else hq.reshape(T * k, Iq))
    hsm = _region(b, lay, T, ws, b.WS_H_SCALES, np.uint8).reshape(T * k, Iq // 32)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    if experts is None:
        experts = np.unique(ids[tok])
    row_of = {int(t): r for r, t in enumerate(tok)}
    sg_pos = scale_pos(np.arange(I // 32))
    pad_pos = scale_pos(np.arange(I // 32, Iq // 32))

    def one(e):  # per expert; numpy releases the interpreter lock in its array loops
        t_idx, j_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            return None
        pos = pos_of[t_idx * k + j_idx]
        assert not hq[pos, I:].any() and (hsm[pos][:, pad_pos] == 127).all()
        wg, wu, wd = dequant_expert(orc.expert_record(int(e)), H, I)
        xin = (F.mxfp4_roundtrip if fp4 else F.mxfp8_roundtrip)(F.bf16_decode(x_bits[t_idx]))
        h, dh = h_error_bound(xin, wg, wu)
        delta, nd = check_h_block_codes(h, dh, hq[pos, :I], hsm[pos][:, sg_pos], fmt)
        return t_idx, j_idx, (delta @ wd.T if nd else None), nd, h.size

    results = threaded_map(one, [int(e) for e in experts], "h-code check")
    eff = np.zeros((len(tok), H))
    n_diff = n_el = 0
    for res in results:
        if res is None:
            continue
        t_idx, j_idx, dy, nd, ne = res
        n_diff += nd
        n_el += ne
        if dy is not None:
            for r, (t, j) in enumerate(zip(t_idx, j_idx)):
                if int(t) in row_of:
                    eff[row_of[int(t)]] += w[t, j] * dy[r]
    assert n_diff <= MAX_FLIP_RATE * max(n_el, 1), f"{n_diff} of {n_el} h codes differ"
    print(f"  [h-code check] {n_diff} of {n_el} h codes differ from the oracle's, each within "
          f"the fp32 bound", flush=True)
    return eff


KERNEL_TOL = 5e-4  # error budget beyond the bf16 rounding floor on short rows


ELEM_TOL = 1e-2  # element-wise, in units of the token's RMS output


def check_parity(y_bits, ref, effect=None, strict=False):
    """Per-token output parity against the unrounded float64 oracle.

    The bar is REL_TOL (relative L2 per token).  That figure is set for
    7168-wide rows, where the rounding of the exact answer to bf16 alone
    costs 1.56-1.66e-3; on the short rows of the small test shapes the
    rounding floor itself scatters around 2e-3 (a 256-wide row's correctly
    rounded answer reached 2.17e-3), so a token also passes within its own
    floor ||bf16(ref) - ref|| plus KERNEL_TOL.  Element by element, every
    output must lie within the bf16 rounding bound 2^-8 |ref_i| plus
    ELEM_TOL times the token's RMS output (catches a large error on a few
    elements that the L2 figure would average away).  effect [T, H] (MFMA
    path) is the exact change that the kernel's legitimately different h
    codes make (check_mxfp8_workspace); it is added to the reference.
    """
    y = F.bf16_decode(y_bits)
    ref = np.asarray(ref, np.float64)
    if effect is not None:
        ref = ref + effect
    num = np.linalg.norm(y - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    floor = np.linalg.norm(F.bf16_decode(F.bf16_encode_rne(ref)) - ref, axis=-1)
    bar = REL_TOL * den if strict else np.maximum(REL_TOL * den, floor + KERNEL_TOL * den)
    ok = num <= bar
    assert ok.all(), (f"tokens {np.nonzero(~ok)[0][:8]}: rel err {(num / den)[~ok][:8]}, "
                      f"rounding floor {(floor / den)[~ok][:8]}")
    rms = den / np.sqrt(ref.shape[-1])
    el_bar = 2.0 ** -8 * np.abs(ref) + ELEM_TOL * rms[:, None]
    el_ok = np.abs(y - ref) <= el_bar
    if not el_ok.all():
        t, i = np.nonzero(~el_ok)
        raise AssertionError(f"{t.size} outputs beyond the element bound, e.g. token {t[0]} "
                             f"column {i[0]}: {y[t[0], i[0]]} vs {ref[t[0], i[0]]}")
    return num / den

"""Shared helpers of the GPU parity tests (not collected by pytest)."""

import numpy as np
import torch

import synth
import synth.device as SD
from oracle import formats as F
from oracle import moe as M

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


def oracle_weights(scores, ids):
    sel = np.take_along_axis(scores, ids.astype(np.int64), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


def mxfp8_h_flip_allowance(x_bits, layer, ids, w, rel=5e-5, tokens=None):
    """Per-token bound on how far a correct MXFP8 path may sit from the
    float64 oracle because of h quantisation decisions.

    The kernel decides each h code (and each block exponent) from its fp32
    h; the oracle from its fp64 h.  Where the fp64 value lies within the
    fp32 result's error of an E4M3 rounding midpoint, or a block maximum
    within it of a power of two, both decisions are correct.  That error is
    taken per element as max(rel, 4 sqrt(K) 2^-24 (c_g kappa_g + kappa_u)):
    kappa = sum|x_k w_k| / |sum x_k w_k| is the condition number of the gate
    or up contraction (the fp32 sum's error grows with it, and like sqrt(K)
    for independent roundings: 4 such standard deviations), c_g =
    |1 + g (1 - sigmoid(g))| carries the gate's error through SiLU, and
    rel = 5e-5 (~800 ulp) is the floor for well-conditioned elements; a
    block exponent takes the window of the block's largest element.  For
    such elements the bound adds the largest change of y_t that taking the
    other decision can make: w_j * ||Wd[:, i]||_2 * |step| per element
    (step = the neighbouring code's distance), and for an ambiguous block
    exponent the whole block's quantised contribution.  Elements far from
    any boundary add nothing, so for most tokens the allowance is 0.
    """
    from oracle import formats as F
    from oracle.record import dequant_expert
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    ids = np.asarray(ids, dtype=np.int64)
    rows = np.arange(x_bits.shape[0]) if tokens is None else np.asarray(tokens)
    xin = F.mxfp8_roundtrip(F.bf16_decode(x_bits[rows]))
    ids = ids[rows]
    w = np.asarray(w, dtype=np.float64)[rows]
    bound = np.zeros(len(rows))
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        wg, wu, wd = dequant_expert(layer.expert_record(int(e)), layer.hidden, layer.inter)
        col_norm = np.linalg.norm(wd, axis=0)  # ||Wd[:, i]||
        g = xin[t_idx] @ wg.T
        u = xin[t_idx] @ wu.T
        h = M.silu(g) * u
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            kap_g = (np.abs(xin[t_idx]) @ np.abs(wg).T) / np.abs(g)
            kap_u = (np.abs(xin[t_idx]) @ np.abs(wu).T) / np.abs(u)
            c_g = np.abs(1.0 + g * (1.0 - M.sigmoid(g)))
            rel_el = np.maximum(rel, 4.0 * np.sqrt(layer.hidden) * 2.0 ** -24
                                * (c_g * kap_g + kap_u))
        rel_el = np.where(np.isfinite(rel_el), rel_el, np.inf)
        codes, scales = F.mxfp8_quantize(h)
        E = scales.astype(np.int64) - 127
        scale = np.repeat(np.ldexp(1.0, E), 32, axis=-1)
        v = h / scale                       # value the code rounds
        q = F.e4m3_decode(codes)
        mag = np.abs(v)
        # code spacing at |v| (normal binades 2^(p-3), subnormals 2^-9)
        with np.errstate(divide="ignore"):
            p = np.floor(np.log2(np.maximum(mag, 2.0 ** -12)))
        ulp = np.where(mag >= 2.0 ** -6, np.ldexp(1.0, (p - 3).astype(np.int64)), 2.0 ** -9)
        # distance from the nearest midpoint between two codes
        frac = np.abs(v - q) / ulp          # 0 at a code, 0.5 at a midpoint
        near_mid = (0.5 - frac) * ulp <= rel_el * mag + 1e-300
        amb = near_mid & (mag > 0) & (mag <= 448.0)  # above 448 every value saturates to 448
        contrib = np.where(amb, col_norm[None, :] * ulp * scale, 0.0).sum(axis=1)
        # ambiguous block exponent: the block's whole quantised contribution
        blocks = np.abs(h).reshape(h.shape[0], -1, 32).max(axis=-1)
        with np.errstate(divide="ignore"):
            lg = np.log2(np.maximum(blocks, 1e-300))
        # the exponent follows the block's largest element: its error decides
        hb = np.abs(h).reshape(h.shape[0], -1, 32)
        rel_blk = np.take_along_axis(rel_el.reshape(hb.shape), hb.argmax(axis=-1)[..., None],
                                     axis=-1)[..., 0]
        amb_blk = (np.abs(lg - np.round(lg)) <= rel_blk) & (blocks > 0)
        if amb_blk.any():
            hq = q * scale
            per_blk = np.linalg.norm(hq.reshape(h.shape[0], -1, 32), axis=-1)
            cn_blk = np.linalg.norm(col_norm.reshape(-1, 32), axis=-1)
            contrib = contrib + 2.0 * (amb_blk * per_blk * cn_blk[None, :]).sum(axis=1)
        np.add.at(bound, t_idx, np.abs(w[t_idx, j_idx]) * contrib)
    return bound


KERNEL_TOL = 5e-4  # error budget beyond the bf16 rounding floor on short rows


def check_parity(y_bits, ref, allowance=0.0):
    """Per-token output parity against the unrounded float64 oracle.

    The bar is REL_TOL (relative L2 per token).  That figure is set for
    7168-wide rows, where the rounding of the exact answer to bf16 alone
    costs 1.56-1.66e-3; on the short rows of the small test shapes the
    rounding floor itself scatters around 2e-3 (a 256-wide row's correctly
    rounded answer reached 2.17e-3), so a token also passes within its own
    floor ||bf16(ref) - ref|| plus KERNEL_TOL.  allowance_t adds the bound
    of mxfp8_h_flip_allowance on the MFMA path.
    """
    y = F.bf16_decode(y_bits)
    num = np.linalg.norm(y - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    floor = np.linalg.norm(F.bf16_decode(F.bf16_encode_rne(ref)) - ref, axis=-1)
    bar = np.maximum(REL_TOL * den, floor + KERNEL_TOL * den) + allowance
    ok = num <= bar
    assert ok.all(), (f"tokens {np.nonzero(~ok)[0][:8]}: rel err {(num / den)[~ok][:8]}, "
                      f"rounding floor {(floor / den)[~ok][:8]}, "
                      f"allowance {(np.broadcast_to(allowance, num.shape) / den)[~ok][:8]}")
    return num / den


def check_mxfp8_parity(y_bits, ref, allowance):
    """check_parity with the MXFP8 h-decision allowance."""
    return check_parity(y_bits, ref, allowance)

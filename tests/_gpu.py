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

    def __init__(self, cfg, seed=0, layer=0, bias=False):
        self.cfg = cfg
        self.seed, self.layer_idx = seed, layer
        d = SD.upload_layer(cfg, seed, layer, bias=bias)
        self.dev = d
        self.repack()
        H, I = cfg["hidden"], cfg["inter"]
        self.oracle = M.Layer(H, I, cfg["n_experts"], cfg["top_k"], d["host_router_w"],
                              expert_record=lambda e: synth.expert_record(seed, layer, e, H, I),
                              shared=d["host_shared"], router_bias=d["host_bias"])

    def repack(self):
        from mxfp4_routed_expert_x896_amd import binding
        c, d = self.cfg, self.dev
        self.lib = binding.Layer.from_canonical(
            c["hidden"], c["inter"], c["n_experts"], c["top_k"], d["router_w"], d["experts"],
            d["shared_gate"], d["shared_up"], d["shared_down"], d["router_bias"])
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

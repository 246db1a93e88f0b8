"""Router, expert FFN, shared experts, combine and RMSNorm in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Per token and MoE layer (Deltafin explainer section 5.1; Deltafin README,
"How it works"): the router picks 16 of the 896 routed experts, the selected
experts' MXFP4 weights are applied, and the results of the two always-on
shared experts are added before the next layer.  The pages do not give the
router's formula or the expert's activation; the readings used here:
  * scores s = sigmoid(router logits), with an optional per-expert bias added
    to the logits before the sigmoid;
  * the k largest scores are selected, exact ties going to the lower expert
    index; combine weights are the selected scores divided by their sum;
  * two router variants the pages leave open, as the DeepSeek-V3 report
    defines its gate (section 2.1.2, auxiliary-loss-free balancing):
    bias_mode "select" adds the bias to the sigmoid scores for the choice
    only (key = s + b) and takes the weights from the unbiased s; and a
    routed scaling factor multiplies the combine weights (1 by default);
  * an expert is a SwiGLU FFN: y = Wd (SiLU(Wg x) * (Wu x));
  * shared experts are bf16 SwiGLU FFNs of the same shape, added with
    weight 1;
  * prefill variant: the routed experts see x, and later h, rounded to MXFP8
    (E4M3 codes plus an E8M0 exponent per 32 elements along the contraction),
    following the MXFP8-activation training noted in the explainer, section
    2.1.  The router and the shared experts keep the bf16 x.  A second
    prefill variant rounds them to MXFP4 instead (E2M1 codes, the weights'
    own format), for the FP4 x FP4 matrix-core rate.
"""

import numpy as np

from .formats import bf16_decode, bf16_encode_rne, mxfp4_roundtrip, mxfp8_roundtrip
from .record import dequant_expert


class Layer:
    """Plain description of one MoE layer for the oracle.

    router_w:      uint16 bf16 bits [E, H]
    router_bias:   float32 [E] or None
    bias_mode:     "logits" (bias added to the logits, for the choice and the
                   weights) or "select" (added to the scores for the choice)
    routed_scale:  factor on the combine weights
    expert_record: callable e -> uint8 record bytes of expert e
    shared:        list of (gate [I,H], up [I,H], down [H,I]) bf16 bit arrays
    """

    def __init__(self, hidden, inter, n_experts, top_k, router_w,
                 expert_record, shared=(), router_bias=None, bias_mode="logits",
                 routed_scale=1.0):
        self.hidden = int(hidden)
        self.inter = int(inter)
        self.n_experts = int(n_experts)
        self.top_k = int(top_k)
        self.router_w = np.asarray(router_w, dtype=np.uint16)
        self.router_bias = None if router_bias is None else np.asarray(router_bias, dtype=np.float32)
        self.expert_record = expert_record
        self.shared = list(shared)
        if bias_mode not in ("logits", "select"):
            raise ValueError("bias_mode is 'logits' or 'select'")
        self.bias_mode = bias_mode
        self.routed_scale = float(routed_scale)
        if self.router_w.shape != (self.n_experts, self.hidden):
            raise ValueError("router weight must be [E, H]")
        if not 1 <= self.top_k <= self.n_experts:
            raise ValueError("top_k out of range")


def sigmoid(z):
    """1 / (1 + exp(-z)) in float64 (exp overflow gives exactly 0)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def silu(z):
    """z * sigmoid(z), written z / (1 + exp(-z)) so overflow gives -0, not NaN."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def router_logits(x_bits, router_w_bits, bias=None):
    """l[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]), exact bf16 inputs."""
    x = bf16_decode(x_bits)
    w = bf16_decode(router_w_bits)
    logits = x @ w.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return logits


def select_topk(scores, k):
    """Indices of the k largest scores per row, ties to the lower index.

    Ordered by (score descending, index ascending): a stable sort on -score.
    """
    scores = np.asarray(scores, dtype=np.float64)
    order = np.argsort(-scores, axis=-1, kind="stable")
    return order[..., :k]


def router_scores(x_bits, layer):
    """(s, key) [T,E]: s weighs the chosen experts, key chooses them."""
    if layer.bias_mode == "logits":
        s = sigmoid(router_logits(x_bits, layer.router_w, layer.router_bias))
        return s, s
    s = sigmoid(router_logits(x_bits, layer.router_w))
    if layer.router_bias is None:
        return s, s
    return s, s + np.asarray(layer.router_bias, dtype=np.float32).astype(np.float64)[None, :]


def combine_weights(s, ids, routed_scale=1.0):
    """routed_scale * s[ids] / sum(s[ids]) per token, for any chosen ids."""
    sel = np.take_along_axis(np.asarray(s, dtype=np.float64), np.asarray(ids, dtype=np.int64),
                             axis=-1)
    return routed_scale * sel / np.sum(sel, axis=-1, keepdims=True)


def route(x_bits, layer):
    """Router: (topk ids int64 [T,k], weights float64 [T,k], selection keys
    [T,E]; the keys are the scores s unless bias_mode is "select")."""
    s, key = router_scores(x_bits, layer)
    ids = select_topk(key, layer.top_k)
    return ids, combine_weights(s, ids, layer.routed_scale), key


def expert_ffn(xv, wg, wu, wd, act_mxfp8=False, act_mxfp4=False):
    """SwiGLU expert on float64 rows xv [T, H]: Wd (SiLU(Wg x) * (Wu x)).

    act_mxfp8 / act_mxfp4: x and h are replaced by their MXFP8 (or MXFP4)
    values along the contraction dimension before the respective products.
    """
    if act_mxfp8 and act_mxfp4:
        raise ValueError("one activation format")
    rnd = mxfp8_roundtrip if act_mxfp8 else mxfp4_roundtrip if act_mxfp4 else None
    xin = rnd(xv) if rnd else xv
    g = xin @ wg.T
    u = xin @ wu.T
    h = silu(g) * u
    if rnd:
        h = rnd(h)
    return h @ wd.T


def shared_ffn(xv, gate_bits, up_bits, down_bits):
    """One bf16 shared expert on float64 rows (exact bf16 weights)."""
    wg = bf16_decode(gate_bits)
    wu = bf16_decode(up_bits)
    wd = bf16_decode(down_bits)
    return (silu(xv @ wg.T) * (xv @ wu.T)) @ wd.T


def routed_sum(x_bits, layer, topk_ids, topk_w, act_mxfp8=False, tokens=None, act_mxfp4=False):
    """sum_j w[t, j] * expert_{ids[t, j]}(x_t) for the given routing.

    Each expert touched is dequantised once and applied to all its tokens.
    tokens: optional subset of token indices to evaluate (rows of the result
    follow that order).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    rows = np.arange(x_bits.shape[0]) if tokens is None else np.asarray(tokens)
    xv = bf16_decode(x_bits[rows])
    ids = ids[rows]
    w = w[rows]
    out = np.zeros((len(rows), layer.hidden), dtype=np.float64)
    # contributions are added in slot order per token
    contrib = {}
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        wg, wu, wd = dequant_expert(layer.expert_record(int(e)), layer.hidden, layer.inter)
        ye = expert_ffn(xv[t_idx], wg, wu, wd, act_mxfp8, act_mxfp4)
        for r, (t, j) in enumerate(zip(t_idx, j_idx)):
            contrib[(int(t), int(j))] = ye[r]
    for t in range(len(rows)):
        for j in range(ids.shape[1]):
            out[t] += w[t, j] * contrib[(t, j)]
    return out


def shared_sum(x_bits, layer, tokens=None):
    """sum_s shared_s(x_t) with weight 1 each (explainer section 5.1)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows = np.arange(x_bits.shape[0]) if tokens is None else np.asarray(tokens)
    xv = bf16_decode(x_bits[rows])
    out = np.zeros((len(rows), layer.hidden), dtype=np.float64)
    for g, u, d in layer.shared:
        out += shared_ffn(xv, g, u, d)
    return out


def moe_forward(x_bits, layer, topk_ids, topk_w, act_mxfp8=False,
                residual_bits=None, tokens=None, act_mxfp4=False):
    """y = [residual +] sum_j w_j expert_{id_j}(x) + sum_s shared_s(x).

    Unrounded float64; the product rounds once, to bf16, at the output.
    """
    y = routed_sum(x_bits, layer, topk_ids, topk_w, act_mxfp8, tokens, act_mxfp4)
    y = y + shared_sum(x_bits, layer, tokens)
    if residual_bits is not None:
        r = np.asarray(residual_bits, dtype=np.uint16)
        rows = np.arange(r.shape[0]) if tokens is None else np.asarray(tokens)
        y = y + bf16_decode(r[rows])
    return y


def moe_layer(x_bits, layer, act_mxfp8=False, residual_bits=None, act_mxfp4=False):
    """Route then combine: (y float64 [T,H], ids, weights)."""
    ids, w, _ = route(x_bits, layer)
    y = moe_forward(x_bits, layer, ids, w, act_mxfp8, residual_bits, act_mxfp4=act_mxfp4)
    return y, ids, w


def rmsnorm(x_bits, gamma_bits, eps=1e-6):
    """x * (mean(x^2) + eps)^(-1/2) * gamma, rounded once to bf16 bits."""
    x = bf16_decode(x_bits)
    g = bf16_decode(gamma_bits)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return bf16_encode_rne(x * r * g)

"""Pins for the oracle's expert FFN, shared experts, combine and RMSNorm.

Closed forms on hand-built sparse experts (which fail on a swapped gate/up,
a transposed matrix, a wrong nibble or block index), the invariants the
layer must satisfy (all experts equal -> one dense FFN independent of
routing; zero routed experts -> shared experts only; one more scale
exponent -> exactly twice the expert output), torch's RMSNorm, and the
whole layer against a result assembled by hand from per-token routing and
closed-form experts.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from oracle import record as R

H, I = 64, 32
ONE, TWO, HALF = 2, 4, 1  # E2M1 codes for 1.0, 2.0, 0.5


def _sparse_record(entries):
    """Record whose matrices are zero except the given (matrix, row, col, code)."""
    rec = np.zeros(R.record_bytes(H, I), dtype=np.uint8)
    # layout written out independently of the oracle's parser
    cg = I * H // 2
    sg = I * H // 32
    base = {0: 0, 1: cg + sg, 2: 2 * (cg + sg)}
    ncols = {0: H, 1: H, 2: I}
    nrows = {0: I, 1: I, 2: H}
    for m in range(3):
        codes = nrows[m] * ncols[m] // 2
        scales = nrows[m] * ncols[m] // 32
        rec[base[m] + codes: base[m] + codes + scales] = 127
    for m, r, c, code in entries:
        byte = base[m] + r * (ncols[m] // 2) + c // 2
        rec[byte] |= code if c % 2 == 0 else code << 4
    return rec


def _expert_a():
    e = [(0, n, n, ONE) for n in range(I)]          # g = x[0:I]
    e += [(1, n, n + 1, TWO) for n in range(I)]     # u = 2 x[1:I+1]
    e += [(2, m, m % I, HALF) for m in range(H)]    # y[m] = h[m % I] / 2
    return _sparse_record(e)


def _expert_b():
    e = [(0, n, n + 2, ONE) for n in range(I)]      # g = x[2:I+2]
    e += [(1, n, n, ONE) for n in range(I)]         # u = x[0:I]
    e += [(2, m, (m + 3) % I, ONE) for m in range(H)]
    return _sparse_record(e)


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _closed_a(x):
    return np.array([0.5 * _silu(x[m % I]) * 2.0 * x[m % I + 1] for m in range(H)])


def _closed_b(x):
    return np.array([_silu(x[(m + 3) % I + 2]) * x[(m + 3) % I] for m in range(H)])


def _x(seed, t=1):
    return synth.activations(seed, t, H)


def _layer(records, shared=(), k=2, router_seed=0, bias=None):
    wr = synth.router_weight(router_seed, 0, len(records), H)
    return M.Layer(H, I, len(records), k, wr, expert_record=lambda e: records[e],
                   shared=shared, router_bias=bias)


def test_sparse_expert_closed_form():
    x_bits = _x(1000, 3)
    xv = F.bf16_decode(x_bits)
    for rec, closed in ((_expert_a(), _closed_a), (_expert_b(), _closed_b)):
        wg, wu, wd = R.dequant_expert(rec, H, I)
        y = M.expert_ffn(xv, wg, wu, wd)
        for t in range(3):
            np.testing.assert_allclose(y[t], closed(xv[t]), rtol=1e-14, atol=1e-300)


def test_combine_closed_form_with_given_routing():
    recs = [_expert_a(), _expert_b()]
    layer = _layer(recs)
    x_bits = _x(1001, 2)
    xv = F.bf16_decode(x_bits)
    ids = np.array([[0, 1], [1, 0]])
    w = np.array([[0.3, 0.7], [0.9, 0.1]])
    y = M.moe_forward(x_bits, layer, ids, w)
    np.testing.assert_allclose(y[0], 0.3 * _closed_a(xv[0]) + 0.7 * _closed_b(xv[0]), rtol=1e-13)
    np.testing.assert_allclose(y[1], 0.9 * _closed_b(xv[1]) + 0.1 * _closed_a(xv[1]), rtol=1e-13)


def test_shared_expert_closed_form_and_added_with_weight_one():
    g = np.zeros((I, H), dtype=np.uint16)
    u = np.zeros((I, H), dtype=np.uint16)
    d = np.zeros((H, I), dtype=np.uint16)
    for n in range(I):
        g[n, n] = 0x3F80
        u[n, n] = 0x4000  # 2.0
    for m in range(H):
        d[m, m % I] = 0x3F00  # 0.5
    zero = np.zeros(R.record_bytes(H, I), dtype=np.uint8)
    layer = _layer([zero, zero, zero], shared=[(g, u, d), (g, u, d)])
    x_bits = _x(1002, 2)
    xv = F.bf16_decode(x_bits)
    y, ids, w = M.moe_layer(x_bits, layer)
    for t in range(2):
        closed = np.array([2 * 0.5 * _silu(xv[t, m % I]) * 2 * xv[t, m % I] for m in range(H)])
        np.testing.assert_allclose(y[t], closed, rtol=1e-14)


def test_all_experts_equal_reduces_to_dense_ffn():
    rec = synth.expert_record(0, 0, 3, H, I)
    sh = [synth.shared_expert(0, 0, 0, H, I)]
    x_bits = _x(1003, 4)
    xv = F.bf16_decode(x_bits)
    wg, wu, wd = R.dequant_expert(rec, H, I)
    dense = M.expert_ffn(xv, wg, wu, wd) + M.shared_ffn(xv, *sh[0])
    outs = []
    for router_seed, bias in ((0, None), (5, None), (9, synth.router_bias(0, 0, 8))):
        layer = _layer([rec] * 8, shared=sh, k=3, router_seed=router_seed, bias=bias)
        y, ids, _ = M.moe_layer(x_bits, layer)
        outs.append(ids)
        np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())
    assert not all(np.array_equal(outs[0], o) for o in outs[1:])  # routing did change


def test_zero_routed_experts_leave_shared_only():
    zero = np.zeros(R.record_bytes(H, I), dtype=np.uint8)  # all codes 0 (scale bytes 0 too)
    sh = [synth.shared_expert(0, 0, s, H, I) for s in range(2)]
    layer = _layer([zero] * 4, shared=sh)
    x_bits = _x(1004, 3)
    xv = F.bf16_decode(x_bits)
    y, _, _ = M.moe_layer(x_bits, layer)
    np.testing.assert_array_equal(y, M.shared_ffn(xv, *sh[0]) + M.shared_ffn(xv, *sh[1]))


@pytest.mark.parametrize("matrix", [R.UP, R.DOWN])
def test_one_more_scale_exponent_doubles_expert_output_exactly(matrix):
    rec = synth.expert_record(0, 0, 1, H, I)
    rec2 = rec.copy()
    R.split(rec2, H, I)[2 * matrix + 1][...] += 1
    xv = F.bf16_decode(_x(1005, 2))
    y1 = M.expert_ffn(xv, *R.dequant_expert(rec, H, I))
    y2 = M.expert_ffn(xv, *R.dequant_expert(rec2, H, I))
    np.testing.assert_array_equal(y2, 2.0 * y1)


def test_mxfp8_activation_path_on_grid_input():
    """x already on the MXFP8 grid is unchanged; h is rounded to MXFP8."""
    g = np.random.default_rng(1)
    xv = g.integers(-4, 5, size=(2, H)).astype(np.float64)
    xv[:, 0] = 4.0  # amax 4 in the first block
    xv[:, 32] = -4.0  # and in the second
    x_bits = F.bf16_encode_rne(xv)
    np.testing.assert_array_equal(F.mxfp8_roundtrip(xv), xv)
    rec = _expert_a()
    wg, wu, wd = R.dequant_expert(rec, H, I)
    y = M.expert_ffn(F.bf16_decode(x_bits), wg, wu, wd, act_mxfp8=True)
    for t in range(2):
        h = np.array([_silu(xv[t, n]) * 2.0 * xv[t, n + 1] for n in range(I)])
        hq = F.mxfp8_roundtrip(h[None, :])[0]
        np.testing.assert_allclose(y[t], [0.5 * hq[m % I] for m in range(H)], rtol=1e-15)
        assert not np.allclose(hq, h, rtol=1e-6)  # the rounding did something


def test_rmsnorm_closed_form_and_torch():
    c = 2.0
    x = F.bf16_encode_rne(np.full((1, H), c))
    gam = F.bf16_encode_rne(np.ones(H))
    expect = F.bf16_encode_rne(np.full((1, H), c / math.sqrt(c * c + 1e-6)))
    np.testing.assert_array_equal(M.rmsnorm(x, gam, 1e-6), expect)
    xb = synth.activations(1006, 8, 7168)
    gb = synth.rms_gamma(0, 0, 7168)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(F.bf16_decode(xb)), (7168,),
                                       weight=torch.from_numpy(F.bf16_decode(gb)), eps=1e-6)
    np.testing.assert_array_equal(M.rmsnorm(xb, gb, 1e-6), F.bf16_encode_rne(ref.numpy()))


def test_mxfp4_activation_path_on_grid_input():
    """x already on the MXFP4 grid is unchanged; h is rounded to MXFP4 (the
    same closed form as the MXFP8 pin above, with the E2M1 grid)."""
    g = np.random.default_rng(2)
    xv = F.e2m1_decode(g.integers(0, 16, size=(2, H))).astype(np.float64)
    xv[:, 0] = 6.0   # amax 6 in both blocks: E = 0, values on the grid stay
    xv[:, 32] = -6.0
    x_bits = F.bf16_encode_rne(xv)
    np.testing.assert_array_equal(F.mxfp4_roundtrip(xv), xv)
    rec = _expert_a()
    wg, wu, wd = R.dequant_expert(rec, H, I)
    y = M.expert_ffn(F.bf16_decode(x_bits), wg, wu, wd, act_mxfp4=True)
    for t in range(2):
        h = np.array([_silu(xv[t, n]) * 2.0 * xv[t, n + 1] for n in range(I)])
        hq = F.mxfp4_roundtrip(h[None, :])[0]
        np.testing.assert_allclose(y[t], [0.5 * hq[m % I] for m in range(H)], rtol=1e-15)
        assert not np.allclose(hq, h, rtol=1e-3)  # the rounding did something
    with pytest.raises(ValueError):
        M.expert_ffn(xv, wg, wu, wd, act_mxfp8=True, act_mxfp4=True)


def test_mxfp4_mode_all_experts_equal_is_dense_ffn_of_rounded_activations():
    """Every expert identical: the routed sum is one expert's FFN, whatever the
    routing, computed on MXFP4-rounded x and h."""
    rec = synth.expert_record(5, 0, 0, H, I)
    layer = M.Layer(H, I, 8, 3, synth.router_weight(5, 0, 8, H), expert_record=lambda e: rec)
    x = synth.activations(1500, 5, H)
    y, ids, w = M.moe_layer(x, layer, act_mxfp4=True)
    wg, wu, wd = R.dequant_expert(rec, H, I)
    xq = F.mxfp4_roundtrip(F.bf16_decode(x))
    hq = F.mxfp4_roundtrip(M.silu(xq @ wg.T) * (xq @ wu.T))
    np.testing.assert_allclose(y, hq @ wd.T, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def _bf16_value(bits):
    """bf16 bit pattern -> float, through the float32 pattern (bits << 16)."""
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_layer_end_to_end_from_per_token_routing_and_closed_forms():
    """The whole layer on 3 tokens and 5 distinct experts against a result
    assembled here by hand: logits as exactly rounded sums (math.fsum) of the
    bf16 products, scores sorted as (score desc, index asc) tuples, weights
    renormalised, and each expert's output from its closed form (expert e is
    closed form a or b, by parity, times 2^e through its down matrix's block
    exponents), plus the residual.  Catches a token's routing applied to
    another token, a weight paired with the wrong expert, or an expert id
    read from the wrong slot -- which the all-experts-equal and zero-expert
    invariants cannot see."""
    E, k, T = 5, 2, 3
    cg, sg = I * H // 2, I * H // 32
    recs = []
    for e in range(E):
        rec = (_expert_a() if e % 2 == 0 else _expert_b()).copy()
        down_scales = 2 * (cg + sg) + H * I // 2
        rec[down_scales: down_scales + H * I // 32] = 127 + e
        recs.append(rec)
    closed = [_closed_a if e % 2 == 0 else _closed_b for e in range(E)]
    layer = _layer(recs, k=k, router_seed=3)
    x_bits = _x(1010, T)
    res_bits = synth.activations(1011, T, H)
    y, ids, w = M.moe_layer(x_bits, layer, residual_bits=res_bits)
    wr = layer.router_w
    for t in range(T):
        xt = [_bf16_value(b) for b in x_bits[t]]
        logit = [math.fsum(xt[h] * _bf16_value(wr[e, h]) for h in range(H)) for e in range(E)]
        score = [1.0 / (1.0 + math.exp(-v)) for v in logit]
        order = sorted(range(E), key=lambda e: (-score[e], e))
        assert score[order[k - 1]] - score[order[k]] > 1e-9  # no near-tie at the cut
        chosen = order[:k]
        total = sum(score[e] for e in chosen)
        assert list(ids[t]) == chosen
        np.testing.assert_allclose(w[t], [score[e] / total for e in chosen], rtol=1e-13)
        want = [_bf16_value(b) for b in res_bits[t]]
        for e in chosen:
            want = np.asarray(want) + (score[e] / total) * 2.0 ** e * closed[e](np.asarray(xt))
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # the tokens do not all take the same experts (else a token mix-up would pass)
    assert len({tuple(r) for r in ids.tolist()}) > 1

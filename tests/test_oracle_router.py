"""Pins for the oracle's router (CPU only).

Selection is checked against brute force over every k-subset, exact ties
against duplicated router rows, scores against the sigmoid's closed form on
one-hot inputs (which also pins the router's orientation), and the combine
weights against the sum-to-one invariant.
"""

import itertools
import math

import numpy as np

import synth
from oracle import formats as F
from oracle import moe as M


def _tiny_layer(seed=0, router=None, bias=None, k=4):
    c = synth.TINY
    wr = synth.router_weight(seed, 0, c["n_experts"], c["hidden"]) if router is None else router
    return M.Layer(c["hidden"], c["inter"], c["n_experts"], k, wr,
                   expert_record=lambda e: synth.expert_record(seed, 0, e, c["hidden"], c["inter"]),
                   router_bias=bias)


def test_topk_equals_brute_force_best_subset():
    """The k-subset with the largest score sum, lexicographically first on ties."""
    for seed in range(6):
        layer = _tiny_layer(seed)
        x = synth.activations(1000 + seed, 3, layer.hidden)
        ids, w, s = M.route(x, layer)
        for t in range(x.shape[0]):
            best, best_sum = None, -1.0
            for sub in itertools.combinations(range(layer.n_experts), layer.top_k):
                tot = sum(s[t, e] for e in sub)
                if tot > best_sum:  # strict: the first (lexicographic) subset wins ties
                    best, best_sum = sub, tot
            assert sorted(ids[t].tolist()) == list(best)
            # ordered by score descending
            assert np.all(np.diff(s[t, ids[t]]) <= 0)


def test_exact_ties_go_to_lower_index():
    c = synth.TINY
    wr = synth.router_weight(0, 0, c["n_experts"], c["hidden"])
    # every router row identical: all scores tie, so experts 0..k-1 win
    same = np.repeat(wr[:1], c["n_experts"], axis=0)
    layer = _tiny_layer(router=same)
    x = synth.activations(1000, 2, c["hidden"])
    ids, w, _ = M.route(x, layer)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2
    np.testing.assert_allclose(w, 0.25, rtol=0, atol=1e-15)
    # duplicate the best row of token 0 into a higher and a lower slot
    layer = _tiny_layer()
    ids0, _, s0 = M.route(x, layer)
    top = int(ids0[0, 0])
    dup = layer.router_w.copy()
    lo_slot = 0 if top != 0 else 1
    dup[lo_slot] = dup[top]
    dup[31 if top != 31 else 30] = dup[top]
    ids1, _, s1 = M.route(x, _tiny_layer(router=dup))
    first_two = ids1[0, :2].tolist()
    assert first_two == sorted([lo_slot, top])


def test_scores_are_sigmoid_of_router_column_for_one_hot_input():
    """x = e_h gives logits = Wr[:, h]; catches a transposed router."""
    layer = _tiny_layer()
    h = 37
    x = np.zeros((1, layer.hidden), dtype=np.uint16)
    x[0, h] = 0x3F80  # bf16 1.0
    _, _, s = M.route(x, layer)
    col = F.bf16_decode(layer.router_w[:, h])
    expect = [1.0 / (1.0 + math.exp(-v)) for v in col]
    np.testing.assert_allclose(s[0], expect, rtol=1e-15, atol=0)


def test_bias_is_added_to_logits_before_sigmoid():
    c = synth.TINY
    bias = synth.router_bias(0, 0, c["n_experts"])
    layer = _tiny_layer(bias=bias)
    h = 5
    x = np.zeros((1, c["hidden"]), dtype=np.uint16)
    x[0, h] = 0x4000  # bf16 2.0
    ids, w, s = M.route(x, layer)
    col = F.bf16_decode(layer.router_w[:, h])
    expect = np.array([1.0 / (1.0 + math.exp(-(2.0 * v + float(b)))) for v, b in zip(col, bias)])
    np.testing.assert_allclose(s[0], expect, rtol=1e-15, atol=0)
    assert sorted(ids[0].tolist()) == sorted(np.argsort(-expect, kind="stable")[:4].tolist())


def test_weights_renormalise_over_selected():
    layer = _tiny_layer()
    x = synth.activations(1001, 16, layer.hidden)
    ids, w, s = M.route(x, layer)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    sel = np.take_along_axis(s, ids, axis=1)
    # weights are proportional to the selected scores
    np.testing.assert_allclose(w / w[:, :1], sel / sel[:, :1], rtol=1e-14)
    # every selected score is at least every unselected one
    for t in range(x.shape[0]):
        rest = np.setdiff1d(np.arange(layer.n_experts), ids[t])
        assert s[t, ids[t]].min() >= s[t, rest].max()

"""Pins for the oracle's router (CPU only).

Selection is checked against brute force over every k-subset, exact ties
against duplicated router rows, scores against the sigmoid's closed form on
one-hot inputs (which also pins the router's orientation), and the combine
weights against the sum-to-one invariant.
"""

import itertools
import math

import numpy as np
import pytest

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


# ---- router variants: bias on the scores for the choice only, routed scale

def _one_hot(h, bits=0x3F80, hidden=256):
    x = np.zeros((1, hidden), dtype=np.uint16)
    x[0, h] = bits
    return x


def _select_layer(bias, k=4, routed_scale=1.0, router=None):
    c = synth.TINY
    wr = synth.router_weight(0, 0, c["n_experts"], c["hidden"]) if router is None else router
    return M.Layer(c["hidden"], c["inter"], c["n_experts"], k, wr,
                   expert_record=lambda e: synth.expert_record(0, 0, e, c["hidden"], c["inter"]),
                   router_bias=bias, bias_mode="select", routed_scale=routed_scale)


def test_select_mode_choice_is_brute_force_over_biased_scores():
    """One-hot x = 4 e_h: logits 4 Wr[:, h] in closed form.  The chosen
    subset maximises sum(s + b); the weights are the UNBIASED s renormalised."""
    c = synth.TINY
    for seed in range(4):
        bias = synth.router_bias(seed, 0, c["n_experts"]).astype(np.float32)
        layer = _select_layer(bias)
        h = 11 + 7 * seed
        ids, w, key = M.route(_one_hot(h, 0x4080), layer)  # bf16 4.0
        col = F.bf16_decode(layer.router_w[:, h])
        s = np.array([1.0 / (1.0 + math.exp(-4.0 * v)) for v in col])
        kk = s + bias.astype(np.float64)
        np.testing.assert_allclose(key[0], kk, rtol=1e-15, atol=0)
        best, best_sum = None, -np.inf
        for sub in itertools.combinations(range(c["n_experts"]), 4):
            tot = sum(kk[e] for e in sub)
            if tot > best_sum:
                best, best_sum = sub, tot
        assert sorted(ids[0].tolist()) == list(best)
        assert np.all(np.diff(kk[ids[0]]) <= 0)
        sel = s[ids[0]]
        np.testing.assert_allclose(w[0], sel / sel.sum(), rtol=1e-15, atol=0)


def test_select_mode_bias_decides_a_choice_the_logits_mode_does_not():
    """A bias of +1 on the expert with the lowest score: on the scores
    (each below 1) it must win; on the logits it need not.  Its weight
    still comes from its own small unbiased score."""
    c = synth.TINY
    h = 3
    x = _one_hot(h, 0x4220)  # bf16 40.0: logits from about -12 to +27
    col = F.bf16_decode(synth.router_weight(0, 0, c["n_experts"], c["hidden"])[:, h])
    s = np.array([1.0 / (1.0 + math.exp(-40.0 * v)) for v in col])
    low = int(np.argmin(s))
    bias = np.zeros(c["n_experts"], dtype=np.float32)
    bias[low] = 1.0
    ids, w, _ = M.route(x, _select_layer(bias))
    assert ids[0, 0] == low
    rest = [e for e in np.argsort(-s, kind="stable") if e != low][:3]
    assert ids[0, 1:].tolist() == rest
    sel = s[[low] + rest]
    np.testing.assert_allclose(w[0], sel / sel.sum(), rtol=1e-15, atol=0)
    assert w[0, 0] < w[0, 1]  # the biased winner carries its small score
    ids_l, _, _ = M.route(x, _tiny_layer(bias=bias))
    assert low not in ids_l[0].tolist()  # +1 on a logit of about -12 is not enough


def test_select_mode_ignores_a_constant_bias_and_equals_logits_mode_at_zero():
    c = synth.TINY
    x = synth.activations(1010, 6, c["hidden"])
    bias = synth.router_bias(3, 0, c["n_experts"]).astype(np.float32)
    ids, w, _ = M.route(x, _select_layer(bias))
    ids2, w2, _ = M.route(x, _select_layer(bias + np.float32(0.25)))
    assert np.array_equal(ids, ids2)
    np.testing.assert_array_equal(w, w2)  # weights never see the bias
    ids0, w0, s0 = M.route(x, _select_layer(np.zeros(c["n_experts"], np.float32)))
    idsn, wn, sn = M.route(x, _tiny_layer())
    assert np.array_equal(ids0, idsn)
    np.testing.assert_array_equal(w0, wn)


def test_routed_scale_multiplies_the_routed_part_only():
    """Weights sum to the scale; y(2) - y(1) equals the routed part y(1) - shared."""
    c = synth.TINY
    shared = [synth.shared_expert(0, 0, 0, c["hidden"], c["inter"])]
    mk = lambda scale: M.Layer(c["hidden"], c["inter"], c["n_experts"], c["top_k"],
                               synth.router_weight(0, 0, c["n_experts"], c["hidden"]),
                               expert_record=lambda e: synth.expert_record(0, 0, e, c["hidden"],
                                                                          c["inter"]),
                               shared=shared, routed_scale=scale)
    x = synth.activations(1011, 3, c["hidden"])
    y1, ids1, w1 = M.moe_layer(x, mk(1.0))
    y2, ids2, w2 = M.moe_layer(x, mk(2.0))
    assert np.array_equal(ids1, ids2)
    np.testing.assert_allclose(w2.sum(axis=1), 2.0, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(w2, 2.0 * w1)
    sh = M.shared_sum(x, mk(1.0))
    np.testing.assert_allclose(y2 - y1, y1 - sh, rtol=0, atol=1e-12 * np.abs(y1).max())
    assert np.abs(y1 - sh).max() > 1e-3  # the routed part is not empty


# ---- the tie rule at the K3 expert count and the largest supported one

def _wide_layer(router, k, bias=None, bias_mode="logits"):
    E, H = router.shape
    return M.Layer(H, 64, E, k, router,
                   expert_record=lambda e: synth.expert_record(0, 0, e, H, 64),
                   router_bias=bias, bias_mode=bias_mode)


@pytest.mark.parametrize("E,k", [(896, 16), (1024, 32)])
def test_all_tied_rows_pick_the_lowest_indices(E, k):
    """Every router row equal: all E scores tie exactly, so the choice is
    experts 0..k-1 in index order and each weight is 1/k.  At these sizes an
    unstable sort returns the top indices first, so this pins the tie rule
    where the K3 layer (E = 896) and the largest layer (E = 1024) use it."""
    H = 256
    row = synth.router_weight(0, 0, 1, H)
    layer = _wide_layer(np.repeat(row, E, axis=0), k)
    x = synth.activations(1020, 3, H)
    ids, w, s = M.route(x, layer)
    assert (s == s[:, :1]).all()
    assert ids.tolist() == [list(range(k))] * 3
    np.testing.assert_allclose(w, 1.0 / k, rtol=0, atol=1e-15)


@pytest.mark.parametrize("E,k", [(896, 16), (1024, 32)])
def test_tied_score_classes_follow_the_lexicographic_order(E, k):
    """Router rows drawn from 5 distinct rows: the scores take 5 values, each
    shared by about E/5 experts spread over all indices.  The selection must
    equal the first k of all experts listed by (score descending, index
    ascending), written here as a plain sort on that tuple."""
    H = 256
    rows = synth.router_weight(7, 0, 5, H)
    pick = np.random.default_rng([7, E]).integers(0, 5, size=E)
    layer = _wide_layer(rows[pick], k)
    x = synth.activations(1021, 4, H)
    ids, w, s = M.route(x, layer)
    for t in range(x.shape[0]):
        want = sorted(range(E), key=lambda e: (-s[t, e], e))[:k]
        assert ids[t].tolist() == want
        assert len(set(s[t].tolist())) == 5


def test_select_mode_ties_at_k3_size_pick_the_lowest_indices():
    """The choice on s + b with every row and bias equal: all keys tie."""
    E, k, H = 896, 16, 256
    row = synth.router_weight(0, 0, 1, H)
    layer = _wide_layer(np.repeat(row, E, axis=0), k, bias=np.full(E, 0.125, np.float32),
                        bias_mode="select")
    ids, w, key = M.route(synth.activations(1022, 2, H), layer)
    assert ids.tolist() == [list(range(k))] * 2
    np.testing.assert_allclose(w, 1.0 / k, rtol=0, atol=1e-15)

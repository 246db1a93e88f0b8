"""GPU parity of the router variants against the float64 oracle: the
per-expert bias in the choice only (ROUTER_BIAS_SELECT: key sigmoid(l) + b,
weights from the unbiased sigmoid, as the DeepSeek-V3 report's gate) and a
routed scale on the combine weights, on the decode and prefill paths.

Bars as for the plain router: routing equal up to near-ties within 1e-6 of
the k-th key, weights within 2e-6 (relative to the scale) of the oracle's
for the chosen experts, layer output within the per-token relative L2 bar.
"""

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from oracle import moe as M
from tests._gpu import (Built, check_mxfp8_workspace, check_parity, check_routing, to_np_u16,
                        topk_candidates)

pytestmark = pytest.mark.gpu

RAGGED = dict(hidden=288, inter=96, n_experts=40, top_k=5, n_shared=2)
MANY = dict(hidden=128, inter=32, n_experts=1024, top_k=32, n_shared=0)


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def _built(cfg, seed, bias_scale, routed_scale, bias_mode="select"):
    built = Built(cfg, seed=seed, bias=True, bias_mode=bias_mode, routed_scale=routed_scale)
    if bias_scale != 1.0:  # a bias of the size of the scores' spread, not larger
        hb = (built.dev["host_bias"] * np.float32(bias_scale)).astype(np.float32)
        built.dev["router_bias"].copy_(torch.from_numpy(hb))
        built.oracle.router_bias = hb
    return built


def _layer(b, built, xd, path, ws=None):
    T, k, H = xd.shape[0], built.cfg["top_k"], built.cfg["hidden"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T) if ws is None else ws
    b.moe_layer(built.lib, xd, y, ids, w, ws, path=path)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)


def _check_route(built, xh, ids, w):
    scale = built.routed_scale
    s, key = M.router_scores(xh, built.oracle)
    n_amb = check_routing(ids, w / np.float32(scale), key, built.cfg["top_k"])
    wo = M.combine_weights(s, ids, scale)
    np.testing.assert_allclose(w, wo, rtol=0, atol=2e-6 * scale)
    return wo, n_amb


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED, MANY], ids=["tiny", "ragged", "many"])
@pytest.mark.parametrize("T", [1, 4, 7, 70])
@pytest.mark.parametrize("bias_scale", [1.0, 0.05], ids=["bias", "small-bias"])
def test_select_mode_decode(b, cfg, T, bias_scale):
    built = _built(cfg, 41, bias_scale, 2.5)
    xh, xd = SD.upload_tokens(4100 + T, T, cfg["hidden"])
    ids, w, y = _layer(b, built, xd, b.PATH_GEMV)
    wo, _ = _check_route(built, xh, ids, w)
    check_parity(y, M.moe_forward(xh, built.oracle, ids, wo))


def test_select_mode_choice_differs_from_logits_mode(b):
    # the same device tensors under the two modes: the bias moves the choice
    built = _built(synth.TINY, 42, 1.0, 1.0)
    xh, xd = SD.upload_tokens(4200, 16, 256)
    ids_s, _, _ = _layer(b, built, xd, b.PATH_GEMV)
    built.bias_mode = built.oracle.bias_mode = "logits"
    built.repack()
    ids_l, w_l, _ = _layer(b, built, xd, b.PATH_GEMV)
    _check_route(built, xh, ids_l, w_l)
    assert not np.array_equal(np.sort(ids_s, axis=1), np.sort(ids_l, axis=1))


def test_route_entry_equals_layer_routing(b):
    built = _built(RAGGED, 43, 0.05, 1.7)
    T = 9
    xh, xd = SD.upload_tokens(4300, T, RAGGED["hidden"])
    ids = torch.empty((T, 5), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 5), dtype=torch.float32, device="cuda")
    b.route(built.lib, xd, ids, w, built.lib.workspace(T))
    ids2, w2, _ = _layer(b, built, xd, b.PATH_GEMV)
    assert np.array_equal(ids.cpu().numpy(), ids2)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w2.view(np.uint32))
    _check_route(built, xh, ids2, w2)


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED], ids=["tiny", "ragged"])
@pytest.mark.parametrize("T", [70, 300])
def test_select_mode_prefill(b, cfg, T):
    built = _built(cfg, 44, 0.05, 2.5)
    xh, xd = SD.upload_tokens(4400 + T, T, cfg["hidden"])
    ws = built.lib.workspace(T)
    ids, w, y = _layer(b, built, xd, b.PATH_MFMA, ws=ws)
    wo, _ = _check_route(built, xh, ids, w)
    ref = M.moe_forward(xh, built.oracle, ids, wo, act_mxfp8=True)
    check_parity(y, ref, check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w, built.oracle))


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_routed_scale_two_doubles_output_bitwise(b, path):
    """Scale 2 doubles every weight exactly in fp32, hence every routed
    partial; with no shared experts the bf16 output doubles bit for bit."""
    cfg = dict(hidden=256, inter=64, n_experts=16, top_k=4, n_shared=0)
    p = b.PATH_GEMV if path == "gemv" else b.PATH_MFMA
    xh, xd = SD.upload_tokens(4500, 40, 256)
    one = Built(cfg, seed=45, bias=True)
    two = Built(cfg, seed=45, bias=True, routed_scale=2.0)
    ids1, w1, y1 = _layer(b, one, xd, p)
    ids2, w2, y2 = _layer(b, two, xd, p)
    assert np.array_equal(ids1, ids2)
    np.testing.assert_array_equal(w2, 2.0 * w1)
    y1f = y1.astype(np.uint32) << 16
    y2f = y2.astype(np.uint32) << 16
    np.testing.assert_array_equal(y2f.view(np.float32), 2.0 * y1f.view(np.float32))


def test_select_mode_many_winners_in_one_lane(b):
    """Experts 5, 69, 133, ... (e = 5 mod 64) sit in one lane of the top-k
    wave; +20 on their score-side bias makes all 16 of them winners, so one
    lane holds 16 of the 32 selected experts while contributing a single
    maximum to the threshold: the candidate list (keys sigmoid(l) + b,
    weights re-read from the unbiased logits) must still rank them all.
    The exact path past 256 candidates is covered by
    test_gpu_topk_exact.py."""
    built = _built(MANY, 46, 0.05, 1.5)
    bias = built.oracle.router_bias.copy()
    bias[5::64] += 20.0
    built.dev["router_bias"].copy_(torch.from_numpy(bias))
    built.oracle.router_bias = bias
    xh, xd = SD.upload_tokens(4600, 5, MANY["hidden"])
    _, key = M.router_scores(xh, built.oracle)
    assert all(32 < topk_candidates(key[t], 32) <= 256 for t in range(5))
    ids, w, y = _layer(b, built, xd, b.PATH_GEMV)
    _check_route(built, xh, ids, w)
    for t in range(5):
        assert set(range(5, 1024, 64)) <= set(ids[t].tolist())
        assert np.all(ids[t][:16] % 64 == 5)
    s, _ = M.router_scores(xh, built.oracle)
    check_parity(y, M.moe_forward(xh, built.oracle, ids, M.combine_weights(s, ids, 1.5)))

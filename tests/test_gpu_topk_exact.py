"""The top-k's exact path and the tie rule at the K3 expert count, and the
give-up of the top-k's bounded wait, through the C ABI.

The per-token top-k gathers the experts at or above a threshold (the k-th
largest of the wave's 64 lane maxima) and ranks them; when more than 256
experts reach it -- heavy ties, e.g. identical router rows or sigmoid
scores saturated in fp32 -- it runs k exact rounds of a wave-wide maximum
instead.  These tests make every expert tie (E = 896 and 1024, so 896 or
1024 experts reach the threshold, computed from the oracle's keys) on every
launch structure: one token (top-k inside the router launch, no plan), 2-4
tokens (the same with a plan), more tokens (a top-k launch) and the MFMA
path.  Exact ties go to the lower expert index (the reading of the tiny
configuration's tie rule), so the choice is experts 0..k-1 and each weight
is 1/k.
"""

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from oracle import formats as F
from oracle import moe as M
from tests._gpu import (Built, check_mxfp8_workspace, check_parity, check_routing,
                        oracle_weights, to_np_u16, topk_candidates)

pytestmark = pytest.mark.gpu

WIDE896 = dict(hidden=256, inter=64, n_experts=896, top_k=16, n_shared=1)
WIDE1024 = dict(hidden=256, inter=64, n_experts=1024, top_k=32, n_shared=1)


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def _tied(cfg, seed, **kw):
    """A layer whose router rows are all equal (device and oracle)."""
    built = Built(cfg, seed=seed, **kw)
    wr = built.dev["router_w"]
    wr[:] = wr[3].clone()
    built.oracle.router_w = np.repeat(built.oracle.router_w[3:4], cfg["n_experts"], axis=0)
    return built


def _layer(b, built, xd, path, ws=None):
    T, k, H = xd.shape[0], built.cfg["top_k"], built.cfg["hidden"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T) if ws is None else ws
    b.moe_layer(built.lib, xd, y, ids, w, ws, path=path)
    assert b.workspace_status(ws) == b.MOE_OK
    return ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)


@pytest.mark.parametrize("cfg,T,path", [
    (WIDE896, 1, "gemv"), (WIDE896, 3, "gemv"), (WIDE896, 8, "gemv"), (WIDE896, 40, "mfma"),
    (WIDE1024, 1, "gemv"), (WIDE1024, 70, "gemv"), (WIDE1024, 70, "mfma")],
    ids=["896-1", "896-3", "896-8", "896-40-mfma", "1024-1", "1024-70", "1024-70-mfma"])
def test_all_tied_rows_take_the_exact_path(b, cfg, T, path):
    E, k = cfg["n_experts"], cfg["top_k"]
    built = _tied(cfg, seed=60)
    xh, xd = SD.upload_tokens(6000 + T, T, cfg["hidden"])
    _, _, s = M.route(xh, built.oracle)
    for t in range(T):
        assert topk_candidates(s[t], k) == E > 256   # every key reaches the threshold
    p = b.PATH_MFMA if path == "mfma" else b.PATH_GEMV
    ws = built.lib.workspace(T)
    ids, w, y = _layer(b, built, xd, p, ws)
    assert ids.tolist() == [list(range(k))] * T
    np.testing.assert_allclose(w, 1.0 / k, rtol=0, atol=1e-7)
    check_routing(ids, w, s, k)
    wo = oracle_weights(s, ids)
    if path == "mfma":
        ref = M.moe_forward(xh, built.oracle, ids, wo, act_mxfp8=True)
        check_parity(y, ref, check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w, built.oracle))
    else:
        check_parity(y, M.moe_forward(xh, built.oracle, ids, wo))


@pytest.mark.parametrize("T", [1, 8])
def test_select_mode_all_tied_keys(b, T):
    """Choice on sigmoid(l) + bias with every row and every bias equal."""
    built = _tied(WIDE896, seed=61, bias=True, bias_mode="select")
    bias = np.full(896, 0.375, np.float32)
    built.dev["router_bias"].copy_(torch.from_numpy(bias))
    built.oracle.router_bias = bias
    built.repack()
    xh, xd = SD.upload_tokens(6100 + T, T, 256)
    s, key = M.router_scores(xh, built.oracle)
    assert all(topk_candidates(key[t], 16) == 896 for t in range(T))
    ids, w, y = _layer(b, built, xd, b.PATH_GEMV)
    assert ids.tolist() == [list(range(16))] * T
    np.testing.assert_allclose(w, 1.0 / 16, rtol=0, atol=1e-7)
    check_parity(y, M.moe_forward(xh, built.oracle, ids, M.combine_weights(s, ids)))


@pytest.mark.parametrize("T", [1, 8])
def test_select_mode_saturated_scores_tie_in_fp32(b, T):
    """Distinct router rows, but logits of 30 or more: every sigmoid score is
    1.0 in fp32, so with a zero bias all 896 keys tie in the kernel's
    precision and the exact path picks experts 0..15.  In float64 the
    scores differ by less than 1e-12, inside the 1e-6 tie exclusion, so
    the oracle's routing admits that choice."""
    built = Built(WIDE896, seed=62, bias=True, bias_mode="select")
    zero = np.zeros(896, np.float32)
    built.dev["router_bias"].copy_(torch.from_numpy(zero))
    built.oracle.router_bias = zero
    col = synth.to_bf16_bits(np.linspace(0.03, 0.05, 896, dtype=np.float32))
    built.dev["router_w"][:, 0] = torch.from_numpy(col.view(np.int16)).cuda()
    built.oracle.router_w = built.oracle.router_w.copy()
    built.oracle.router_w[:, 0] = col
    built.repack()
    xh = synth.activations(6200 + T, T, 256)
    xh[:, 0] = 0x4480  # bf16 1024.0
    xd = torch.from_numpy(xh.view(np.int16)).cuda()
    s, key = M.router_scores(xh, built.oracle)
    logits = M.router_logits(xh, built.oracle.router_w)
    assert logits.min() > 29.0
    s32 = (np.float32(1) / (np.float32(1) + np.exp(-logits.astype(np.float32)))).astype(np.float32)
    assert (s32 == 1.0).all()
    assert all(topk_candidates(s32[t], 16) == 896 for t in range(T))
    ids, w, y = _layer(b, built, xd, b.PATH_GEMV)
    assert ids.tolist() == [list(range(16))] * T
    np.testing.assert_allclose(w, 1.0 / 16, rtol=0, atol=1e-7)
    check_routing(ids, w, key, 16)
    check_parity(y, M.moe_forward(xh, built.oracle, ids, M.combine_weights(s, ids)))


@pytest.mark.parametrize("T", [1, 3, 8])
def test_wait_give_up_is_reported(b, T):
    """With a wait limit of 0 the top-k workgroup of the router launch gives
    up at once (every kernel still runs to its end); the call's workspace
    then reports MOE_ETIMEOUT once, and calls under the default limit
    report MOE_OK and match the oracle again."""
    built = Built(synth.TINY, seed=63)
    ws = torch.zeros(built.lib.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, 4), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 4), dtype=torch.float32, device="cuda")
    y = torch.empty((T, 256), dtype=torch.int16, device="cuda")
    xh, xd = SD.upload_tokens(6300 + T, T, 256)
    b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_GEMV)
    assert b.workspace_status(ws) == b.MOE_OK
    try:
        b.set_wait_limit(0)
        b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_GEMV)
        torch.cuda.synchronize()
        assert b.workspace_status(ws) == b.MOE_ETIMEOUT
        assert b.workspace_status(ws) == b.MOE_OK       # reported once
        # a call structure without the in-launch wait (more than 8 tokens:
        # the top-k has a launch of its own) is unaffected
        x9h, x9d = SD.upload_tokens(6310, 9, 256)
        ws9 = built.lib.workspace(9)
        i9 = torch.empty((9, 4), dtype=torch.int32, device="cuda")
        w9 = torch.empty((9, 4), dtype=torch.float32, device="cuda")
        y9 = torch.empty((9, 256), dtype=torch.int16, device="cuda")
        b.moe_layer(built.lib, x9d, y9, i9, w9, ws9, path=b.PATH_GEMV)
        assert b.workspace_status(ws9) == b.MOE_OK
    finally:
        b.set_wait_limit(-1)
    b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_GEMV)
    assert b.workspace_status(ws) == b.MOE_OK
    ids_np = ids.cpu().numpy()
    _, _, s = M.route(xh, built.oracle)
    check_routing(ids_np, w.cpu().numpy(), s, 4)
    check_parity(to_np_u16(y), M.moe_forward(xh, built.oracle, ids_np, oracle_weights(s, ids_np)))

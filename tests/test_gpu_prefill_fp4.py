"""GPU parity of the prefill path with MXFP4 activations (MOE_PATH_MFMA_FP4):
routed experts on the block-scaled FP4 x FP4 matrix cores, x and h rounded
to MXFP4 (E2M1 codes, one E8M0 exponent per 32 along the contraction).

Reference: the float64 oracle in its MXFP4-activation mode, under the same
routing.  The layer's MXFP4 x codes (read from its workspace) must equal the
oracle's bit for bit; every h code equals the oracle's or lies within the
rigorous fp32 bound of a rounding boundary (tests/_gpu.py
check_mxfp8_workspace with fmt "e2m1"); the output is compared with the
oracle's plus the exact effect of the differing codes, at the per-token
relative L2 bar and the element-wise bound.
"""

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from oracle import moe as M
from tests._gpu import (Built, check_mxfp8_workspace, check_parity, check_routing,
                        oracle_weights, to_np_u16)

pytestmark = pytest.mark.gpu

RAGGED = dict(hidden=288, inter=96, n_experts=40, top_k=5, n_shared=2)
WIDE = dict(hidden=8192, inter=64, n_experts=24, top_k=3, n_shared=1)
MANY = dict(hidden=128, inter=32, n_experts=1024, top_k=32, n_shared=0)
MID = dict(hidden=1024, inter=512, n_experts=16, top_k=4, n_shared=1)
ALL = dict(hidden=256, inter=128, n_experts=8, top_k=8, n_shared=1)


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def _forward(b, built, x_dev, ids_np, w_np, residual=None):
    T = x_dev.shape[0]
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    w = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).cuda()
    y = torch.empty((T, built.cfg["hidden"]), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.forward(built.lib, x_dev, ids, w, y, ws, residual=residual, path=b.PATH_MFMA_FP4)
    torch.cuda.synchronize()
    return to_np_u16(y), ws


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED, WIDE, MANY, MID, ALL],
                         ids=["tiny", "ragged", "wide", "many", "mid", "all"])
@pytest.mark.parametrize("T", [1, 7, 70, 200])
def test_fp4_forward_matches_oracle(b, cfg, T):
    built = Built(cfg, seed=81)
    xh, xd = SD.upload_tokens(8100 + T, T, cfg["hidden"])
    ids, w, _ = M.route(xh, built.oracle)
    w32 = w.astype(np.float32)
    y, ws = _forward(b, built, xd, ids, w32)
    ref = M.moe_forward(xh, built.oracle, ids, w32.astype(np.float64), act_mxfp4=True)
    eff = check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w32, built.oracle, fmt="e2m1")
    check_parity(y, ref, eff)


def test_fp4_skewed_routing_many_tiles_per_expert(b):
    # every token picks experts 0..3: 300 pairs per expert, four 96-token tiles each (the last ragged)
    built = Built(MID, seed=82)
    T = 300
    xh, xd = SD.upload_tokens(8200, T, MID["hidden"])
    ids = np.tile(np.arange(4, dtype=np.int32), (T, 1))
    w = np.random.default_rng(8).random((T, 4)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    y, ws = _forward(b, built, xd, ids, w)
    ref = M.moe_forward(xh, built.oracle, ids, w.astype(np.float64), act_mxfp4=True)
    check_parity(y, ref, check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w, built.oracle,
                                               fmt="e2m1"))


def test_fp4_layer_entry_with_residual_and_bias(b):
    built = Built(RAGGED, seed=83, bias=True)
    T = 90
    xh, xd = SD.upload_tokens(8300, T, RAGGED["hidden"])
    rh, rd = SD.upload_tokens(8301, T, RAGGED["hidden"])
    ids = torch.empty((T, 5), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 5), dtype=torch.float32, device="cuda")
    y = torch.empty((T, RAGGED["hidden"]), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.moe_layer(built.lib, xd, y, ids, w, ws, residual=rd, path=b.PATH_MFMA_FP4)
    torch.cuda.synchronize()
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    _, _, s = M.route(xh, built.oracle)
    check_routing(ids_np, w_np, s, 5)
    ref = M.moe_forward(xh, built.oracle, ids_np, oracle_weights(s, ids_np), act_mxfp4=True,
                        residual_bits=rh)
    check_parity(to_np_u16(y), ref,
                 check_mxfp8_workspace(b, built.lib, ws, T, xh, ids_np, w_np, built.oracle,
                                       fmt="e2m1"))


def test_fp4_and_fp8_paths_differ_by_the_activation_rounding(b):
    """The two MX paths run the same weights and routing; the MXFP4 one is
    further from the exact layer than the MXFP8 one, as its coarser grid
    implies (relative L2 per token: E2M1 rounding ~1e-1, E4M3 ~1e-2)."""
    built = Built(MID, seed=84)
    T = 40
    xh, xd = SD.upload_tokens(8400, T, MID["hidden"])
    ids, w, _ = M.route(xh, built.oracle)
    w32 = w.astype(np.float32)
    exact = M.moe_forward(xh, built.oracle, ids, w32.astype(np.float64))
    y4, _ = _forward(b, built, xd, ids, w32)
    idt = torch.from_numpy(ids.astype(np.int32)).cuda()
    wt = torch.from_numpy(w32).cuda()
    y8 = torch.empty((T, MID["hidden"]), dtype=torch.int16, device="cuda")
    b.forward(built.lib, xd, idt, wt, y8, built.lib.workspace(T), path=b.PATH_MFMA)
    torch.cuda.synchronize()
    from tests._gpu import rel_l2_per_token
    e4 = rel_l2_per_token(y4, exact)
    e8 = rel_l2_per_token(to_np_u16(y8), exact)
    assert (e4 > e8).all() and e4.max() < 0.5 and e8.max() < 0.1

"""GPU parity of the prefill (MFMA) path: routed experts on the block-scaled
FP4 x FP8 matrix cores, x and h quantised to MXFP8 along the contraction.

Reference: the float64 oracle with its MXFP8 activation reading (x and h
replaced by their MXFP8 values, Deltafin explainer section 2.1), under the
same routing.  The layer's MXFP8 codes of x (read from its workspace) must
equal the oracle's bit for bit.  The GPU quantises its fp32 h where the
oracle quantises float64 h, so an h code may differ where a fp32
evaluation's error bound reaches an E4M3 rounding midpoint (or a block
maximum a power of two); every h code is checked element by element
against that bound, and the output is compared with the oracle's plus the
exact effect of the codes that differ, at the per-token relative L2 bar
and the element-wise bound.
"""

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from oracle import moe as M

from tests._gpu import (Built, check_mxfp8_workspace, check_parity, check_routing,
                        oracle_weights, rel_l2_per_token, to_np_u16)

pytestmark = pytest.mark.gpu

RAGGED = dict(hidden=288, inter=96, n_experts=40, top_k=5, n_shared=2)
WIDE = dict(hidden=8192, inter=64, n_experts=24, top_k=3, n_shared=1)
MANY = dict(hidden=128, inter=32, n_experts=1024, top_k=32, n_shared=0)
MID = dict(hidden=1024, inter=512, n_experts=16, top_k=4, n_shared=1)
ALL = dict(hidden=256, inter=128, n_experts=8, top_k=8, n_shared=1)  # k = E


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
    b.forward(built.lib, x_dev, ids, w, y, ws, residual=residual, path=b.PATH_MFMA)
    torch.cuda.synchronize()
    return to_np_u16(y), ws


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED, WIDE, MANY, MID, ALL],
                         ids=["tiny", "ragged", "wide", "many", "mid", "all"])
@pytest.mark.parametrize("T", [1, 7, 70, 200])
def test_mfma_forward_matches_oracle_mxfp8(b, cfg, T):
    built = Built(cfg, seed=21)
    xh, xd = SD.upload_tokens(1400 + T, T, cfg["hidden"])
    ids, w, _ = M.route(xh, built.oracle)
    w32 = w.astype(np.float32)
    y, ws = _forward(b, built, xd, ids, w32)
    ref = M.moe_forward(xh, built.oracle, ids, w32.astype(np.float64), act_mxfp8=True)
    eff = check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w32, built.oracle)
    check_parity(y, ref, eff)


def test_mfma_skewed_routing_many_tiles_per_expert(b):
    # every token picks experts 0..3: 300 pairs per expert, four 96-token
    # tiles each (the last ragged)
    built = Built(MID, seed=22)
    T = 300
    xh, xd = SD.upload_tokens(1450, T, MID["hidden"])
    ids = np.tile(np.arange(4, dtype=np.int32), (T, 1))
    rng = np.random.default_rng(5)
    w = rng.random((T, 4)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    y, ws = _forward(b, built, xd, ids, w)
    ref = M.moe_forward(xh, built.oracle, ids, w.astype(np.float64), act_mxfp8=True)
    check_parity(y, ref, check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w, built.oracle))


@pytest.mark.parametrize("fp4", [False, True], ids=["mxfp8", "mxfp4"])
def test_mfma_token_tile_boundaries(b, fp4):
    """Experts with 1, 15, 16, 17, 95, 96, 97, 192 and 193 pairs: tiles of
    one to six 16-token groups, a tile exactly full, one pair past a full
    tile, two full tiles and one past them (plan tiles of 96 pairs)."""
    built = Built(MID, seed=26)
    counts = [1, 15, 16, 17, 95, 96, 97, 192, 193]
    k = MID["top_k"]
    # 204 tokens x 4 slots = 816 pairs; expert e < 9 gets counts[e] of them,
    # the rest go to experts 9..15, each token's slots distinct
    T = 204
    pool = np.concatenate([np.full(c, e) for e, c in enumerate(counts)])
    rest = T * k - pool.size
    pool = np.concatenate([pool, 9 + np.arange(rest) % 7])
    # slot j of token t takes pair j T + t of the expert-sorted list: no
    # expert has more than T pairs, so a token's slots are distinct
    ids = np.ascontiguousarray(pool.reshape(k, T).T, dtype=np.int32)
    rng = np.random.default_rng(8)
    assert all(len(set(r)) == k for r in ids)
    got = np.bincount(ids.ravel(), minlength=MID["n_experts"])
    assert list(got[:9]) == counts
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    xh, xd = SD.upload_tokens(1470 + fp4, T, MID["hidden"])
    idt = torch.from_numpy(ids).cuda()
    wt = torch.from_numpy(w).cuda()
    y = torch.empty((T, MID["hidden"]), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.forward(built.lib, xd, idt, wt, y, ws, path=b.PATH_MFMA_FP4 if fp4 else b.PATH_MFMA)
    torch.cuda.synchronize()
    ref = M.moe_forward(xh, built.oracle, ids, w.astype(np.float64), act_mxfp8=not fp4,
                        act_mxfp4=fp4)
    eff = check_mxfp8_workspace(b, built.lib, ws, T, xh, ids, w, built.oracle,
                                fmt="e2m1" if fp4 else "e4m3")
    check_parity(to_np_u16(y), ref, eff)


def test_mfma_residual_and_layer_entry(b):
    built = Built(RAGGED, seed=23, bias=True)
    T = 90
    xh, xd = SD.upload_tokens(1460, T, RAGGED["hidden"])
    rh, rd = SD.upload_tokens(1461, T, RAGGED["hidden"])
    ids = torch.empty((T, 5), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 5), dtype=torch.float32, device="cuda")
    y = torch.empty((T, RAGGED["hidden"]), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.moe_layer(built.lib, xd, y, ids, w, ws, residual=rd, path=b.PATH_MFMA)
    torch.cuda.synchronize()
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    _, _, s = M.route(xh, built.oracle)
    check_routing(ids_np, w_np, s, 5)
    wref = oracle_weights(s, ids_np)
    ref = M.moe_forward(xh, built.oracle, ids_np, wref, act_mxfp8=True, residual_bits=rh)
    check_parity(to_np_u16(y), ref,
                 check_mxfp8_workspace(b, built.lib, ws, T, xh, ids_np, w_np, built.oracle))


@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_layer_at_the_token_limit(b, path):
    # 65,536 tokens, the most one call takes (about 85 96-token tiles per
    # expert at the tiny shape), on either path; routing and output checked
    # on a sample of tokens spread over the batch, the first and last included
    cfg = synth.TINY
    built = Built(cfg, seed=25, bias=True)
    T = 1 << 16
    xh, xd = SD.upload_tokens(1480, T, cfg["hidden"])
    k = cfg["top_k"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, cfg["hidden"]), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_MFMA if path == "mfma" else b.PATH_GEMV)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([np.arange(0, T, 251), [T - 1]]))
    ids_all, w_all = ids.cpu().numpy(), w.cpu().numpy()
    ids_np, w_np = ids_all[sample], w_all[sample]
    xs = np.ascontiguousarray(xh[sample])
    _, _, s = M.route(xs, built.oracle)
    check_routing(ids_np, w_np, s, k)
    wref = oracle_weights(s, ids_np)
    if path == "mfma":
        ref = M.moe_forward(xs, built.oracle, ids_np, wref, act_mxfp8=True)
        # h codes of every pair of the sampled tokens' experts (all 32)
        eff = check_mxfp8_workspace(b, built.lib, ws, T, xh, ids_all, w_all, built.oracle,
                                    tokens=sample, x_rows=sample)
        check_parity(to_np_u16(y)[sample], ref, eff)
    else:
        check_parity(to_np_u16(y)[sample], M.moe_forward(xs, built.oracle, ids_np, wref))


def test_mfma_and_gemv_paths_agree_closely(b):
    # the two paths differ only by the MXFP8 rounding of x and h
    built = Built(MID, seed=24)
    T = 40
    xh, xd = SD.upload_tokens(1470, T, MID["hidden"])
    ids, w, _ = M.route(xh, built.oracle)
    w32 = w.astype(np.float32)
    y_mx, _ = _forward(b, built, xd, ids, w32)
    ref_exact = M.moe_forward(xh, built.oracle, ids, w32.astype(np.float64))
    err = rel_l2_per_token(y_mx, ref_exact)
    assert err.max() < 0.1  # MXFP8 activations: a few percent from the exact layer


def test_auto_path_threshold(b):
    assert b.mfma_min_tokens() >= 1

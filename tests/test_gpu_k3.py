"""GPU parity at the full K3 layer shape (hidden 7168, 896 experts of
intermediate 1536, top-16, 2 shared experts): batch 1, batched decode of 64
tokens, and 8 tokens with a residual, in the launch configuration the
benchmark times.  The oracle checks sampled tokens one by one; routing is
checked for every token.
"""

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from oracle import moe as M
from oracle import record as R
from tests._gpu import REL_TOL, Built, check_routing, oracle_weights, rel_l2_per_token, to_np_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


@pytest.fixture(scope="module")
def k3():
    print("building K3 layer (15.7 GB of expert records)", flush=True)
    return Built(synth.K3, seed=0)


def _run(b, built, xd, residual=None):
    T = xd.shape[0]
    ids = torch.empty((T, 16), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 16), dtype=torch.float32, device="cuda")
    y = torch.empty((T, 7168), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.moe_layer(built.lib, xd, y, ids, w, ws, residual=residual, path=b.PATH_GEMV)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)


def test_k3_dequant_sampled_experts_bit_exact(b, k3):
    for e in (0, 517, 895):
        rec = k3.oracle.expert_record(e)
        for m in (R.GATE, R.UP, R.DOWN):
            shape = (7168, 1536) if m == R.DOWN else (1536, 7168)
            out = torch.empty(shape, dtype=torch.float32, device="cuda")
            b.dequant_export(k3.lib, e, m, out)
            torch.cuda.synchronize()
            ref = R.dequant_matrix(rec, 7168, 1536, m).astype(np.float32)
            np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("seed", [1000, 1001, 1002])
def test_k3_decode_batch1(b, k3, seed):
    xh, xd = SD.upload_tokens(seed, 1, 7168)
    ids, w, y = _run(b, k3, xd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    ref = M.moe_forward(xh, k3.oracle, ids, oracle_weights(s, ids))
    err = rel_l2_per_token(y, ref)
    print(f"K3 b=1 seed {seed}: rel L2 {err.max():.3e}")
    assert err.max() <= REL_TOL


def test_k3_batched_decode_64(b, k3):
    xh, xd = SD.upload_tokens(2000, 64, 7168)
    ids, w, y = _run(b, k3, xd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    distinct = len(np.unique(ids))
    print(f"K3 b=64: {distinct} distinct experts")
    assert 500 < distinct < 700
    sample = [0, 21, 42, 63]
    ref = M.moe_forward(xh, k3.oracle, ids, oracle_weights(s, ids), tokens=sample)
    err = rel_l2_per_token(y[sample], ref)
    print(f"K3 b=64 sampled rel L2 {err.max():.3e}")
    assert err.max() <= REL_TOL


def test_k3_eight_tokens_with_residual(b, k3):
    xh, xd = SD.upload_tokens(3000, 8, 7168)
    rh, rd = SD.upload_tokens(3001, 8, 7168)
    ids, w, y = _run(b, k3, xd, residual=rd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    sample = [1, 6]
    ref = M.moe_forward(xh, k3.oracle, ids, oracle_weights(s, ids), residual_bits=rh,
                        tokens=sample)
    assert rel_l2_per_token(y[sample], ref).max() <= REL_TOL


@pytest.mark.parametrize("top_k,T", [(8, 1), (8, 8), (4, 64)])
def test_k3_reduced_top_k(b, k3, top_k, T):
    """The pages' experimental switch that lowers the number of routed experts
    per token (K3_MOE_TOP_K): the same K3 weights with top-8 and top-4, on the
    launch paths of 1, 8 and 64 tokens."""
    lay = b.Layer(7168, 1536, 896, top_k, k3.lib.router_w, k3.lib.experts, k3.lib.shared_gate,
                  k3.lib.shared_up, k3.lib.shared_down)
    orc = M.Layer(7168, 1536, 896, top_k, k3.oracle.router_w, k3.oracle.expert_record,
                  shared=k3.oracle.shared)
    xh, xd = SD.upload_tokens(5000 + T, T, 7168)
    ids = torch.empty((T, top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, 7168), dtype=torch.int16, device="cuda")
    b.moe_layer(lay, xd, y, ids, w, lay.workspace(T), path=b.PATH_GEMV)
    torch.cuda.synchronize()
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)
    _, _, s = M.route(xh, orc)
    check_routing(ids, w, s, top_k)
    sample = sorted({0, T // 2, T - 1})
    ref = M.moe_forward(xh, orc, ids, oracle_weights(s, ids), tokens=sample)
    err = rel_l2_per_token(y[sample], ref)
    print(f"K3 top-{top_k} T={T}: rel L2 {err.max():.3e}")
    assert err.max() <= REL_TOL


def test_k3_prefill_4096_with_bias(b, k3):
    """K3 prefill (4096 tokens, per-expert logit bias N(0, 0.5)) on the MFMA
    path: routing for every token, output on sampled tokens against the
    oracle in its MXFP8-activation mode."""
    from synth import router_bias
    bias_h = router_bias(0, 0, 896)
    lay = b.Layer(7168, 1536, 896, 16, k3.lib.router_w, k3.lib.experts, k3.lib.shared_gate,
                  k3.lib.shared_up, k3.lib.shared_down, router_bias=torch.from_numpy(bias_h).cuda())
    orc = M.Layer(7168, 1536, 896, 16, k3.oracle.router_w, k3.oracle.expert_record,
                  shared=k3.oracle.shared, router_bias=bias_h)
    T = 4096
    xh, xd = SD.upload_tokens(4000, T, 7168)
    ids = torch.empty((T, 16), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 16), dtype=torch.float32, device="cuda")
    y = torch.empty((T, 7168), dtype=torch.int16, device="cuda")
    b.moe_layer(lay, xd, y, ids, w, lay.workspace(T), path=b.PATH_MFMA)
    torch.cuda.synchronize()
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)
    _, _, s = M.route(xh, orc)
    n_amb = check_routing(ids, w, s, 16)
    per_expert = np.bincount(ids.ravel(), minlength=896)
    print(f"K3 prefill: {n_amb} near-tie tokens; pairs per expert min {per_expert.min()} "
          f"median {int(np.median(per_expert))} max {per_expert.max()}")
    assert per_expert.sum() == T * 16 and (per_expert > 0).all()
    sample = [0, 1777, 4095]
    ref = M.moe_forward(xh, orc, ids, oracle_weights(s, ids), act_mxfp8=True, tokens=sample)
    err = rel_l2_per_token(y[sample], ref)
    print(f"K3 prefill sampled rel L2 {err.max():.3e}")
    assert err.max() <= REL_TOL


@pytest.mark.parametrize("T", [1, 64])
def test_k3_router_bias_in_choice_only_with_routed_scale(b, k3, T):
    """K3 decode with the bias in the choice only (key sigmoid(l) + b, b of
    N(0, 0.025)) and a routed scale of 2.5."""
    from synth import router_bias
    bias_h = (router_bias(0, 0, 896) * np.float32(0.05)).astype(np.float32)
    lay = b.Layer(7168, 1536, 896, 16, k3.lib.router_w, k3.lib.experts, k3.lib.shared_gate,
                  k3.lib.shared_up, k3.lib.shared_down, router_bias=torch.from_numpy(bias_h).cuda(),
                  router_mode=b.ROUTER_BIAS_SELECT, routed_scale=2.5)
    orc = M.Layer(7168, 1536, 896, 16, k3.oracle.router_w, k3.oracle.expert_record,
                  shared=k3.oracle.shared, router_bias=bias_h, bias_mode="select",
                  routed_scale=2.5)
    xh, xd = SD.upload_tokens(5100 + T, T, 7168)
    ids = torch.empty((T, 16), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 16), dtype=torch.float32, device="cuda")
    y = torch.empty((T, 7168), dtype=torch.int16, device="cuda")
    b.moe_layer(lay, xd, y, ids, w, lay.workspace(T), path=b.PATH_GEMV)
    torch.cuda.synchronize()
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)
    s, key = M.router_scores(xh, orc)
    check_routing(ids, w / np.float32(2.5), key, 16)
    wo = M.combine_weights(s, ids, 2.5)
    np.testing.assert_allclose(w, wo, rtol=0, atol=5e-6)
    sample = sorted({0, T - 1})
    err = rel_l2_per_token(y[sample], M.moe_forward(xh, orc, ids, wo, tokens=sample))
    print(f"K3 select-mode bias, scale 2.5, T={T}: rel L2 {err.max():.3e}")
    assert err.max() <= REL_TOL


def test_k3_decode_batch2_speculative_verify(b, k3):
    """T = 2, the shape a speculative step verifies (the current token and
    one drafted token), in the launch configuration the benchmark times."""
    xh, xd = SD.upload_tokens(5200, 2, 7168)
    ids, w, y = _run(b, k3, xd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    ref = M.moe_forward(xh, k3.oracle, ids, oracle_weights(s, ids))
    err = rel_l2_per_token(y, ref)
    print(f"K3 T=2: rel L2 {err}")
    assert err.max() <= REL_TOL


def test_k3_pooled_experts_equal_resident(b, k3):
    """The 896 K3 records in pinned host memory, 64 HBM slots filled on
    demand: consecutive single tokens (new experts each time, some slots
    evicted) give the resident layer's output bit for bit."""
    host = torch.empty(k3.lib.experts.shape, dtype=torch.uint8, pin_memory=True)
    host.copy_(k3.lib.experts)
    pool = b.ExpertPool(host, 64)
    lay = b.Layer(7168, 1536, 896, 16, k3.lib.router_w, pool.slots, k3.lib.shared_gate,
                  k3.lib.shared_up, k3.lib.shared_down, pool=pool)
    copied = 0
    for i in range(6):
        xh, xd = SD.upload_tokens(5300 + i, 1, 7168)
        ids = torch.empty((1, 16), dtype=torch.int32, device="cuda")
        w = torch.empty((1, 16), dtype=torch.float32, device="cuda")
        b.route(k3.lib, xd, ids, w, k3.lib.workspace(1))
        copied += pool.fetch(ids.cpu().numpy())
        ys = []
        for layer in (lay, k3.lib):
            y = torch.empty((1, 7168), dtype=torch.int16, device="cuda")
            b.forward(layer, xd, ids, w, y, layer.workspace(1), path=b.PATH_GEMV)
            torch.cuda.synchronize()
            ys.append(to_np_u16(y))
        np.testing.assert_array_equal(ys[0], ys[1])
    assert copied > 64  # the pool evicted and refilled
    del lay, pool, host

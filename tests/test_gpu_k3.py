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
from tests._gpu import (Built, check_mxfp8_workspace, check_parity, check_routing, oracle_rows,
                        oracle_weights, to_np_u16)

pytestmark = pytest.mark.gpu

PLAN_TILE = 96  # pairs of one expert per prefill token tile (the plan's tiles)


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
    ref = oracle_rows(xh, k3.oracle, ids, oracle_weights(s, ids), [0])
    err = check_parity(y, ref, strict=True)
    print(f"K3 b=1 seed {seed}: rel L2 {err.max():.3e}")


def test_k3_batched_decode_64(b, k3):
    xh, xd = SD.upload_tokens(2000, 64, 7168)
    ids, w, y = _run(b, k3, xd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    distinct = len(np.unique(ids))
    print(f"K3 b=64: {distinct} distinct experts")
    assert 500 < distinct < 700
    # tokens of the experts that 4 or more tokens share, plus a spread
    cnt = np.bincount(ids.ravel(), minlength=896)
    busy = np.nonzero(np.isin(ids, np.nonzero(cnt >= 4)[0]).any(axis=1))[0]
    sample = sorted(set([0, 21, 42, 63]) | set(busy[:12].tolist()))
    ref = oracle_rows(xh, k3.oracle, ids, oracle_weights(s, ids), sample)
    err = check_parity(y[sample], ref, strict=True)
    print(f"K3 b=64 {len(sample)} sampled tokens rel L2 {err.max():.3e}")


def test_k3_eight_tokens_with_residual(b, k3):
    xh, xd = SD.upload_tokens(3000, 8, 7168)
    rh, rd = SD.upload_tokens(3001, 8, 7168)
    ids, w, y = _run(b, k3, xd, residual=rd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    sample = list(range(8))
    ref = oracle_rows(xh, k3.oracle, ids, oracle_weights(s, ids), sample, residual_bits=rh)
    check_parity(y[sample], ref, strict=True)


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
    ref = oracle_rows(xh, orc, ids, oracle_weights(s, ids), sample)
    err = check_parity(y[sample], ref, strict=True)
    print(f"K3 top-{top_k} T={T}: rel L2 {err.max():.3e}")


def test_k3_prefill_4096_with_bias(b, k3):
    """K3 prefill (4096 tokens, per-expert logit bias N(0, 0.5)) on the MFMA
    path: routing for every token; the layer's MXFP8 x codes bit-exact on
    512 tokens; its h codes element by element for every pair of every
    expert the sampled tokens use; and the output of 32 or more
    tokens against the oracle in its MXFP8-activation mode -- every token of
    the most loaded expert's last (ragged) 96-token tile, every token of
    the least loaded expert and of one with about 3 pairs, the first and
    last token, and a spread."""
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
    ws = lay.workspace(T)
    b.moe_layer(lay, xd, y, ids, w, ws, path=b.PATH_MFMA)
    torch.cuda.synchronize()
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)
    _, _, s = M.route(xh, orc)
    n_amb = check_routing(ids, w, s, 16)
    per_expert = np.bincount(ids.ravel(), minlength=896)
    print(f"K3 prefill: {n_amb} near-tie tokens; pairs per expert min {per_expert.min()} "
          f"median {int(np.median(per_expert))} max {per_expert.max()}")
    assert per_expert.sum() == T * 16 and (per_expert > 0).all()
    busiest, idlest = int(per_expert.argmax()), int(per_expert.argmin())
    few = int(np.argmin(np.abs(per_expert - 3)))  # an expert with (about) 3 pairs
    assert per_expert[busiest] % PLAN_TILE != 0 and per_expert[few] <= 4
    # the busiest expert's last tile: its last pairs in the plan's order
    pairs = b.workspace_region(lay, T, b.WS_PAIRS, ws).cpu().numpy().view(np.int32)
    grp = pairs[ids.reshape(-1)[pairs] == busiest]
    last_tile = grp[(len(grp) - 1) // PLAN_TILE * PLAN_TILE:] // 16
    small = np.nonzero(np.isin(ids, [idlest, few]).any(axis=1))[0]
    rng = np.random.default_rng(4)
    sample = set(last_tile.tolist()) | set(small.tolist()) | {0, T - 1}
    sample |= set(rng.choice(T, 6, replace=False).tolist())
    while len(sample) < 32:
        sample.add(int(rng.integers(T)))
    sample = sorted(sample)
    # h codes of every pair of every expert the sampled tokens use (the
    # busiest, idlest and 3-pair experts among them), and the exact effect of
    # the legitimately different codes on the sampled tokens
    eff = check_mxfp8_workspace(b, lay, ws, T, xh, ids, w, orc, tokens=sample,
                                x_rows=np.sort(rng.choice(T, 512, replace=False)))
    ref = oracle_rows(xh, orc, ids, oracle_weights(s, ids), sample, act_mxfp8=True)
    err = check_parity(y[sample], ref, eff, strict=True)
    moved = np.linalg.norm(eff, axis=1) / np.linalg.norm(ref, axis=1)
    print(f"K3 prefill: h-code flips move {np.count_nonzero(moved)} of {len(sample)} sampled "
          f"tokens, by at most {moved.max():.2e} relative")
    print(f"K3 prefill {len(sample)} sampled tokens (busiest expert {busiest}: "
          f"{per_expert[busiest]} pairs, last tile {len(last_tile)}; idlest {idlest}: "
          f"{per_expert[idlest]}; {few}: {per_expert[few]}): rel L2 max {err.max():.3e}")


def test_k3_prefill_4096_mxfp4_activations(b, k3):
    """K3 prefill (4096 tokens, logit bias) on the FP4 x FP4 path
    (MOE_PATH_MFMA_FP4): routing for every token, MXFP4 x codes bit-exact on
    256 tokens, h codes of every pair of every expert the sampled tokens use,
    and the output of 32 tokens (the busiest expert's last tile first)
    against the oracle in its MXFP4-activation mode."""
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
    ws = lay.workspace(T)
    b.moe_layer(lay, xd, y, ids, w, ws, path=b.PATH_MFMA_FP4)
    torch.cuda.synchronize()
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)
    _, _, s = M.route(xh, orc)
    check_routing(ids, w, s, 16)
    per_expert = np.bincount(ids.ravel(), minlength=896)
    busiest = int(per_expert.argmax())
    pairs = b.workspace_region(lay, T, b.WS_PAIRS, ws).cpu().numpy().view(np.int32)
    grp = pairs[ids.reshape(-1)[pairs] == busiest]
    rng = np.random.default_rng(5)
    sample = set((grp[(len(grp) - 1) // 64 * 64:] // 16)[:24].tolist()) | {0, T - 1}
    while len(sample) < 32:
        sample.add(int(rng.integers(T)))
    sample = sorted(sample)
    eff = check_mxfp8_workspace(b, lay, ws, T, xh, ids, w, orc, tokens=sample, fmt="e2m1",
                                x_rows=np.sort(rng.choice(T, 256, replace=False)))
    ref = oracle_rows(xh, orc, ids, oracle_weights(s, ids), sample, act_mxfp4=True)
    err = check_parity(y[sample], ref, eff, strict=True)
    print(f"K3 prefill MXFP4 activations, {len(sample)} sampled tokens: rel L2 max {err.max():.3e}")


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
    err = check_parity(y[sample], oracle_rows(xh, orc, ids, wo, sample), strict=True)
    print(f"K3 select-mode bias, scale 2.5, T={T}: rel L2 {err.max():.3e}")


def test_k3_decode_batch2_speculative_verify(b, k3):
    """T = 2, the shape a speculative step verifies (the current token and
    one drafted token), in the launch configuration the benchmark times."""
    xh, xd = SD.upload_tokens(5200, 2, 7168)
    ids, w, y = _run(b, k3, xd)
    _, _, s = M.route(xh, k3.oracle)
    check_routing(ids, w, s, 16)
    ref = oracle_rows(xh, k3.oracle, ids, oracle_weights(s, ids), [0, 1])
    err = check_parity(y, ref, strict=True)
    print(f"K3 T=2: rel L2 {err}")


def test_k3_pooled_experts_equal_resident(b, k3):
    """The 896 K3 records in pinned host memory, 64 HBM slots filled on
    demand: consecutive single tokens (new experts each time, some slots
    evicted) give the resident layer's output bit for bit, and the first and
    last tokens' pooled outputs match the oracle."""
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
        if i in (0, 5):
            ids_np = ids.cpu().numpy()
            _, _, s = M.route(xh, k3.oracle)
            check_routing(ids_np, w.cpu().numpy(), s, 16)
            ref = oracle_rows(xh, k3.oracle, ids_np, oracle_weights(s, ids_np), [0])
            print(f"K3 pooled token {i}: rel L2 {check_parity(ys[0], ref, strict=True)[0]:.3e}")
    assert copied > 64  # the pool evicted and refilled
    del lay, pool, host


def test_k3_three_stacked_layers_teacher_forced(b, k3):
    """Three resident K3 layers (seeds [0, l, ...]), each RMSNorm -> MoE ->
    residual, 8 decode tokens, in the launch configuration of the 12-layer
    benchmark: per layer, the RMSNorm output within one bf16 ulp of the
    oracle's, routing, and every token's output against the oracle given the
    GPU's input to that layer (teacher forcing)."""
    layers = [k3]
    for l in (1, 2):
        built = Built(synth.K3, seed=0, layer=l)
        del built.dev["experts"]  # the packed copy is what the layer reads
        layers.append(built)
    T = 8
    gammas = [SD.upload_gamma(0, l, 7168) for l in range(3)]
    xh, xd = SD.upload_tokens(5400, T, 7168)
    ws = k3.lib.workspace(T)
    ys, normed, ids, wts = [xd], [], [], []
    for l in range(3):
        nd = torch.empty_like(xd)
        b.rmsnorm(ys[-1], gammas[l][1], 1e-6, nd)
        i_d = torch.empty((T, 16), dtype=torch.int32, device="cuda")
        w_d = torch.empty((T, 16), dtype=torch.float32, device="cuda")
        y = torch.empty_like(xd)
        b.moe_layer(layers[l].lib, nd, y, i_d, w_d, ws, residual=ys[-1], path=b.PATH_GEMV)
        normed.append(nd)
        ids.append(i_d)
        wts.append(w_d)
        ys.append(y)
    torch.cuda.synchronize()
    assert b.workspace_status(ws) == b.MOE_OK
    for l in range(3):
        x_in, n_gpu = to_np_u16(ys[l]), to_np_u16(normed[l])
        n_ref = M.rmsnorm(x_in, gammas[l][0])
        ulps = np.abs(n_gpu.view(np.int16).astype(np.int32) - n_ref.view(np.int16).astype(np.int32))
        assert ulps.max() <= 1, f"layer {l}: RMSNorm off by {ulps.max()} ulp"
        orc = layers[l].oracle
        _, _, s = M.route(n_gpu, orc)
        i_np = ids[l].cpu().numpy()
        check_routing(i_np, wts[l].cpu().numpy(), s, 16)
        ref = oracle_rows(n_gpu, orc, i_np, oracle_weights(s, i_np), range(T), residual_bits=x_in)
        err = check_parity(to_np_u16(ys[l + 1]), ref, strict=True)
        print(f"K3 stack layer {l}: {len(np.unique(i_np))} experts, rel L2 max {err.max():.3e}")
    del layers[1:]

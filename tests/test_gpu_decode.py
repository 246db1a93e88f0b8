"""GPU parity of the decode path (router, dequant-fused GEMV, shared experts,
combine) against the float64 oracle, through the C ABI.

Bars: bit-exact dequantised weights; routing equal up to near-ties within
1e-6 of the k-th score; layer output max over tokens of relative L2 error
<= 2e-3 (bf16 output vs float64 oracle).
"""

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from oracle import formats as F
from oracle import moe as M
from oracle import record as R
from tests._gpu import (Built, check_parity, check_routing, oracle_weights, to_np_u16,
                        topk_candidates)

pytestmark = pytest.mark.gpu

RAGGED = dict(hidden=288, inter=96, n_experts=40, top_k=5, n_shared=2)
WIDE = dict(hidden=8192, inter=64, n_experts=24, top_k=3, n_shared=1)
MANY = dict(hidden=128, inter=32, n_experts=1024, top_k=32, n_shared=0)
# every expert selected by every token (k = E), and a wide intermediate
ALL = dict(hidden=256, inter=128, n_experts=8, top_k=8, n_shared=1)
WIDE_I = dict(hidden=256, inter=2048, n_experts=16, top_k=4, n_shared=1)


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


@pytest.fixture(scope="module")
def tiny():
    return Built(synth.TINY, seed=0)


def _run_layer(b, built, x_dev, residual=None, path=1):
    T = x_dev.shape[0]
    k, H = built.cfg["top_k"], built.cfg["hidden"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.moe_layer(built.lib, x_dev, y, ids, w, ws, residual=residual, path=path)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), to_np_u16(y)


def _forward(b, built, x_dev, ids_np, w_np, residual=None):
    T = x_dev.shape[0]
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    w = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).cuda()
    y = torch.empty((T, built.cfg["hidden"]), dtype=torch.int16, device="cuda")
    ws = built.lib.workspace(T)
    b.forward(built.lib, x_dev, ids, w, y, ws, residual=residual, path=b.PATH_GEMV)
    torch.cuda.synchronize()
    return to_np_u16(y)


# ------------------------------------------------------------ dequant ----

def _export(b, built, e, m):
    H, I = built.cfg["hidden"], built.cfg["inter"]
    shape = (H, I) if m == R.DOWN else (I, H)
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    b.dequant_export(built.lib, e, m, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _bits_equal(gpu_f32, ref_f64):
    ref = ref_f64.astype(np.float32)
    g = gpu_f32.view(np.uint32)
    r = ref.view(np.uint32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(gpu_f32), nan)
    np.testing.assert_array_equal(g[~nan], r[~nan])


def test_dequant_export_bit_exact_tiny(b, tiny):
    for e in range(tiny.cfg["n_experts"]):
        rec = tiny.oracle.expert_record(e)
        for m in (R.GATE, R.UP, R.DOWN):
            _bits_equal(_export(b, tiny, e, m), R.dequant_matrix(rec, 256, 64, m))


def test_dequant_export_extreme_scales_and_every_code(b):
    H, I = 64, 32
    rb = R.record_bytes(H, I)
    recs = np.zeros((2, rb), dtype=np.uint8)
    for j in range(2):
        views = R.split(recs[j], H, I)
        for m in range(3):
            codes, scales = views[2 * m], views[2 * m + 1]
            codes[...] = np.arange(codes.size, dtype=np.int64).reshape(codes.shape) % 256
            pattern = np.array([0, 1, 2, 126, 127, 128, 253, 254, 255] if j == 0 else [118, 126])
            scales[...] = pattern[np.arange(scales.size) % len(pattern)].reshape(scales.shape)
    experts = torch.from_numpy(recs).cuda()
    wr = torch.zeros((2, H), dtype=torch.int16, device="cuda")
    layer = b.Layer.from_canonical(H, I, 2, 1, wr, experts)
    for j in range(2):
        for m in range(3):
            shape = (H, I) if m == 2 else (I, H)
            out = torch.empty(shape, dtype=torch.float32, device="cuda")
            b.dequant_export(layer, j, m, out)
            torch.cuda.synchronize()
            _bits_equal(out.cpu().numpy(), R.dequant_matrix(recs[j], H, I, m))


# ------------------------------------------------------------- router ----

def test_route_tiny_matches_oracle(b, tiny):
    xh, xd = SD.upload_tokens(1000, 64, 256)
    ids, w, _ = _run_layer(b, tiny, xd)
    _, _, s = M.route(xh, tiny.oracle)
    check_routing(ids, w, s, 4)
    np.testing.assert_allclose(w, oracle_weights(s, ids), rtol=0, atol=2e-6)


def test_route_exact_ties_lower_index(b):
    cfg = dict(hidden=256, inter=64, n_experts=32, top_k=4, n_shared=0)
    built = Built(cfg, seed=3)
    wr = built.dev["router_w"]
    wr[:] = wr[5]            # every row equal: all logits tie exactly
    xh, xd = SD.upload_tokens(1001, 3, 256)
    ids, w, _ = _run_layer(b, built, xd)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    np.testing.assert_allclose(w, 0.25, atol=1e-7)


def _route(b, built, x_dev):
    T, k = x_dev.shape[0], built.cfg["top_k"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    b.route(built.lib, x_dev, ids, w, built.lib.workspace(T))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def test_route_entry_matches_oracle_and_layer_routing(b):
    # 70 tokens: 18 top-k workgroups, the last of which builds the plan
    built = Built(MANY, seed=5, bias=True)
    xh, xd = SD.upload_tokens(1300, 70, MANY["hidden"])
    ids, w = _route(b, built, xd)
    _, _, s = M.route(xh, built.oracle)
    check_routing(ids, w, s, MANY["top_k"])
    np.testing.assert_allclose(w, oracle_weights(s, ids), rtol=0, atol=2e-6)
    ids2, w2, _ = _run_layer(b, built, xd)
    assert np.array_equal(ids, ids2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32))


def test_route_many_winners_in_one_lane(b):
    """Experts 5, 69, 133, ... (e = 5 mod 64) sit in one lane of the top-k
    wave; a bias of +20 makes all 16 of them winners, so one lane contributes
    a single maximum but 16 of the 32 selected experts.  The threshold (k-th
    of the 64 lane maxima) then admits 56-58 candidates, all ranked in the
    candidate list (the exact path past 256 candidates is covered by
    test_gpu_topk_exact.py)."""
    built = Built(MANY, seed=6, bias=True)
    bias = built.dev["host_bias"].copy()
    bias[5::64] += 20.0
    built.dev["router_bias"].copy_(torch.from_numpy(bias))
    built.oracle.router_bias = bias
    xh, xd = SD.upload_tokens(1301, 5, MANY["hidden"])
    ids, w = _route(b, built, xd)
    _, _, s = M.route(xh, built.oracle)
    assert all(32 < topk_candidates(s[t], 32) <= 256 for t in range(5))
    check_routing(ids, w, s, MANY["top_k"])
    np.testing.assert_allclose(w, oracle_weights(s, ids), rtol=0, atol=2e-6)
    for t in range(5):
        assert set(range(5, 1024, 64)) <= set(ids[t].tolist())
        assert np.all(ids[t][:16] % 64 == 5)


# ------------------------------------------------------------- layer -----

@pytest.mark.parametrize("T", [1, 3, 16])
def test_forward_tiny_given_oracle_routing(b, tiny, T):
    xh, xd = SD.upload_tokens(1002 + T, T, 256)
    ids, w, _ = M.route(xh, tiny.oracle)
    w32 = w.astype(np.float32)
    y = _forward(b, tiny, xd, ids, w32)
    ref = M.moe_forward(xh, tiny.oracle, ids, w32.astype(np.float64))
    check_parity(y, ref)


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED, WIDE, MANY, ALL, WIDE_I],
                         ids=["tiny", "ragged", "wide", "many", "all", "wide_i"])
@pytest.mark.parametrize("T", [1, 4, 7, 70])
def test_layer_matches_oracle(b, cfg, T):
    built = Built(cfg, seed=11)
    xh, xd = SD.upload_tokens(1100 + T, T, cfg["hidden"])
    ids, w, y = _run_layer(b, built, xd)
    _, _, s = M.route(xh, built.oracle)
    check_routing(ids, w, s, cfg["top_k"])
    ref = M.moe_forward(xh, built.oracle, ids, oracle_weights(s, ids))
    check_parity(y, ref)


def test_residual_added(b, tiny):
    xh, xd = SD.upload_tokens(1200, 5, 256)
    rh, rd = SD.upload_tokens(1201, 5, 256)
    ids, w, _ = M.route(xh, tiny.oracle)
    y = _forward(b, tiny, xd, ids, w, residual=rd)
    ref = M.moe_forward(xh, tiny.oracle, ids, w.astype(np.float32).astype(np.float64),
                        residual_bits=rh)
    check_parity(y, ref)


def test_one_more_scale_exponent_doubles_output_bitwise(b):
    """All up scales +1 doubles every routed partial exactly in fp32; with no
    shared experts the bf16 output doubles bit for bit."""
    cfg = dict(hidden=256, inter=64, n_experts=8, top_k=2, n_shared=0)
    built = Built(cfg, seed=4)
    xh, xd = SD.upload_tokens(1300, 4, 256)
    _, _, y1 = _run_layer(b, built, xd)
    ex = built.dev["experts"].cpu().numpy()
    for e in range(8):
        R.split(ex[e], 256, 64)[3][...] += 1
    built.dev["experts"].copy_(torch.from_numpy(ex))
    built.repack()
    _, _, y2 = _run_layer(b, built, xd)
    np.testing.assert_array_equal(F.bf16_decode(y2), 2.0 * F.bf16_decode(y1))


def test_zero_routed_experts_leave_shared_only(b):
    cfg = dict(hidden=256, inter=64, n_experts=8, top_k=3, n_shared=2)
    built = Built(cfg, seed=5)
    built.dev["experts"].zero_()
    built.repack()
    xh, xd = SD.upload_tokens(1400, 4, 256)
    _, _, y = _run_layer(b, built, xd)
    ref = M.shared_sum(xh, built.oracle)
    check_parity(y, ref)


def test_all_experts_equal_is_routing_independent(b):
    cfg = dict(hidden=256, inter=64, n_experts=16, top_k=4, n_shared=1)
    built = Built(cfg, seed=6)
    built.dev["experts"][:] = built.dev["experts"][7]
    built.repack()
    xh, xd = SD.upload_tokens(1500, 6, 256)
    ids1, _, y1 = _run_layer(b, built, xd)
    built.dev["router_w"].copy_(torch.flip(built.dev["router_w"], dims=[0]))
    built.repack()
    ids2, _, y2 = _run_layer(b, built, xd)
    assert not np.array_equal(ids1, ids2)
    rec = synth.expert_record(6, 0, 7, 256, 64)
    xv = F.bf16_decode(xh)
    dense = M.expert_ffn(xv, *R.dequant_expert(rec, 256, 64)) + M.shared_sum(xh, built.oracle)
    check_parity(y1, dense)
    check_parity(y2, dense)


def test_deterministic(b, tiny):
    xh, xd = SD.upload_tokens(1600, 9, 256)
    a = _run_layer(b, tiny, xd)
    c = _run_layer(b, tiny, xd)
    for u, v in zip(a, c):
        np.testing.assert_array_equal(u, v)


# --------------------------------------------------------------- misc ----

def test_rmsnorm_within_one_bf16_ulp(b):
    H = 7168
    xh, xd = SD.upload_tokens(1700, 8, H)
    gh, gd = SD.upload_gamma(0, 0, H)
    out = torch.empty_like(xd)
    b.rmsnorm(xd, gd, 1e-6, out)
    torch.cuda.synchronize()
    got = to_np_u16(out).astype(np.int32)
    ref = M.rmsnorm(xh, gh, 1e-6).astype(np.int32)
    d = np.abs(got - ref)
    assert d.max() <= 1
    assert (d > 0).mean() < 1e-3


def test_mxfp8_quantize_bit_exact(b):
    g = np.random.default_rng(0)
    v = g.standard_normal((16, 7168)).astype(np.float32) * np.exp(g.uniform(-30, 30, (16, 1)))
    v[0, :32] = 0.0
    v[1, 32:64] = -0.0
    v[2, 64] = 3e38
    xh = synth.to_bf16_bits(v)
    xd = torch.from_numpy(xh.view(np.int16)).cuda()
    codes = torch.empty((16, 7168), dtype=torch.uint8, device="cuda")
    scales = torch.empty((16, 224), dtype=torch.uint8, device="cuda")
    b.mxfp8_quantize(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = F.mxfp8_quantize(F.bf16_decode(xh))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_consecutive_calls_with_changing_inputs(b):
    """Back-to-back calls on one workspace, each with new tokens and its own
    check: partials of an earlier call must never leak into a later one."""
    cfg = dict(hidden=512, inter=128, n_experts=64, top_k=6, n_shared=2)
    built = Built(cfg, seed=8)
    T = 3
    ids = torch.empty((T, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 6), dtype=torch.float32, device="cuda")
    ws = built.lib.workspace(T)
    outs, xs = [], []
    for i in range(12):
        xh, xd = SD.upload_tokens(1800 + i, T, 512)
        y = torch.empty((T, 512), dtype=torch.int16, device="cuda")
        b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_GEMV)
        outs.append((y, ids.clone(), w.clone()))
        xs.append(xh)
    torch.cuda.synchronize()
    for xh, (y, i_, w_) in zip(xs, outs):
        _, _, s = M.route(xh, built.oracle)
        ids_np = i_.cpu().numpy()
        check_routing(ids_np, w_.cpu().numpy(), s, 6)
        ref = M.moe_forward(xh, built.oracle, ids_np, oracle_weights(s, ids_np))
        check_parity(to_np_u16(y), ref)


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_one_token_on_an_uninitialised_workspace(b, fill):
    """One token runs the whole layer in one launch whose workgroups hand
    over through the workspace: epoch-tagged expert words and flags, and
    arrival counters the top-k clears.  None of it needs initialising: calls
    on a workspace refilled before each call with zero bytes, all-one bytes
    or random bytes match the oracle and report no give-up.  The ragged
    shape leaves a short last output tile (288 = 256 + 32 rows)."""
    built = Built(RAGGED, seed=17)
    H, k = RAGGED["hidden"], RAGGED["top_k"]
    ws = built.lib.workspace(1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H), dtype=torch.int16, device="cuda")
    for i in range(3):
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(255)
        else:
            ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda",
                                   generator=gen))
        xh, xd = SD.upload_tokens(7100 + i, 1, H)
        b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_GEMV)
        torch.cuda.synchronize()
        assert b.workspace_status(ws) == b.MOE_OK
        _, _, s = M.route(xh, built.oracle)
        ids_np = ids.cpu().numpy()
        check_routing(ids_np, w.cpu().numpy(), s, k)
        check_parity(to_np_u16(y), M.moe_forward(xh, built.oracle, ids_np,
                                                 oracle_weights(s, ids_np)))


def test_alternating_batch_sizes_share_a_workspace(b):
    """One workspace, token counts alternating over the three launch
    structures (one token: no plan; 2-4 tokens: top-k and plan inside the
    router launch; more: a top-k launch).  Every call matches the oracle,
    and after each call the logits completion flags (after the status
    word's 256-byte slot at the start of the workspace) are all clear (the
    top-k workgroup clears what it waited on) and no wait gave up."""
    cfg = dict(hidden=512, inter=128, n_experts=64, top_k=6, n_shared=2)
    built = Built(cfg, seed=11)
    ws = built.lib.workspace(9)
    n_flags = (64 + 3) // 4
    for i, T in enumerate([1, 4, 9, 2, 1, 3, 9, 1]):
        xh, xd = SD.upload_tokens(1900 + i, T, 512)
        ids = torch.empty((T, 6), dtype=torch.int32, device="cuda")
        w = torch.empty((T, 6), dtype=torch.float32, device="cuda")
        y = torch.empty((T, 512), dtype=torch.int16, device="cuda")
        b.moe_layer(built.lib, xd, y, ids, w, ws, path=b.PATH_GEMV)
        torch.cuda.synchronize()
        if T <= 8:
            flags = ws[256:256 + 8 * n_flags].cpu().numpy().view(np.uint64)
            assert not flags.any(), (T, flags)
        assert b.workspace_status(ws) == b.MOE_OK
        _, _, s = M.route(xh, built.oracle)
        ids_np = ids.cpu().numpy()
        check_routing(ids_np, w.cpu().numpy(), s, 6)
        ref = M.moe_forward(xh, built.oracle, ids_np, oracle_weights(s, ids_np))
        check_parity(to_np_u16(y), ref)

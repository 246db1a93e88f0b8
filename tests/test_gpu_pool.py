"""GPU tests of the expert pool (experts not resident: records in host memory,
a few HBM slots filled on demand; Deltafin README, I/O and streaming).

The pooled layer runs the same kernels on the same packed records, only
found through the slot map, so its output must equal the resident layer's
bit for bit; it is also compared with the oracle directly (routing, the
per-token relative L2 bar and the element-wise bound; on the MFMA path the
pooled call's MXFP8 codes too).  The fetch bookkeeping (copies, hits, least-recently-used
eviction among the experts a call does not need) is checked by counts.
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


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def _pooled(b, built, n_slots, pinned=True):
    host = built.lib.experts.cpu()
    if pinned:
        host = host.pin_memory()
    pool = b.ExpertPool(host, n_slots)
    c = built.cfg
    lay = b.Layer(c["hidden"], c["inter"], c["n_experts"], c["top_k"], built.lib.router_w,
                  pool.slots, built.lib.shared_gate, built.lib.shared_up, built.lib.shared_down,
                  built.lib.router_bias, pool=pool)
    return pool, lay


def _route(b, built, xd):
    T, k = xd.shape[0], built.cfg["top_k"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    b.route(built.lib, xd, ids, w, built.lib.workspace(T))
    return ids, w


def _forward(b, lay, xd, ids, w, path, ws=None):
    y = torch.empty((xd.shape[0], lay.hidden), dtype=torch.int16, device="cuda")
    ws = lay.workspace(xd.shape[0]) if ws is None else ws
    b.forward(lay, xd, ids, w, y, ws, path=path)
    torch.cuda.synchronize()
    return to_np_u16(y)


def _check_oracle(built, xh, ids, w, y, mx=None):
    """Pooled output against the oracle under the call's routing; mx =
    (binding, layer, workspace) of an MFMA-path call to check its codes."""
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    _, _, s = M.route(xh, built.oracle)
    check_routing(ids_np, w_np, s, built.cfg["top_k"])
    ref = M.moe_forward(xh, built.oracle, ids_np, oracle_weights(s, ids_np),
                        act_mxfp8=mx is not None)
    eff = None
    if mx is not None:
        b, lay, ws = mx
        eff = check_mxfp8_workspace(b, lay, ws, xh.shape[0], xh, ids_np, w_np, built.oracle)
    check_parity(y, ref, eff)


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED], ids=["tiny", "ragged"])
@pytest.mark.parametrize("T", [1, 3, 6])
def test_pooled_layer_equals_resident_gemv(b, cfg, T):
    built = Built(cfg, seed=31)
    calls = []
    for call in range(6):  # new tokens each call
        xh, xd = SD.upload_tokens(3100 + 10 * T + call, T, cfg["hidden"])
        calls.append((xh, xd, *_route(b, built, xd)))
    # as many slots as the largest call needs: later calls must evict
    n_slots = max(np.unique(ids.cpu().numpy()).size for _, _, ids, _ in calls)
    pool, lay = _pooled(b, built, n_slots)
    copied_total = 0
    for xh, xd, ids, w in calls:
        copied_total += pool.fetch(ids.cpu().numpy())
        y = _forward(b, lay, xd, ids, w, b.PATH_GEMV)
        np.testing.assert_array_equal(y, _forward(b, built.lib, xd, ids, w, b.PATH_GEMV))
        _check_oracle(built, xh, ids, w, y)
    assert copied_total > n_slots  # some records were evicted and refilled


@pytest.mark.parametrize("cfg", [synth.TINY, RAGGED], ids=["tiny", "ragged"])
@pytest.mark.parametrize("T", [70, 300])
def test_pooled_layer_equals_resident_mfma(b, cfg, T):
    # a batch this large reaches nearly every expert, so the pool holds all
    # of them, in a shuffled slot order: the slot map is a real permutation
    built = Built(cfg, seed=35, bias=True)
    E = cfg["n_experts"]
    pool, lay = _pooled(b, built, E)
    order = np.random.default_rng(7).permutation(E)
    assert pool.fetch(order) == E
    smap = pool.slot_map.cpu().numpy()
    np.testing.assert_array_equal(smap[order], np.arange(E))
    xh, xd = SD.upload_tokens(3300 + T, T, cfg["hidden"])
    ids, w = _route(b, built, xd)
    assert pool.fetch(ids.cpu().numpy()) == 0
    ws = lay.workspace(T)
    y = _forward(b, lay, xd, ids, w, b.PATH_MFMA, ws)
    np.testing.assert_array_equal(y, _forward(b, built.lib, xd, ids, w, b.PATH_MFMA))
    _check_oracle(built, xh, ids, w, y, mx=(b, lay, ws))


def test_fetch_counts_and_lru_eviction(b):
    built = Built(synth.TINY, seed=32)
    pool, lay = _pooled(b, built, 4)
    assert pool.fetch([0, 1, 2, 3]) == 4
    assert pool.fetch([3, 2, 3]) == 0           # repeats and residents copy nothing
    assert pool.fetch([4, 5]) == 2              # evicts 0 and 1: used longest ago
    assert pool.fetch([2, 3]) == 0              # 2 and 3 were kept
    assert pool.fetch([0, 1, 2, 3]) == 2        # 0 and 1 come back in 4's and 5's slots
    copied, resident = pool.stats()
    assert copied == 8 and resident == 2 + 2 + 2
    # the slot map the kernels read names the slot holding each expert
    smap = pool.slot_map.cpu().numpy()
    slots = pool.slots.cpu()
    for e in (0, 1, 2, 3):
        assert torch.equal(slots[smap[e]], built.lib.experts[e].cpu())


def test_more_distinct_experts_than_slots_is_refused(b):
    built = Built(synth.TINY, seed=33)
    pool, _ = _pooled(b, built, 3)
    with pytest.raises(b.MoeError, match="MOE_ESHAPE"):
        pool.fetch([0, 1, 2, 3])
    with pytest.raises(b.MoeError, match="MOE_EINVAL"):
        pool.fetch([0, 32])                     # not an expert of this layer
    assert pool.stats() == (0, 0)               # nothing was done


def test_pageable_host_records(b):
    built = Built(synth.TINY, seed=34)
    pool, lay = _pooled(b, built, 8, pinned=False)
    xh, xd = SD.upload_tokens(3200, 2, 256)
    ids, w = _route(b, built, xd)
    pool.fetch(ids.cpu().numpy())
    np.testing.assert_array_equal(_forward(b, lay, xd, ids, w, b.PATH_GEMV),
                                  _forward(b, built.lib, xd, ids, w, b.PATH_GEMV))


@pytest.mark.parametrize("path,T", [("gemv", 1), ("gemv", 3), ("mfma", 8)])
def test_forward_pooled_waits_for_fetch_on_another_stream(b, path, T):
    """The records are fetched on a second stream while the shared experts
    run; the routed part waits for the event recorded after the fetch.  Each
    call evicts records the previous one used (few slots), so a routed kernel
    that ran before its copies landed would read another expert's record."""
    cfg = RAGGED
    built = Built(cfg, seed=36)
    p = b.PATH_GEMV if path == "gemv" else b.PATH_MFMA
    calls = []
    for call in range(4):
        xh, xd = SD.upload_tokens(3400 + 10 * T + call, T, cfg["hidden"])
        calls.append((xh, xd, *_route(b, built, xd)))
    n_slots = max(np.unique(ids.cpu().numpy()).size for _, _, ids, _ in calls)
    pool, lay = _pooled(b, built, n_slots)
    copy_stream = torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    ws = lay.workspace(T)
    copied_total = 0
    for xh, xd, ids, w in calls:
        ids_host = ids.cpu().numpy()
        copy_stream.wait_stream(main)  # earlier reads of the slots come first
        copied_total += pool.fetch(ids_host, stream=copy_stream)
        ready = torch.cuda.Event()
        ready.record(copy_stream)
        y = torch.empty((T, cfg["hidden"]), dtype=torch.int16, device="cuda")
        b.forward_pooled(lay, xd, ids, w, y, ws, ready, path=p)
        torch.cuda.synchronize()
        yn = to_np_u16(y)
        np.testing.assert_array_equal(yn, _forward(b, built.lib, xd, ids, w, p))
        _check_oracle(built, xh, ids, w, yn, mx=(b, lay, ws) if path == "mfma" else None)
    assert copied_total > n_slots


def test_forward_pooled_without_event_is_forward(b):
    built = Built(synth.TINY, seed=37)
    pool, lay = _pooled(b, built, 8)
    xh, xd = SD.upload_tokens(3500, 2, 256)
    ids, w = _route(b, built, xd)
    pool.fetch(ids.cpu().numpy())
    y = torch.empty((2, 256), dtype=torch.int16, device="cuda")
    b.forward_pooled(lay, xd, ids, w, y, lay.workspace(2), None, path=b.PATH_GEMV)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np_u16(y), _forward(b, lay, xd, ids, w, b.PATH_GEMV))

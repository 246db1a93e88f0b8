"""C-ABI library: loads, exports exactly the header's functions, and rejects
invalid arguments on the host before launching anything (CPU only: every
call here fails validation, so no device pointer is ever dereferenced).
"""

import ctypes
import os

import pytest
import torch

from mxfp4_routed_expert_x896_amd import build as B


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        B.build()
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def test_exports_match_header(lib):
    lib.lib()
    want = B.header_functions()
    assert "moe_route" in want and "moe_forward" in want and "moe_layer" in want
    assert B.exported_functions() == want


def test_library_is_gfx950_only():
    import re
    blob = open(B.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[-a-z]*gfx[0-9a-z]+", blob))
    assert targets == {b"amdgcn-amd-amdhsa--gfx950"}


def test_abi_version_and_record_bytes(lib):
    assert lib.lib().moe_abi_version() >> 16 == lib.ABI_MAJOR
    assert lib.record_bytes(7168, 1536) == 17_547_264
    assert lib.record_bytes(256, 64) == 26_112
    out = ctypes.c_uint64()
    assert lib.lib().moe_record_bytes(100, 64, ctypes.byref(out)) == -3
    assert lib.lib().moe_record_bytes(256, 64, None) == -1


PACKED_TINY = 38_912  # packed record of H=256, I=64 (K=64 padded to 128 columns, scales to 4 tiles)


def _desc(lib, **kw):
    d = dict(hidden=256, inter=64, n_experts=32, top_k=4, n_shared=1, router_mode=0,
             router_w=0x10000, router_bias=None, experts=0x20000, expert_stride=PACKED_TINY,
             shared_gate=0x30000, shared_up=0x40000, shared_down=0x50000)
    d.update(kw)
    return lib.LayerDesc(**d)


def test_packed_record_bytes(lib):
    assert lib.packed_record_bytes(7168, 1536) == 17_547_264  # same bytes as canonical
    assert lib.packed_record_bytes(256, 64) == PACKED_TINY
    out = ctypes.c_uint64()
    assert lib.lib().moe_packed_record_bytes(96, 64, ctypes.byref(out)) == 0
    assert lib.lib().moe_packed_record_bytes(100, 64, ctypes.byref(out)) == -3


def test_pack_calls_reject_bad_arguments(lib):
    L = lib.lib()
    P = ctypes.c_void_p
    a, b = P(0x100000), P(0x900000)
    assert L.moe_pack_experts(None, 26_112, b, PACKED_TINY, 4, 256, 64, None) == -1
    assert L.moe_pack_experts(a, 26_112, b, PACKED_TINY, 0, 256, 64, None) == -1
    assert L.moe_pack_experts(a, 26_112, b, PACKED_TINY, 4, 250, 64, None) == -3
    assert L.moe_pack_experts(a, 26_000, b, PACKED_TINY, 4, 256, 64, None) == -3
    assert L.moe_pack_experts(a, 26_112, b, PACKED_TINY - 16, 4, 256, 64, None) == -3
    assert L.moe_pack_experts(a, 26_112, P(0x900008), PACKED_TINY, 4, 256, 64, None) == -2
    assert L.moe_pack_bf16(a, b, 2, 20, 64, None) == -3
    assert L.moe_pack_bf16(a, b, 2, 16, 48, None) == -3
    assert L.moe_pack_bf16(a, None, 2, 16, 64, None) == -1


def _ws(lib, desc, t):
    out = ctypes.c_uint64()
    st = lib.lib().moe_workspace_bytes(ctypes.byref(desc), t, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(hidden=250), -3),
    (dict(inter=48), -3),
    (dict(hidden=8224), -3),
    (dict(n_experts=1025), -3),
    (dict(top_k=33, n_experts=64), -3),
    (dict(top_k=40), -3),
    (dict(n_shared=5), -3),
    (dict(router_w=None), -1),
    (dict(experts=None), -1),
    (dict(shared_down=None), -1),
    (dict(n_shared=0, shared_gate=None, shared_up=None, shared_down=None), 0),
    (dict(router_w=0x10008), -2),
    (dict(expert_stride=PACKED_TINY + 8), -2),
    (dict(expert_stride=PACKED_TINY - 16), -3),
    (dict(router_mode=1), 0),
    (dict(router_mode=2), -1),
    (dict(router_mode=-1), -1),
    (dict(routed_scale=2.5), 0),
    (dict(routed_scale=-1.0), -1),
    (dict(routed_scale=float("nan")), -1),
    (dict(routed_scale=float("inf")), -1),
    (dict(expert_slot=0x20000, n_slots=3), 0),     # an expert pool of 3 records
    (dict(expert_slot=0x20000, n_slots=0), -1),
    (dict(expert_slot=None, n_slots=2), -1),
    (dict(expert_slot=0x20002, n_slots=3), -2),
])
def test_descriptor_validation(lib, kw, status):
    st, nbytes = _ws(lib, _desc(lib, **kw), 4)
    assert st == status
    if status == 0:
        assert nbytes > 0


def test_workspace_grows_with_tokens_and_token_limits(lib):
    d = _desc(lib)
    s1, b1 = _ws(lib, d, 1)
    s2, b2 = _ws(lib, d, 64)
    assert s1 == 0 and s2 == 0 and b2 > b1
    assert _ws(lib, d, 0)[0] == -1
    assert _ws(lib, d, 1 << 16)[0] == 0   # the largest batch one call takes
    assert _ws(lib, d, (1 << 16) + 1)[0] == -3
    assert _ws(lib, d, 1 << 17)[0] == -3


def test_calls_reject_bad_arguments_before_launch(lib):
    L = lib.lib()
    d = _desc(lib)
    _, need = _ws(lib, d, 2)
    P = ctypes.c_void_p
    x, ids, w, y, ws = P(0x100000), P(0x200000), P(0x300000), P(0x400000), P(0x500000)
    dp = ctypes.byref(d)
    assert L.moe_route(dp, None, 2, ids, w, ws, need, None) == -1
    assert L.moe_route(dp, x, 0, ids, w, ws, need, None) == -1
    assert L.moe_route(dp, P(0x100004), 2, ids, w, ws, need, None) == -2
    assert L.moe_route(dp, x, 2, ids, w, ws, need - 1, None) == -4
    assert L.moe_forward(dp, x, 2, ids, w, None, None, 1, ws, need, None) == -1
    assert L.moe_forward(dp, x, 2, ids, w, None, y, 7, ws, need, None) == -1
    assert L.moe_forward(dp, x, 2, ids, w, P(0x600002), y, 1, ws, need, None) == -2
    assert L.moe_forward(dp, x, 2, ids, w, None, y, 1, ws, 16, None) == -4
    assert L.moe_layer(dp, x, 2, None, y, ids, None, 1, ws, need, None) == -1
    assert L.moe_rmsnorm(x, None, 1e-6, 2, 256, y, None) == -1
    assert L.moe_rmsnorm(x, x, 1e-6, 2, 100, y, None) == -3
    assert L.moe_rmsnorm(x, x, -1.0, 2, 256, y, None) == -1
    assert L.moe_dequant_export(dp, 32, 0, y, None) == -1
    assert L.moe_dequant_export(dp, 0, 3, y, None) == -1
    assert L.moe_mxfp8_quantize(x, 2, 48, y, w, None) == -3
    for code in (0, -1, -2, -3, -4, -5, -6, -7, 99):
        assert L.moe_status_string(code)


def test_int8_dequant_rejects_bad_arguments(lib):
    L = lib.lib()
    P = ctypes.c_void_p
    q, s, o = P(0x100000), P(0x200000), P(0x300000)
    assert L.moe_int8_row_dequant(None, s, 4, 64, o, None) == -1
    assert L.moe_int8_row_dequant(q, s, 0, 64, o, None) == -1
    assert L.moe_int8_row_dequant(q, s, 4, -4, o, None) == -1
    assert L.moe_int8_row_dequant(q, s, 4, 66, o, None) == -3
    assert L.moe_int8_row_dequant(P(0x100002), s, 4, 64, o, None) == -2
    assert L.moe_int8_row_dequant(q, P(0x200002), 4, 64, o, None) == -2
    assert L.moe_int8_row_dequant(q, s, 4, 64, P(0x300004), None) == -2
    assert L.moe_int8_row_dequant(q, s, 1 << 30, 1 << 12, o, None) == -3  # 2^42 elements


def test_pool_calls_reject_bad_arguments(lib):
    L = lib.lib()
    P = ctypes.c_void_p
    host, slots, smap = P(0x100000), P(0x200000), P(0x300000)
    out = P()
    o = ctypes.byref(out)
    assert L.moe_pool_create(host, PACKED_TINY, 32, slots, 8, smap, None, None) == -1
    assert L.moe_pool_create(None, PACKED_TINY, 32, slots, 8, smap, None, o) == -1
    assert L.moe_pool_create(host, PACKED_TINY, 32, None, 8, smap, None, o) == -1
    assert L.moe_pool_create(host, PACKED_TINY, 32, slots, 0, smap, None, o) == -1
    assert L.moe_pool_create(host, PACKED_TINY, 32, slots, 33, smap, None, o) == -3
    assert L.moe_pool_create(host, PACKED_TINY + 8, 32, slots, 8, smap, None, o) == -2
    assert L.moe_pool_create(host, PACKED_TINY, 32, P(0x200008), 8, smap, None, o) == -2
    assert L.moe_pool_create(host, PACKED_TINY, 32, slots, 8, P(0x300002), None, o) == -2
    assert out.value is None
    ids = (ctypes.c_int32 * 2)(1, 2)
    assert L.moe_pool_fetch(None, ids, 2, None, None) == -1
    assert L.moe_pool_stats(None, None, None) == -1
    assert L.moe_pool_destroy(None) == -1


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU refusal")
def test_valid_call_without_gfx950_refuses(lib):
    L = lib.lib()
    d = _desc(lib)
    _, need = _ws(lib, d, 2)
    P = ctypes.c_void_p
    st = L.moe_route(ctypes.byref(d), P(0x100000), 2, P(0x200000), P(0x300000), P(0x500000),
                     need, None)
    assert st == -5


def test_status_and_region_calls(lib):
    """The workspace status query and the region export validate on the host;
    the regions of one workspace are disjoint and inside it."""
    L = lib.lib()
    P = ctypes.c_void_p
    assert L.moe_workspace_status(None, 64, None) == -1
    assert L.moe_workspace_status(P(0x100000), 4, None) == -1
    assert L.moe_workspace_status(P(0x100004), 64, None) == -2
    assert L.moe_set_wait_limit(-1) == 0
    assert L.moe_status_string(-8)
    d = _desc(lib)
    off, n = ctypes.c_uint64(), ctypes.c_uint64()
    for T in (1, 7, 300):
        _, total = _ws(lib, d, T)
        spans = []
        for region in range(5):
            assert L.moe_workspace_region(ctypes.byref(d), T, region, ctypes.byref(off),
                                          ctypes.byref(n)) == 0
            assert off.value % 16 == 0 and off.value + n.value <= total
            spans.append((off.value, off.value + n.value))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert spans[0][0] >= 8  # the status word stays first
    assert L.moe_workspace_region(ctypes.byref(d), 4, 5, ctypes.byref(off), ctypes.byref(n)) == -1
    assert L.moe_workspace_region(ctypes.byref(d), 0, 0, ctypes.byref(off), ctypes.byref(n)) == -1
    assert L.moe_workspace_region(ctypes.byref(d), 4, 0, None, ctypes.byref(n)) == -1


def test_mfma_rate_rejects_bad_arguments(lib):
    L = lib.lib()
    P = ctypes.c_void_p
    out = P(0x100000)
    assert L.moe_mfma_rate(4, 4, 10, 4, None, None) == -1
    assert L.moe_mfma_rate(4, 4, 0, 4, out, None) == -1
    assert L.moe_mfma_rate(4, 4, 10, 0, out, None) == -1
    assert L.moe_mfma_rate(0, 4, 10, 4, out, None) == -7   # FP8 x FP4: not offered
    assert L.moe_mfma_rate(2, 2, 10, 4, out, None) == -7
    assert L.moe_mfma_rate(4, 0, 10, 4, P(0x100002), None) == -2

"""ctypes binding of libmoe_mxfp4.so (argument marshalling only).

Every call forwards device pointers of torch tensors and torch's current HIP
stream to the C ABI in include/moe_mxfp4.h; all arithmetic runs in the
library's gfx950 kernels.  torch is used for device memory and streams only.
Loading fails loudly when the library has not been built: there is no
fallback path.
"""

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library links against)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mxfp4.so")

ABI_MAJOR = 3

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EALIGN", -3: "MOE_ESHAPE",
                -4: "MOE_EWORKSPACE", -5: "MOE_EDEVICE", -6: "MOE_ELAUNCH",
                -7: "MOE_EUNSUPPORTED", -8: "MOE_ETIMEOUT"}

PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_MFMA_FP4 = 0, 1, 2, 3
ROUTER_BIAS_LOGITS, ROUTER_BIAS_SELECT = 0, 1
GATE, UP, DOWN = 0, 1, 2
WS_PAIRS, WS_X_CODES, WS_X_SCALES, WS_H_CODES, WS_H_SCALES = range(5)
MOE_ETIMEOUT = -8


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib().moe_status_string(status).decode()
        extra = ""
        if status == -6:
            extra = f" (hipError {_lib().moe_last_hip_error()})"
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}{extra}")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
        ("router_mode", ctypes.c_int32),
        ("router_w", ctypes.c_void_p),
        ("router_bias", ctypes.c_void_p),
        ("experts", ctypes.c_void_p),
        ("expert_stride", ctypes.c_uint64),
        ("shared_gate", ctypes.c_void_p),
        ("shared_up", ctypes.c_void_p),
        ("shared_down", ctypes.c_void_p),
        ("expert_slot", ctypes.c_void_p),
        ("n_slots", ctypes.c_int32),
        ("routed_scale", ctypes.c_float),
    ]


_LIB = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_DESC = ctypes.POINTER(LayerDesc)

_SIGNATURES = {
    "moe_abi_version": (ctypes.c_uint32, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_hip_error": (ctypes.c_int, []),
    "moe_record_bytes": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(_U64)]),
    "moe_workspace_bytes": (ctypes.c_int, [_DESC, _I64, ctypes.POINTER(_U64)]),
    "moe_route": (ctypes.c_int, [_DESC, _P, _I64, _P, _P, _P, _U64, _P]),
    "moe_forward": (ctypes.c_int, [_DESC, _P, _I64, _P, _P, _P, _P, _I32, _P, _U64, _P]),
    "moe_layer": (ctypes.c_int, [_DESC, _P, _I64, _P, _P, _P, _P, _I32, _P, _U64, _P]),
    "moe_forward_pooled": (ctypes.c_int, [_DESC, _P, _I64, _P, _P, _P, _P, _I32, _P, _U64, _P,
                                          _P]),
    "moe_mfma_min_tokens": (ctypes.c_int64, []),
    "moe_rmsnorm": (ctypes.c_int, [_P, _P, ctypes.c_float, _I64, _I32, _P, _P]),
    "moe_dequant_export": (ctypes.c_int, [_DESC, _I32, _I32, _P, _P]),
    "moe_mxfp8_quantize": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P]),
    "moe_int8_row_dequant": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "moe_packed_record_bytes": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(_U64)]),
    "moe_pack_experts": (ctypes.c_int, [_P, _U64, _P, _U64, _I32, _I32, _I32, _P]),
    "moe_pack_bf16": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P]),
    "moe_profile_events": (ctypes.c_int, [_P, _I32]),
    "moe_profile_count": (ctypes.c_int, []),
    "moe_pool_create": (ctypes.c_int, [_P, _U64, _I32, _P, _I32, _P, _P, ctypes.POINTER(_P)]),
    "moe_pool_fetch": (ctypes.c_int, [_P, _P, _I64, _P, ctypes.POINTER(_I32)]),
    "moe_pool_stats": (ctypes.c_int, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "moe_pool_destroy": (ctypes.c_int, [_P]),
    "moe_workspace_status": (ctypes.c_int, [_P, _U64, _P]),
    "moe_layer_scratch": (ctypes.c_int, [_DESC, _P, _I64, _P, _P, _P, _P, _I32, _P]),
    "moe_mfma_rate": (ctypes.c_int, [_I32, _I32, _I64, _I32, _P, _P]),
    "moe_set_wait_limit": (ctypes.c_int, [_I64]),
    "moe_workspace_region": (ctypes.c_int, [_DESC, _I64, _I32, ctypes.POINTER(_U64),
                                            ctypes.POINTER(_U64)]),
}


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mxfp4_routed_expert_x896_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        ver = lib.moe_abi_version()
        if ver >> 16 != ABI_MAJOR:
            raise ImportError(f"library ABI {ver >> 16}.{ver & 0xFFFF}, binding expects {ABI_MAJOR}.x")
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises ImportError when not built)."""
    return _lib()


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def record_bytes(hidden, inter):
    out = _U64()
    _check(_lib().moe_record_bytes(hidden, inter, ctypes.byref(out)), "moe_record_bytes")
    return out.value


def packed_record_bytes(hidden, inter):
    out = _U64()
    _check(_lib().moe_packed_record_bytes(hidden, inter, ctypes.byref(out)),
           "moe_packed_record_bytes")
    return out.value


def pack_experts(src, n_experts, hidden, inter, dst=None, stream=None):
    """Canonical uint8 records [E, record_bytes] -> packed uint8 [E, packed_bytes]."""
    pb = packed_record_bytes(hidden, inter)
    if dst is None:
        dst = torch.empty((n_experts, pb), dtype=torch.uint8, device=src.device)
    src_stride = src.numel() // n_experts
    _check(_lib().moe_pack_experts(_ptr(src), src_stride, _ptr(dst), dst.numel() // n_experts,
                                   n_experts, hidden, inter, _stream(stream)), "moe_pack_experts")
    return dst


def pack_bf16(src, stream=None):
    """Row-major bf16 matrices [count, rows, cols] (int16/bf16) -> packed, same shape."""
    count, rows, cols = src.shape
    dst = torch.empty_like(src)
    _check(_lib().moe_pack_bf16(_ptr(src), _ptr(dst), count, rows, cols, _stream(stream)),
           "moe_pack_bf16")
    return dst


def mfma_min_tokens():
    return _lib().moe_mfma_min_tokens()


class Layer:
    """Device tensors of one MoE layer plus the C descriptor that points at them.

    router_w: bf16/uint16-viewable [E, H]; experts: PACKED uint8 records
    [E, stride] (pack_experts); shared_*: PACKED bf16 [S, I, H] / [S, H, I]
    (pack_bf16) or None; router_bias: fp32 [E] or None; router_mode:
    ROUTER_BIAS_LOGITS or ROUTER_BIAS_SELECT (where the bias enters);
    routed_scale: factor on the combine weights.
    """

    def __init__(self, hidden, inter, n_experts, top_k, router_w, experts,
                 shared_gate=None, shared_up=None, shared_down=None, router_bias=None,
                 expert_stride=None, pool=None, router_mode=0, routed_scale=1.0):
        self.hidden, self.inter = int(hidden), int(inter)
        self.n_experts, self.top_k = int(n_experts), int(top_k)
        self.router_w = router_w
        self.experts = experts
        self.shared_gate, self.shared_up, self.shared_down = shared_gate, shared_up, shared_down
        self.router_bias = router_bias
        self.n_shared = 0 if shared_gate is None else int(shared_gate.shape[0])
        stride = expert_stride if expert_stride is not None else packed_record_bytes(hidden, inter)
        self.expert_stride = int(stride)
        self._desc = LayerDesc(
            self.hidden, self.inter, self.n_experts, self.top_k, self.n_shared, int(router_mode),
            router_w.data_ptr(),
            None if router_bias is None else router_bias.data_ptr(),
            experts.data_ptr(), self.expert_stride,
            None if shared_gate is None else shared_gate.data_ptr(),
            None if shared_up is None else shared_up.data_ptr(),
            None if shared_down is None else shared_down.data_ptr(),
            None if pool is None else pool.slot_map.data_ptr(),
            0 if pool is None else pool.n_slots, float(routed_scale))
        self.pool = pool

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def workspace_bytes(self, n_tokens):
        out = _U64()
        _check(_lib().moe_workspace_bytes(self.desc, n_tokens, ctypes.byref(out)),
               "moe_workspace_bytes")
        return out.value

    @classmethod
    def from_canonical(cls, hidden, inter, n_experts, top_k, router_w, experts,
                       shared_gate=None, shared_up=None, shared_down=None, router_bias=None,
                       **kw):
        """Packs canonical expert records and row-major shared matrices first."""
        packed = pack_experts(experts, n_experts, hidden, inter)
        sg = None if shared_gate is None else pack_bf16(shared_gate)
        su = None if shared_up is None else pack_bf16(shared_up)
        sd = None if shared_down is None else pack_bf16(shared_down)
        return cls(hidden, inter, n_experts, top_k, router_w, packed, sg, su, sd, router_bias, **kw)

    def workspace(self, n_tokens, device=None):
        dev = device if device is not None else self.router_w.device
        return torch.empty(self.workspace_bytes(n_tokens), dtype=torch.uint8, device=dev)


class ExpertPool:
    """HBM slots for n_slots of the E packed records, filled on demand from
    host memory (moe_pool_*).  host_records: packed uint8 [E, stride] in
    host memory (pinned for asynchronous copies); the slots and the slot map
    are allocated here on `device`.  Layer(..., experts=pool.slots,
    pool=pool) runs on the resident records."""

    def __init__(self, host_records, n_slots, device="cuda", stream=None):
        self.host = host_records
        self.n_experts, self.stride = int(host_records.shape[0]), int(host_records.shape[1])
        self.n_slots = int(n_slots)
        self.slots = torch.empty((self.n_slots, self.stride), dtype=torch.uint8, device=device)
        self.slot_map = torch.empty(self.n_experts, dtype=torch.int32, device=device)
        h = _P()
        _check(_lib().moe_pool_create(host_records.data_ptr(), self.stride, self.n_experts,
                                      self.slots.data_ptr(), self.n_slots,
                                      self.slot_map.data_ptr(), _stream(stream), ctypes.byref(h)),
               "moe_pool_create")
        self._h = h

    def fetch(self, ids, stream=None):
        """Makes the experts in ids (host int32 array-like) resident; returns
        how many records were copied."""
        import numpy as np
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
        n = _I32()
        _check(_lib().moe_pool_fetch(self._h, a.ctypes.data, a.size, _stream(stream),
                                     ctypes.byref(n)), "moe_pool_fetch")
        return n.value

    def stats(self):
        c, r = _I64(), _I64()
        _check(_lib().moe_pool_stats(self._h, ctypes.byref(c), ctypes.byref(r)), "moe_pool_stats")
        return c.value, r.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _LIB is not None:
            _LIB.moe_pool_destroy(h)
            self._h = None


def route(layer, x, topk_ids, topk_w, ws, stream=None):
    _check(_lib().moe_route(layer.desc, _ptr(x), x.shape[0], _ptr(topk_ids), _ptr(topk_w),
                            _ptr(ws), ws.numel(), _stream(stream)), "moe_route")


def forward(layer, x, topk_ids, topk_w, y, ws, residual=None, path=PATH_AUTO, stream=None):
    _check(_lib().moe_forward(layer.desc, _ptr(x), x.shape[0], _ptr(topk_ids), _ptr(topk_w),
                              _ptr(residual), _ptr(y), path, _ptr(ws), ws.numel(),
                              _stream(stream)), "moe_forward")


def forward_pooled(layer, x, topk_ids, topk_w, y, ws, records_ready, residual=None,
                   path=PATH_AUTO, stream=None):
    """forward whose routed part waits for records_ready (a torch.cuda.Event
    recorded after the pool's fetch on another stream); the shared experts
    run before the wait."""
    ev = None if records_ready is None else ctypes.c_void_p(records_ready.cuda_event)
    _check(_lib().moe_forward_pooled(layer.desc, _ptr(x), x.shape[0], _ptr(topk_ids),
                                     _ptr(topk_w), _ptr(residual), _ptr(y), path, _ptr(ws),
                                     ws.numel(), ev, _stream(stream)), "moe_forward_pooled")


def moe_layer(layer, x, y, topk_ids, topk_w, ws, residual=None, path=PATH_AUTO, stream=None):
    _check(_lib().moe_layer(layer.desc, _ptr(x), x.shape[0], _ptr(residual), _ptr(y),
                            _ptr(topk_ids), _ptr(topk_w), path, _ptr(ws), ws.numel(),
                            _stream(stream)), "moe_layer")


def moe_layer_scratch(layer, x, y, topk_ids, topk_w, residual=None, path=PATH_AUTO, stream=None):
    """moe_layer on the library's static per-device scratch (no workspace)."""
    _check(_lib().moe_layer_scratch(layer.desc, _ptr(x), x.shape[0], _ptr(residual), _ptr(y),
                                    _ptr(topk_ids), _ptr(topk_w), path, _stream(stream)),
           "moe_layer_scratch")


def rmsnorm(x, gamma, eps, out, stream=None):
    _check(_lib().moe_rmsnorm(_ptr(x), _ptr(gamma), ctypes.c_float(eps), x.shape[0],
                              x.shape[1], _ptr(out), _stream(stream)), "moe_rmsnorm")


def dequant_export(layer, expert, matrix, out, stream=None):
    _check(_lib().moe_dequant_export(layer.desc, expert, matrix, _ptr(out), _stream(stream)),
           "moe_dequant_export")


def profile_events(event_array, n):
    """Register an array of n hipEvent_t handles (ctypes array) for per-kernel
    timing on this host thread; pass None to stop."""
    _check(_lib().moe_profile_events(event_array, n if event_array is not None else 0),
           "moe_profile_events")


def profile_count():
    return _lib().moe_profile_count()


def mxfp8_quantize(x, codes, scales, stream=None):
    _check(_lib().moe_mxfp8_quantize(_ptr(x), x.shape[0], x.shape[1], _ptr(codes),
                                     _ptr(scales), _stream(stream)), "moe_mxfp8_quantize")


def int8_row_dequant(q, scale, out, stream=None):
    """out[r][c] = q[r][c] * scale[r] (int8 [R, C], fp32 [R] -> fp32 [R, C])."""
    _check(_lib().moe_int8_row_dequant(_ptr(q), _ptr(scale), q.shape[0], q.shape[1], _ptr(out),
                                       _stream(stream)), "moe_int8_row_dequant")


def workspace_status(ws, stream=None):
    """MOE_OK, or MOE_ETIMEOUT if a top-k wait of a call on ws gave up since
    the last query (synchronises the stream; clears the marker)."""
    st = _lib().moe_workspace_status(_ptr(ws), ws.numel(), _stream(stream))
    if st not in (MOE_OK, MOE_ETIMEOUT):
        _check(st, "moe_workspace_status")
    return st


def set_wait_limit(polls):
    """Polls before a top-k wait gives up (this host thread); -1: default."""
    _check(_lib().moe_set_wait_limit(int(polls)), "moe_set_wait_limit")


def workspace_region(layer, n_tokens, region, ws):
    """uint8 view of one region of a workspace tensor (test export)."""
    off, n = _U64(), _U64()
    _check(_lib().moe_workspace_region(layer.desc, n_tokens, region, ctypes.byref(off),
                                       ctypes.byref(n)), "moe_workspace_region")
    return ws[off.value:off.value + n.value]


def mfma_rate(a_fmt, b_fmt, iters, n_blocks, out, stream=None):
    """Block-scaled MFMA issue-rate launch (formats 4 = FP4, 0 = FP8)."""
    _check(_lib().moe_mfma_rate(a_fmt, b_fmt, iters, n_blocks, _ptr(out), _stream(stream)),
           "moe_mfma_rate")

"""moe_layer_scratch, the entry point that allocates nothing (its workspace
is the library's static per-device scratch array), against moe_layer with a
caller-allocated workspace: the same kernels, so every output, routing id
and weight must be identical bit for bit, on two calls in a row with the
second smaller than the first (stale contents of the scratch from the
first call must not leak into the second).  Also: a call too large for the
scratch is refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import synth
import synth.device as SD
from tests._gpu import Built, to_np_u16

pytestmark = pytest.mark.gpu

MID = dict(hidden=1024, inter=512, n_experts=64, top_k=8, n_shared=2)


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def _outs(T, k, H):
    return (torch.empty((T, H), dtype=torch.int16, device="cuda"),
            torch.empty((T, k), dtype=torch.int32, device="cuda"),
            torch.empty((T, k), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_scratch_entry_equals_workspace_entry(b, path):
    built = Built(MID, seed=70, bias=True)
    H, k = MID["hidden"], MID["top_k"]
    p = b.PATH_GEMV if path == "gemv" else b.PATH_MFMA
    for i, T in enumerate([9, 3, 1] if path == "gemv" else [300, 40]):
        xh, xd = SD.upload_tokens(7000 + 10 * i + p, T, H)
        rh, rd = SD.upload_tokens(7100 + 10 * i + p, T, H)
        y1, i1, w1 = _outs(T, k, H)
        y2, i2, w2 = _outs(T, k, H)
        b.moe_layer_scratch(built.lib, xd, y1, i1, w1, residual=rd, path=p)
        b.moe_layer(built.lib, xd, y2, i2, w2, built.lib.workspace(T), residual=rd, path=p)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(i1.cpu().numpy(), i2.cpu().numpy())
        np.testing.assert_array_equal(w1.cpu().numpy().view(np.uint32),
                                      w2.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(to_np_u16(y1), to_np_u16(y2))


def test_scratch_entry_refuses_a_workspace_beyond_its_size(b):
    built = Built(synth.TINY, seed=71)
    T = 1 << 16
    assert built.lib.workspace_bytes(T) > (64 << 20)
    P = ctypes.c_void_p
    st = b.lib().moe_layer_scratch(built.lib.desc, P(0x100000), T, None, P(0x200000),
                                   P(0x300000), P(0x400000), b.PATH_GEMV, None)
    assert st == -4  # MOE_EWORKSPACE, nothing launched

"""GPU parity of the row-scaled int8 -> fp32 expansion against the oracle,
bit for bit (one fp32 rounding of an exact product on both sides), through
the C ABI: ragged widths around the 1024-element chunk a workgroup takes,
IEEE special values, and the benchmark's size on sampled rows.
"""

import numpy as np
import pytest
import torch

from oracle import spine as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def _inputs(seed, rows, cols):
    rng = np.random.default_rng(seed)
    q = rng.integers(-128, 128, size=(rows, cols), dtype=np.int16).astype(np.int8)
    # row scales like a symmetric int8 quantiser's: amax / 127 of N(0, 0.02) rows
    scale = (np.abs(rng.standard_normal(rows)) * 0.02 * 4 / 127 + 1e-6).astype(np.float32)
    return q, scale


def _run(b, q, scale):
    qd = torch.from_numpy(q).cuda()
    sd = torch.from_numpy(scale).cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    b.int8_row_dequant(qd, sd, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("rows,cols", [(1, 4), (3, 12), (4, 1020), (5, 1028), (3, 2044), (7, 4096), (2, 4100),
                                       (9, 8188), (300, 7168), (64, 12292)])
def test_bit_exact(b, rows, cols):
    q, scale = _inputs(rows * 7 + cols, rows, cols)
    got = _run(b, q, scale)
    want = S.int8_row_dequant(q, scale)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_special_scales(b):
    q = np.tile(np.array([0, 1, -1, 127, -128, 3, -77, 5], dtype=np.int8), (8, 16))  # 8 x 128
    scale = np.array([-2.0, 3.0e38, np.inf, -np.inf, np.nan, 1e-40, -0.0, 1.0], dtype=np.float32)
    got = _run(b, q, scale)
    want = S.int8_row_dequant(q, scale)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_bench_size_sampled_rows(b):
    """32768 x 7168 (235 MB int8 -> 940 MB fp32): 40 rows checked."""
    rows, cols = 32768, 7168
    g = torch.Generator(device="cuda").manual_seed(11)
    qd = torch.randint(-128, 128, (rows, cols), dtype=torch.int8, device="cuda", generator=g)
    sd = (torch.rand(rows, device="cuda", generator=g) * 1e-3 + 1e-5).float()
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    b.int8_row_dequant(qd, sd, out)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, 1, rows - 1], np.random.default_rng(1).integers(0, rows, 37)]))
    q = qd[pick].cpu().numpy()
    want = S.int8_row_dequant(q, sd[pick].cpu().numpy())
    np.testing.assert_array_equal(out[pick].cpu().numpy().view(np.uint32), want.view(np.uint32))

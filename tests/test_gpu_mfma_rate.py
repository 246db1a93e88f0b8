"""The MFMA issue-rate diagnostic (moe_mfma_rate) runs for every supported
format pair and returns finite, reproducible checksums; the two FP4 operand
readings give different sums (the format argument reaches the instruction)."""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from mxfp4_routed_expert_x896_amd import binding
    return binding


def test_rate_kernel_formats(b):
    outs = {}
    for af, bf in ((4, 4), (4, 0), (0, 0)):
        o1 = torch.empty(8 * 4, dtype=torch.float32, device="cuda")
        o2 = torch.empty_like(o1)
        b.mfma_rate(af, bf, 3, 8, o1)
        b.mfma_rate(af, bf, 3, 8, o2)
        torch.cuda.synchronize()
        assert torch.isfinite(o1).all() and torch.equal(o1, o2)
        outs[(af, bf)] = o1.cpu()
    assert not torch.equal(outs[(4, 4)], outs[(4, 0)])

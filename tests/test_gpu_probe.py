"""The matrix-core rate probe (a diagnostic beside the method): it runs,
writes finite values, and two runs agree bit for bit."""
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_mfma_loop_probe(smoe):
    say("mfma loop probe")
    out1 = torch.empty(16 * 256, dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out1)
    smoe.smoe_probe_mfma_loop(out1, 16, 50)
    smoe.smoe_probe_mfma_loop(out2, 16, 50)
    torch.cuda.synchronize()
    assert torch.isfinite(out1).all()
    assert torch.equal(out1, out2)
    assert out1.abs().sum() > 0

"""The sustained-MFMA-ceiling probe (a measurement kernel, not part of the
loss) runs through the C ABI: zero operands give exactly zero, random
operands finite, nonzero sums."""
import pytest

from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_zero_operands_give_zero():
    import torch
    import chunked_top_kl_lm_amd as kd
    log("[gpu-probe] MFMA ceiling probe")
    out = torch.full((8 * 512,), -1.0, dtype=torch.float32, device="cuda:0")
    kd.mfma_probe(out, 8, 4, zero_operands=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    kd.mfma_probe(out, 8, 4)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and torch.count_nonzero(out).item() > 0

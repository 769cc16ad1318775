"""The Python binding rejects, on the host, arguments the library would
dereference on the wrong device or misread: CPU tensors, mismatched
dtypes and shapes, a non-byte workspace."""
import pytest
import torch

import chunked_top_kl_lm_amd as kd


def _cpu_inputs(T=8, d=16, V=32, K=4):
    return (torch.zeros((T, d), dtype=torch.bfloat16), torch.zeros((V, d), dtype=torch.bfloat16),
            torch.zeros((T, K), dtype=torch.int32), torch.zeros((T, K), dtype=torch.float32),
            torch.ones(T, dtype=torch.uint8))


@pytest.mark.parametrize("entry", ["fwd_bwd", "fwd", "bwd"])
def test_cpu_tensors_are_rejected(entry):
    h, w, idx, logit, mask = _cpu_inputs()
    with pytest.raises(ValueError, match="CUDA"):
        if entry == "fwd_bwd":
            kd.fwd_bwd(h, w, idx, logit, mask)
        elif entry == "fwd":
            kd.fwd(h, w, idx, logit, mask)
        else:
            kd.bwd(h, w, idx, logit, mask, torch.zeros(8))


def test_topk_cache_and_probe_reject_cpu_tensors():
    h, w, *_ = _cpu_inputs()
    with pytest.raises(ValueError, match="CUDA"):
        kd.topk_cache(h, w, K=4)
    with pytest.raises(ValueError, match="CUDA"):
        kd.mfma_probe(torch.zeros(512), 1, 1)


def test_workspace_and_status_types():
    with pytest.raises(ValueError, match="workspace"):
        kd._check_workspace(torch.zeros(16, dtype=torch.float32), None)
    with pytest.raises(ValueError, match="status"):
        kd._check_workspace(None, torch.zeros(1, dtype=torch.int64))
    kd._check_workspace(torch.zeros(16, dtype=torch.uint8), torch.zeros(1, dtype=torch.int32))


def test_event_count_is_checked_before_the_call():
    """The timed entry points record into 2 * (phases * nchunks + extra)
    caller events; a shorter list would make the library read past it."""
    class Ev:
        cuda_event = 0
    assert kd._nchunks(10, 4) == 3 and kd._nchunks(10, 64) == 1 and kd._nchunks(4096, 1024) == 4
    with pytest.raises(ValueError, match="expected 52"):
        kd._loss_events([Ev()] * 51, 10, 4)
    with pytest.raises(ValueError, match="expected 52"):
        kd._loss_events([Ev()] * 53, 10, 4)
    assert len(kd._loss_events([Ev()] * 52, 10, 4)) == 52
    need = 2 * (kd.KD_CACHE_PHASES * 3 + 1)
    with pytest.raises(ValueError, match=f"expected {need}"):
        kd._events([Ev()] * (need - 1), need)

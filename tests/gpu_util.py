"""Helpers shared by the GPU tests: move seeded inputs to the device, call the
HIP library through its binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

from datagen import to_device  # noqa: F401  (re-exported for the tests)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(x: dict, chunk: int | None = None, tau: float | None = None, row_stats=True, status=False):
    """One call of the HIP path; returns numpy results (and device status)."""
    import torch
    import chunked_top_kl_lm_amd as kd
    t = to_device(x)
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0") if status else None
    out = kd.fwd_bwd(t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"],
                     tau=x["tau"] if tau is None else tau,
                     chunk=x["chunk"] if chunk is None else chunk, row_stats=row_stats, status=st)
    torch.cuda.synchronize()
    res = dict(loss=float(out[0].item()), grad_hidden=out[1].cpu().numpy(),
               grad_W=out[2].cpu().numpy())
    if row_stats:
        res["row_lse"] = out[3].cpu().numpy()
        res["row_kl"] = out[4].cpu().numpy()
    if status:
        res["status"] = int(st.item())
    return res


def rel_f(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def rel(a: float, b: float) -> float:
    return abs(a - b) / abs(b) if b != 0 else abs(a)


# Acceptance bounds: loss relative error and relative Frobenius error of each
# gradient.  Derivation: the kernels multiply bf16 inputs exactly and sum in
# fp32 (relative error ~1e-6 on each logit), so the loss (an fp64 sum of fp32
# row terms) sits far inside 1e-3; the logit gradient G is rounded to bf16
# (relative 2^-9 per element) before the two gradient GEMMs, so each gradient
# carries ~2e-3 relative error, an order of magnitude inside 2e-2.
LOSS_TOL = 1e-3
GRAD_TOL = 2e-2

# Per-row statistics (returned through row_lse / row_kl): |LSE_gpu - LSE| <=
# ROW_LSE_TOL nats and |KL_gpu - KL| <= ROW_KL_TOL * max(1, |KL|).  Each is a
# logsumexp of, or a difference between, logits carrying the fp32 summation
# error above (~1e-6 relative, measured |dLSE| <= 2e-6 at d = 2880); the bar
# is the loss bar applied row by row, so a wrong row cannot hide in the mean.
ROW_LSE_TOL = 1e-3
ROW_KL_TOL = 1e-3


def row_errors(g_lse, g_kl, r_lse, r_kl):
    """(max |dLSE|, max |dKL| / max(1, |KL|)) over the rows given."""
    e_lse = float(np.max(np.abs(np.asarray(g_lse, np.float64) - r_lse))) if len(r_lse) else 0.0
    e_kl = float(np.max(np.abs(np.asarray(g_kl, np.float64) - r_kl) / np.maximum(1.0, np.abs(r_kl)))) \
        if len(r_kl) else 0.0
    return e_lse, e_kl

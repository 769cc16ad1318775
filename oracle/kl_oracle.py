"""Plain fp64 CPU oracle for the fused chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library and never reads its outputs.

What it computes.  The pages describe a KL-divergence distillation loss in
which the student is trained against a cache of the teacher's top-100 logits
per position (Glonce, "Multiverse Computing cuts LLM distillation VRAM by 15x
with chunked KL loss", paragraph on Multiverse's two-part fix; epoka.news,
"Two systems changes ...", section "The two proposed changes").  The pages
give no formula; the reading adopted here is:

  S[t,v]      = (h_t . W_v) / tau                      all v in [0, V)
  log q[t,v]  = S[t,v] - logsumexp_v S[t,:]            full-vocabulary student
  p[t,k]      = softmax_k(teacher_logit[t,:] / tau)    renormalised over K ids
  KL_t        = sum_k p[t,k] (log p[t,k] - log q[t, idx[t,k]])   (0 log 0 = 0)
  N           = number of positions with mask != 0
  loss        = tau^2 * sum_t m_t KL_t / N             (N = 0 gives loss 0)

and its exact gradient with respect to the logits z = S*tau,
  G[t,v] = (tau / N) m_t (q[t,v] - P[t,v]),  P[t,v] = sum_k p[t,k] [idx[t,k]=v]
(duplicate ids add), followed by grad_hidden = G W and grad_W = G^T H.

The fused method reaches exactly this result (up to rounding order): it only
avoids storing the T x V logits grid by working one sequence chunk at a time
and recomputing in the backward pass (Glonce, same paragraph).  So the oracle
is the plain definition: a dense, unchunked log-softmax over the whole
vocabulary.  Rows are independent, so the rows are processed in blocks to
bound host memory; blocking changes only the summation order of grad_W.

Ids outside [0, V) are the library's documented error case: such an entry
contributes nothing (no loss term, no gradient), while p is still normalised
over all K logits of the row.

All inputs are upcast exactly to float64 (bfloat16 bit patterns are widened
bit-exactly, fp32 is exact in fp64).
"""
from __future__ import annotations

import numpy as np

__all__ = ["as_f64", "teacher_distribution", "student_lse", "fused_kl",
           "fused_kl_rows"]


def as_f64(x: np.ndarray, is_bf16_bits: bool | None = None) -> np.ndarray:
    """Exact float64 copy of fp32 data or of bfloat16 bit patterns (uint16)."""
    x = np.asarray(x)
    if is_bf16_bits is None:
        is_bf16_bits = x.dtype == np.uint16
    if is_bf16_bits:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def teacher_distribution(teacher_logit: np.ndarray, tau: float):
    """p = softmax over the K cached ids of teacher_logit / tau, and log p.

    The teacher's cached logits are renormalised over the K ids only (the
    cache holds just the top-K entries; Glonce, paragraph on the two-part fix).
    """
    a = np.asarray(teacher_logit, dtype=np.float64) / tau
    amax = a.max(axis=1, keepdims=True)
    log_z = amax + np.log(np.exp(a - amax).sum(axis=1, keepdims=True))
    log_p = a - log_z
    return np.exp(log_p), log_p


def student_lse(h_rows: np.ndarray, W: np.ndarray, tau: float):
    """Logits z = h W^T of a block of rows, S = z/tau, and logsumexp_v S."""
    z = h_rows @ W.T
    S = z / tau
    smax = S.max(axis=1, keepdims=True)
    lse = smax[:, 0] + np.log(np.exp(S - smax).sum(axis=1))
    return z, S, lse


def _row_terms(S, lse, idx_rows, p, log_p, V):
    """KL_t for a block of rows, from S, LSE and the teacher distribution."""
    valid = (idx_rows >= 0) & (idx_rows < V)
    safe = np.where(valid, idx_rows, 0)
    log_q_idx = np.take_along_axis(S, safe, axis=1) - lse[:, None]
    term = np.where(valid & (p > 0), p * (log_p - log_q_idx), 0.0)
    return term.sum(axis=1)


def _sparse_target(p, idx_rows, V):
    """P[t,v] = sum_k p[t,k] [idx[t,k] = v] over valid ids (duplicates add)."""
    P = np.zeros((idx_rows.shape[0], V), dtype=np.float64)
    valid = (idx_rows >= 0) & (idx_rows < V)
    rr, kk = np.nonzero(valid)
    np.add.at(P, (rr, idx_rows[rr, kk]), p[rr, kk])
    return P


def fused_kl(hidden, W, teacher_idx, teacher_logit, mask, tau,
             rows_per_block: int = 256, want_grads: bool = True):
    """Loss and gradients of the top-K KL distillation loss, in float64.

    hidden [T,d] and W [V,d] are fp32 arrays or bfloat16 bit patterns;
    teacher_idx [T,K] int; teacher_logit [T,K]; mask [T] (nonzero = counts)
    or None (all count); tau > 0.

    Returns dict(loss, grad_hidden [T,d], grad_W [V,d], row_kl [T], row_lse [T],
    N).  grad_* are None when want_grads is False.
    """
    H = as_f64(hidden)
    Wf = as_f64(W)
    idx = np.asarray(teacher_idx).astype(np.int64)
    T, d = H.shape
    V = Wf.shape[0]
    m = np.ones(T) if mask is None else (np.asarray(mask) != 0).astype(np.float64)
    N = int(m.sum())
    s = tau / N if N > 0 else 0.0

    p, log_p = teacher_distribution(teacher_logit, tau)
    row_kl = np.zeros(T)
    row_lse = np.zeros(T)
    gH = np.zeros((T, d)) if want_grads else None
    gW = np.zeros((V, d)) if want_grads else None

    for r0 in range(0, T, rows_per_block):
        r1 = min(T, r0 + rows_per_block)
        z, S, lse = student_lse(H[r0:r1], Wf, tau)
        row_lse[r0:r1] = lse
        row_kl[r0:r1] = _row_terms(S, lse, idx[r0:r1], p[r0:r1], log_p[r0:r1], V)
        if want_grads:
            q = np.exp(S - lse[:, None])
            P = _sparse_target(p[r0:r1], idx[r0:r1], V)
            G = (s * m[r0:r1])[:, None] * (q - P)
            gH[r0:r1] = G @ Wf
            gW += G.T @ H[r0:r1]

    loss = tau * tau * float((m * row_kl).sum()) / N if N > 0 else 0.0
    return dict(loss=loss, grad_hidden=gH, grad_W=gW, row_kl=row_kl,
                row_lse=row_lse, N=N)


def fused_kl_rows(hidden, W, teacher_idx, teacher_logit, mask, tau, rows,
                  vocab_block: int = 16384):
    """Per-row results for selected rows only, at any T.

    For each row t in `rows`: LSE_t, KL_t and grad_hidden[t] (which needs only
    row t's logits and the global count N).  W is upcast in blocks of
    `vocab_block` rows so that full-vocabulary rows fit in host memory.
    Returns dict(row_lse, row_kl, grad_hidden_rows [len(rows), d], N).
    """
    rows = np.asarray(rows, dtype=np.int64)
    H = as_f64(np.asarray(hidden)[rows])
    idx = np.asarray(teacher_idx)[rows].astype(np.int64)
    V = np.asarray(W).shape[0]
    mask_all = None if mask is None else np.asarray(mask)
    T = np.asarray(hidden).shape[0]
    m_all = np.ones(T) if mask_all is None else (mask_all != 0).astype(np.float64)
    N = int(m_all.sum())
    s = tau / N if N > 0 else 0.0
    m = m_all[rows]

    z = np.empty((rows.size, V))
    for v0 in range(0, V, vocab_block):
        z[:, v0:v0 + vocab_block] = H @ as_f64(np.asarray(W)[v0:v0 + vocab_block]).T
    S = z / tau
    smax = S.max(axis=1, keepdims=True)
    lse = smax[:, 0] + np.log(np.exp(S - smax).sum(axis=1))
    p, log_p = teacher_distribution(np.asarray(teacher_logit)[rows], tau)
    kl = _row_terms(S, lse, idx, p, log_p, V)

    q = np.exp(S - lse[:, None])
    G = (s * m)[:, None] * (q - _sparse_target(p, idx, V))
    gH = np.zeros((rows.size, H.shape[1]))
    for v0 in range(0, V, vocab_block):
        gH += G[:, v0:v0 + vocab_block] @ as_f64(np.asarray(W)[v0:v0 + vocab_block])
    return dict(row_lse=lse, row_kl=kl, grad_hidden_rows=gH, N=N)

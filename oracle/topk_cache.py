"""Plain fp64 CPU oracle for the offline top-K teacher-logit cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
this module: only the tests and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library and never reads its outputs.

What it computes.  Before the student is trained, the teacher runs once and
the K largest of its output logits at every position are stored with their
token ids; training then reads that record instead of running the teacher
(Glonce, "Multiverse Computing cuts LLM distillation VRAM by 15x with chunked
KL loss", paragraph on Multiverse's two-part fix: the top 100 per position;
ainewsbank.com, "Multiverse Computing Tests Lower-Memory Long-Context
Distillation", section "Two changes remove different bottlenecks"; epoka.news,
"Two systems changes that cut the cost of knowledge distillation", section
"The two proposed changes").  With the teacher's final hidden states H [T, d]
and output head W [V, d]:

  z[t, v]  = h_t . W_v                                  all v in [0, V)
  cache_t  = the K ids with the largest z[t, :], in descending order of z,
             equal logits ordered by the lower id first
  outputs    idx [T, K] (int32) and the logits z[t, idx] (float64 here)

The pages do not say how equal logits are ordered; the reading used is the
lower id first, which makes the record unique.  Rows are independent and are
processed in blocks to bound host memory.
"""
from __future__ import annotations

import numpy as np

from .kl_oracle import as_f64

__all__ = ["topk_cache", "teacher_logits"]


def teacher_logits(hidden, W, rows=None) -> np.ndarray:
    """z = H W^T in float64 (for the given rows, default all)."""
    H = as_f64(hidden)
    if rows is not None:
        H = H[np.asarray(rows)]
    return H @ as_f64(W).T


def topk_cache(hidden, W, K: int, rows_per_block: int = 256):
    """(idx [T, K] int32, logit [T, K] float64): the K largest logits per row,
    descending, ties by the lower id."""
    Wd = as_f64(W)
    T = np.asarray(hidden).shape[0]
    V = Wd.shape[0]
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    idx = np.empty((T, K), dtype=np.int32)
    val = np.empty((T, K), dtype=np.float64)
    ids = np.arange(V)
    for r0 in range(0, T, rows_per_block):
        z = as_f64(np.asarray(hidden)[r0:r0 + rows_per_block]) @ Wd.T
        for i, row in enumerate(z):
            order = np.lexsort((ids, -row))[:K]      # primary: z descending; then id ascending
            idx[r0 + i] = order
            val[r0 + i] = row[order]
    return idx, val

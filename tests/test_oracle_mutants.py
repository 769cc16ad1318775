"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch them.

Each mutant replaces one helper of the oracle module with a subtly wrong
version (a dropped term, a wrong sign, a missing tau, duplicates not added,
wrong normaliser).  The pin tests of test_oracle_pins must then fail for at
least one of their cases.
"""
import numpy as np
import pytest

import oracle.kl_oracle as ok
import tests.test_oracle_pins as pins


def _teacher_no_tau(teacher_logit, tau):
    return ok.__dict__["_orig_teacher"](teacher_logit, 1.0)


def _student_no_tau(h_rows, W, tau):
    return ok.__dict__["_orig_student"](h_rows, W, 1.0)


def _row_terms_no_logp(S, lse, idx_rows, p, log_p, V):
    return ok.__dict__["_orig_rows"](S, lse, idx_rows, p, np.zeros_like(log_p), V)


def _row_terms_sign(S, lse, idx_rows, p, log_p, V):
    return -ok.__dict__["_orig_rows"](S, lse, idx_rows, p, log_p, V)


def _sparse_assign(p, idx_rows, V):
    P = np.zeros((idx_rows.shape[0], V))
    valid = (idx_rows >= 0) & (idx_rows < V)
    rr, kk = np.nonzero(valid)
    P[rr, idx_rows[rr, kk]] = p[rr, kk]          # duplicates overwrite instead of add
    return P


def _sparse_sign(p, idx_rows, V):
    return -ok.__dict__["_orig_sparse"](p, idx_rows, V)


def _student_lse_off_by_max(h_rows, W, tau):
    z, S, lse = ok.__dict__["_orig_student"](h_rows, W, tau)
    return z, S, S.max(axis=1)                   # max instead of logsumexp


MUTANTS = {
    "teacher softmax ignores tau": ("teacher_distribution", _teacher_no_tau),
    "student logits not divided by tau": ("student_lse", _student_no_tau),
    "KL drops the log p term": ("_row_terms", _row_terms_no_logp),
    "KL sign flipped": ("_row_terms", _row_terms_sign),
    "duplicate ids overwrite": ("_sparse_target", _sparse_assign),
    "sparse target sign flipped": ("_sparse_target", _sparse_sign),
    "LSE replaced by max": ("student_lse", _student_lse_off_by_max),
}

PIN_CASES = [
    lambda: pins.test_finite_differences_tiny(2.0),
    lambda: pins.test_kl_zero_limit_closed_form(2.0),
    lambda: pins.test_zero_head_equal_logits_gives_log_v_over_k(),
    lambda: pins.test_k1_is_masked_cross_entropy(3.0),
    lambda: pins.test_k_equals_v_is_full_kl_scipy(2.0),
    lambda: pins.test_tau_homogeneity(),
    lambda: pins.test_invariants(),
]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(ok.__dict__, "_orig_teacher", ok.teacher_distribution)
    monkeypatch.setitem(ok.__dict__, "_orig_student", ok.student_lse)
    monkeypatch.setitem(ok.__dict__, "_orig_rows", ok._row_terms)
    monkeypatch.setitem(ok.__dict__, "_orig_sparse", ok._sparse_target)
    monkeypatch.setattr(ok, attr, fn)
    caught = 0
    for case in PIN_CASES:
        try:
            case()
        except (AssertionError, FloatingPointError, ValueError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant: {name}"

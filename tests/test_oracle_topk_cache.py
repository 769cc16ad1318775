"""Pins of the top-K cache oracle to facts other than its own code.

The brute force re-derives every cache entry with exact sums (math.fsum) and
a plain Python sort; the planted heads give logits whose order is known in
closed form (increasing, decreasing, all equal); K = V must return a
permutation of every id.  A sort in the wrong direction, ties broken by the
higher id, an off-by-one in K or a transposed product fails one of them.
"""
import math

import numpy as np
import pytest

from oracle import topk_cache


@pytest.mark.parametrize("T,d,V,K", [(5, 4, 30, 7), (3, 6, 64, 64), (4, 3, 17, 1), (6, 5, 40, 12)])
def test_brute_force(T, d, V, K):
    rng = np.random.default_rng(T * 100 + V)
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((V, d))
    W[3] = W[5]                        # an exact tie between ids 3 and 5
    idx, val = topk_cache(H, W, K)
    for t in range(T):
        z = [math.fsum(H[t, j] * W[v, j] for j in range(d)) for v in range(V)]
        want = sorted(range(V), key=lambda v: (-z[v], v))[:K]
        assert idx[t].tolist() == want
        assert np.allclose(val[t], [z[v] for v in want], rtol=1e-12, atol=1e-12)


def test_planted_order():
    T, d, V, K = 4, 3, 50, 10
    W = np.zeros((V, d))
    W[:, 0] = np.arange(1, V + 1)      # z[t, v] = h[t, 0] * (v + 1)
    H = np.zeros((T, d))
    H[:, 0] = [2.0, -1.0, 0.5, -3.0]
    idx, val = topk_cache(H, W, K)
    assert idx[0].tolist() == list(range(V - 1, V - 1 - K, -1))   # positive scale: largest ids
    assert idx[2].tolist() == list(range(V - 1, V - 1 - K, -1))
    assert idx[1].tolist() == list(range(K))                      # negative scale: smallest ids
    assert idx[3].tolist() == list(range(K))
    assert np.allclose(val[0], 2.0 * (idx[0] + 1)) and np.allclose(val[3], -3.0 * (idx[3] + 1))


def test_all_equal_logits_take_the_lowest_ids():
    T, d, V, K = 3, 4, 25, 6
    W = np.ones((V, d))
    H = np.random.default_rng(1).standard_normal((T, d))
    idx, val = topk_cache(H, W, K)
    assert np.all(idx == np.arange(K))
    assert np.allclose(val, H.sum(1, keepdims=True))


def test_k_equals_v_is_a_sorted_permutation():
    rng = np.random.default_rng(2)
    H, W = rng.standard_normal((3, 5)), rng.standard_normal((20, 5))
    idx, val = topk_cache(H, W, 20)
    for t in range(3):
        assert sorted(idx[t].tolist()) == list(range(20))
        assert np.all(np.diff(val[t]) <= 0)


def test_row_blocking_does_not_change_the_result():
    rng = np.random.default_rng(3)
    H, W = rng.standard_normal((37, 8)), rng.standard_normal((300, 8))
    a = topk_cache(H, W, 16, rows_per_block=1)
    b = topk_cache(H, W, 16, rows_per_block=256)
    # BLAS may sum a 1-row block in another order: values agree to rounding
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], rtol=1e-13, atol=1e-13)


def test_bf16_bits_are_widened_exactly():
    # 1.5 and -2.0 in bf16 bits; z = 1.5 * -2.0 = -3.0 exactly
    H = np.array([[0x3FC0]], dtype=np.uint16)
    W = np.array([[0xC000], [0x3F80]], dtype=np.uint16)   # -2.0, 1.0
    idx, val = topk_cache(H, W, 2)
    assert idx.tolist() == [[1, 0]] and val.tolist() == [[1.5, -3.0]]


# ---------------------------------------------------------------------------
# teacher_logits: the fp64 logits the cache builder's GPU checks compare to.
# Pinned by an exact brute force (math.fsum over exactly widened inputs, the
# bf16 widening written out here with struct, independent of the oracle's
# own conversion), for fp32 and bf16-bit inputs and the `rows` selection;
# planted mistakes (a transposed product, bf16 bits read as integers, rows
# ignored) must fail it.
# ---------------------------------------------------------------------------
import importlib
import struct

from oracle import teacher_logits

otc = importlib.import_module("oracle.topk_cache")   # the module (the package re-exports a function of that name)


def _widen_bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _brute_logits(H, W, rows, bf16: bool):
    conv = _widen_bf16 if bf16 else float
    out = []
    for t in rows:
        h = [conv(v) for v in H[t]]
        out.append([math.fsum(h[j] * conv(W[v][j]) for j in range(len(h))) for v in range(len(W))])
    return np.array(out)


def _pin_teacher_logits():
    rng = np.random.default_rng(17)
    T, d, V = 5, 7, 13
    Hf = rng.standard_normal((T, d)).astype(np.float32)
    Wf = rng.standard_normal((V, d)).astype(np.float32)
    z = teacher_logits(Hf, Wf)
    want = _brute_logits(Hf, Wf, range(T), bf16=False)
    assert z.shape == (T, V) and z.dtype == np.float64
    assert np.allclose(z, want, rtol=0, atol=1e-12 * np.abs(want).max())
    # bf16 bit patterns: every product of two bf16 values is exact in fp64
    Hb = (Hf.view(np.uint32) >> 16).astype(np.uint16)
    Wb = (Wf.view(np.uint32) >> 16).astype(np.uint16)
    zb = teacher_logits(Hb, Wb)
    wantb = _brute_logits(Hb, Wb, range(T), bf16=True)
    assert zb.shape == (T, V)
    assert np.allclose(zb, wantb, rtol=0, atol=1e-12 * np.abs(wantb).max())
    # rows: in the given order, repeats allowed
    rows = [3, 0, 3, 4]
    zr = teacher_logits(Hb, Wb, rows=rows)
    assert zr.shape == (len(rows), V)
    assert np.allclose(zr, wantb[rows], rtol=0, atol=1e-12 * np.abs(wantb).max())


def test_teacher_logits_exact_brute_force():
    _pin_teacher_logits()


def _transposed(hidden, W, rows=None):
    Hd = otc.as_f64(hidden)
    if rows is not None:
        Hd = Hd[np.asarray(rows)]
    return (Hd @ otc.as_f64(W).T).T


def _no_widening(x, is_bf16_bits=None):
    return np.asarray(x).astype(np.float64)        # bf16 bits read as integers


def _rows_ignored(hidden, W, rows=None):
    return otc.as_f64(hidden) @ otc.as_f64(W).T


@pytest.mark.parametrize("attr,fn", [("teacher_logits", _transposed), ("as_f64", _no_widening),
                                     ("teacher_logits", _rows_ignored)])
def test_teacher_logits_pin_catches_planted_mistakes(attr, fn, monkeypatch):
    import tests.test_oracle_topk_cache as me
    monkeypatch.setattr(otc, attr, fn)
    if attr == "teacher_logits":
        monkeypatch.setattr(me, "teacher_logits", fn)
    with pytest.raises(AssertionError):
        _pin_teacher_logits()

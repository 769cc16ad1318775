"""Pins of the fp64 oracle to facts other than its own formulas.

Each test targets a distinct plausible mistake in the oracle: finite
differences pin the gradient to the loss; the W = 0, K = 1, K = V and KL -> 0
cases pin the loss to closed forms or to independent library routines
(torch cross-entropy, scipy rel_entr); the invariants pin signs, indices and
the scaling by tau^2 and 1/N.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle import fused_kl, fused_kl_rows, teacher_distribution


def _rand_case(rng, T, d, V, K, tau, masked_rows=(), dup_row=None, scale=1.0):
    H = rng.standard_normal((T, d)) * scale
    W = rng.standard_normal((V, d)) * scale
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)])
    if dup_row is not None and K >= 2:
        idx[dup_row, 1] = idx[dup_row, 0]
    logit = -np.sort(-rng.standard_normal((T, K)) * 2.0, axis=1)
    mask = np.ones(T, dtype=np.uint8)
    for r in masked_rows:
        mask[r] = 0
    return H, W, idx.astype(np.int32), logit, mask, tau


# -- 1. finite differences ----------------------------------------------------

@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_finite_differences_tiny(tau):
    rng = np.random.default_rng(11)
    H, W, idx, logit, mask, tau = _rand_case(rng, 6, 5, 11, 3, tau,
                                             masked_rows=(2,), dup_row=4)
    ref = fused_kl(H, W, idx, logit, mask, tau, rows_per_block=4)

    def loss_at(H_, W_):
        return fused_kl(H_, W_, idx, logit, mask, tau, want_grads=False)["loss"]

    def fd(X, which):
        g = np.zeros_like(X)
        for i in np.ndindex(X.shape):
            step = 1e-5 * max(1.0, abs(X[i]))
            Xp = X.copy(); Xp[i] += step
            Xm = X.copy(); Xm[i] -= step
            lp = loss_at(Xp, W) if which == "H" else loss_at(H, Xp)
            lm = loss_at(Xm, W) if which == "H" else loss_at(H, Xm)
            g[i] = (lp - lm) / (2 * step)
        return g

    for which, X, g in (("H", H, ref["grad_hidden"]), ("W", W, ref["grad_W"])):
        num = fd(X, which)
        rel = np.linalg.norm(num - g) / np.linalg.norm(g)
        assert rel <= 1e-6, (which, rel)
        assert np.max(np.abs(num - g)) <= 1e-6 * np.max(np.abs(g)), which
    # the masked row's hidden gradient is exactly zero
    assert np.all(ref["grad_hidden"][2] == 0.0)


# -- 2. KL = 0 in the limit (closed form) ------------------------------------

@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_kl_zero_limit_closed_form(tau):
    rng = np.random.default_rng(5)
    T, V, K = 4, 13, 4
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    logit = -np.sort(-rng.standard_normal((T, K)) * 3.0, axis=1)
    c = rng.standard_normal(T)
    W = np.eye(V)                 # d = V, so z = h
    prev = None
    for Mmul in (5, 10, 20, 40):
        M = Mmul * tau
        H = np.full((T, V), -M)
        for t in range(T):
            H[t, idx[t]] = logit[t] + c[t]
        out = fused_kl(H, W, idx, logit, None, tau)
        # KL_t = log(1 + (V-K) e^{(-M-c_t)/tau} / sum_k e^{l_k/tau})
        want = np.array([math.log1p((V - K) * math.exp((-M - c[t]) / tau)
                                    / sum(math.exp(l / tau) for l in logit[t]))
                         for t in range(T)])
        np.testing.assert_allclose(out["row_kl"], want, rtol=1e-9, atol=1e-15)
        assert out["loss"] >= 0
        gnorm = np.linalg.norm(out["grad_hidden"])
        if prev is not None:
            assert out["loss"] < prev[0] and gnorm < prev[1]
        prev = (out["loss"], gnorm)
    assert prev[0] < 1e-12 * tau * tau
    assert prev[1] < 1e-12


# -- 3. chunk-size (row-block) invariance and the vocab-tiled LSE merge --------

def test_row_block_invariance():
    rng = np.random.default_rng(7)
    H, W, idx, logit, mask, tau = _rand_case(rng, 70, 9, 40, 5, 1.5,
                                             masked_rows=(3, 50), dup_row=9)
    outs = [fused_kl(H, W, idx, logit, mask, tau, rows_per_block=b) for b in (1, 3, 64, 70)]
    for o in outs[1:]:
        assert abs(o["loss"] - outs[0]["loss"]) <= 1e-12 * abs(outs[0]["loss"])
        for k in ("grad_hidden", "grad_W"):
            rel = np.linalg.norm(o[k] - outs[0][k]) / np.linalg.norm(outs[0][k])
            assert rel <= 1e-12, k


def _tiled_online_lse(S, tile):
    """Plain fp64 model of a vocabulary-tiled online logsumexp merge."""
    T, V = S.shape
    m = np.full(T, -np.inf)
    l = np.zeros(T)
    for v0 in range(0, V, tile):
        blk = S[:, v0:v0 + tile]
        bm = blk.max(axis=1)
        bl = np.exp(blk - bm[:, None]).sum(axis=1)
        M = np.maximum(m, bm)
        l = l * np.exp(m - M) + bl * np.exp(bm - M)
        m = M
    return m + np.log(l)


@pytest.mark.parametrize("tile", [1, 7, 128])
def test_vocab_tiled_lse_merge_equals_dense(tile):
    rng = np.random.default_rng(3)
    H, W, idx, logit, mask, tau = _rand_case(rng, 16, 8, 300, 4, 1.0, scale=2.0)
    out = fused_kl(H, W, idx, logit, mask, tau, want_grads=False)
    S = (H @ W.T) / tau
    np.testing.assert_allclose(_tiled_online_lse(S, tile), out["row_lse"], rtol=1e-12)


# -- 4. brute force from the definition, pure Python ---------------------------

def _brute(H, W, idx, logit, mask, tau):
    T, d = len(H), len(H[0])
    V = len(W)
    N = sum(1 for t in range(T) if mask[t])
    s = tau / N
    loss_terms = []
    G = [[0.0] * V for _ in range(T)]
    for t in range(T):
        z = [math.fsum(H[t][j] * W[v][j] for j in range(d)) for v in range(V)]
        S = [x / tau for x in z]
        mx = max(S)
        lse = mx + math.log(math.fsum(math.exp(x - mx) for x in S))
        a = [x / tau for x in logit[t]]
        amx = max(a)
        lz = amx + math.log(math.fsum(math.exp(x - amx) for x in a))
        p = [math.exp(x - lz) for x in a]
        kl = math.fsum(p[k] * ((a[k] - lz) - (S[idx[t][k]] - lse)) for k in range(len(a)))
        if mask[t]:
            loss_terms.append(kl)
            for v in range(V):
                Pv = math.fsum(p[k] for k in range(len(a)) if idx[t][k] == v)
                G[t][v] = s * (math.exp(S[v] - lse) - Pv)
    loss = tau * tau * math.fsum(loss_terms) / N
    gH = [[math.fsum(G[t][v] * W[v][j] for v in range(V)) for j in range(d)] for t in range(T)]
    gW = [[math.fsum(G[t][v] * H[t][j] for t in range(T)) for j in range(d)] for v in range(V)]
    return loss, np.array(gH), np.array(gW)


@pytest.mark.parametrize("shape", [(5, 4, 7, 3, 1.0), (4, 6, 64, 64, 0.7), (7, 3, 33, 1, 2.5),
                                   (3, 5, 20, 6, 1.0)])
def test_brute_force_small_vocab(shape):
    T, d, V, K, tau = shape
    rng = np.random.default_rng(T * 1000 + V)
    H, W, idx, logit, mask, tau = _rand_case(rng, T, d, V, K, tau, masked_rows=(1,),
                                             dup_row=(2 if K >= 2 else None))
    out = fused_kl(H, W, idx, logit, mask, tau)
    loss, gH, gW = _brute(H.tolist(), W.tolist(), idx.tolist(), logit.tolist(), mask.tolist(), tau)
    assert abs(out["loss"] - loss) <= 1e-12 * abs(loss)
    assert np.linalg.norm(out["grad_hidden"] - gH) <= 1e-12 * np.linalg.norm(gH)
    assert np.linalg.norm(out["grad_W"] - gW) <= 1e-12 * np.linalg.norm(gW)


# -- closed forms and library special cases ------------------------------------

def test_zero_head_equal_logits_gives_log_v_over_k():
    # W = 0: the student is uniform, q = 1/V.  Equal teacher logits: p = 1/K.
    # KL = sum_k (1/K)(log(1/K) - log(1/V)) = log(V/K); log(4096/16) = log 256.
    T, d, V, K = 8, 16, 4096, 16
    rng = np.random.default_rng(0)
    H = rng.standard_normal((T, d))
    W = np.zeros((V, d))
    idx = np.stack([rng.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    logit = np.full((T, K), 1.25)
    mask = np.ones(T, dtype=np.uint8); mask[5] = 0
    out = fused_kl(H, W, idx, logit, mask, 1.0)
    assert abs(out["loss"] - 5.545177444479562) < 1e-12
    # G = s m (1/V - P): with W = 0, grad_hidden = G W = 0 and grad_W = G^T H.
    s = 1.0 / 7
    G = np.full((T, V), 1.0 / V) * s
    for t in range(T):
        G[t, idx[t]] -= s / K
    G[5] = 0
    np.testing.assert_allclose(out["grad_W"], G.T @ H, rtol=1e-12, atol=1e-15)
    assert np.all(out["grad_hidden"] == 0)


@pytest.mark.parametrize("tau", [1.0, 3.0])
def test_k1_is_masked_cross_entropy(tau):
    import torch
    rng = np.random.default_rng(21)
    T, d, V = 40, 12, 50
    H = rng.standard_normal((T, d)); W = rng.standard_normal((V, d))
    idx = rng.integers(0, V, size=(T, 1)).astype(np.int32)
    logit = rng.standard_normal((T, 1))
    mask = (rng.random(T) > 0.2).astype(np.uint8)
    out = fused_kl(H, W, idx, logit, mask, tau, rows_per_block=16)
    target = torch.tensor(np.where(mask > 0, idx[:, 0], -100), dtype=torch.long)
    ce = torch.nn.functional.cross_entropy(torch.tensor(H @ W.T / tau, dtype=torch.float64),
                                           target, ignore_index=-100, reduction="mean")
    assert abs(out["loss"] - tau * tau * ce.item()) <= 1e-12 * abs(out["loss"])


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_k_equals_v_is_full_kl_scipy(tau):
    rng = np.random.default_rng(8)
    T, d, V = 6, 7, 24
    H = rng.standard_normal((T, d)); W = rng.standard_normal((V, d))
    idx = np.stack([rng.permutation(V) for _ in range(T)]).astype(np.int32)
    logit = rng.standard_normal((T, V)) * 2
    out = fused_kl(H, W, idx, logit, None, tau)
    q = scipy.special.softmax(H @ W.T / tau, axis=1)
    want = []
    for t in range(T):
        p_full = np.zeros(V)
        p_full[idx[t]] = scipy.special.softmax(logit[t] / tau)
        want.append(scipy.special.rel_entr(p_full, q[t]).sum())
    np.testing.assert_allclose(out["row_kl"], want, rtol=1e-11)
    assert abs(out["loss"] - tau * tau * np.mean(want)) <= 1e-11 * out["loss"]


def test_tau_homogeneity():
    rng = np.random.default_rng(9)
    H, W, idx, logit, mask, _ = _rand_case(rng, 12, 6, 30, 5, 1.0, masked_rows=(0,))
    tau = 2.5
    a = fused_kl(H, W, idx, logit, mask, tau)["loss"]
    b = fused_kl(H / tau, W, idx, logit / tau, mask, 1.0)["loss"]
    assert abs(a - tau * tau * b) <= 1e-12 * abs(a)


def test_torch_autograd_gradients():
    import torch
    rng = np.random.default_rng(13)
    H, W, idx, logit, mask, tau = _rand_case(rng, 10, 6, 25, 4, 1.7, masked_rows=(4,), dup_row=7)
    out = fused_kl(H, W, idx, logit, mask, tau)
    Ht = torch.tensor(H, requires_grad=True); Wt = torch.tensor(W, requires_grad=True)
    logq = torch.log_softmax(Ht @ Wt.T / tau, dim=1)
    logp = torch.log_softmax(torch.tensor(logit) / tau, dim=1)
    kl = (logp.exp() * (logp - torch.gather(logq, 1, torch.tensor(idx, dtype=torch.long)))).sum(1)
    m = torch.tensor(mask, dtype=torch.float64)
    loss = tau * tau * (m * kl).sum() / m.sum()
    loss.backward()
    assert abs(loss.item() - out["loss"]) <= 1e-12 * out["loss"]
    np.testing.assert_allclose(Ht.grad.numpy(), out["grad_hidden"], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(Wt.grad.numpy(), out["grad_W"], rtol=1e-10, atol=1e-14)


# -- invariants -----------------------------------------------------------------

def test_invariants():
    rng = np.random.default_rng(17)
    H, W, idx, logit, mask, tau = _rand_case(rng, 30, 8, 60, 6, 1.3, masked_rows=(2, 11), dup_row=5)
    out = fused_kl(H, W, idx, logit, mask, tau)
    # Gibbs: KL_t >= -log sum_k q[idx_k] >= 0
    S = H @ W.T / tau
    lse = scipy.special.logsumexp(S, axis=1)
    q = np.exp(S - lse[:, None])
    uniq_mass = np.array([q[t, np.unique(idx[t])].sum() for t in range(30)])
    assert np.all(out["row_kl"] >= -np.log(uniq_mass) - 1e-12)
    assert out["loss"] >= 0
    # joint permutation of k
    perm = rng.permutation(6)
    o2 = fused_kl(H, W, idx[:, perm], logit[:, perm], mask, tau)
    assert abs(o2["loss"] - out["loss"]) <= 1e-12 * out["loss"]
    # per-row teacher shift
    o3 = fused_kl(H, W, idx, logit + rng.standard_normal((30, 1)) * 5, mask, tau)
    assert abs(o3["loss"] - out["loss"]) <= 1e-11 * out["loss"]
    # W <- W + 1 c^T leaves every row's log-softmax unchanged
    o4 = fused_kl(H, W + rng.standard_normal((1, 8)), idx, logit, mask, tau)
    assert abs(o4["loss"] - out["loss"]) <= 1e-11 * out["loss"]
    # zero column sums of grad_W
    colsum = out["grad_W"].sum(axis=0)
    assert np.linalg.norm(colsum) <= 1e-12 * np.abs(out["grad_W"]).sum()
    # homogeneity: <gH, H> = <gW, W> = sum G o Z
    a = np.vdot(out["grad_hidden"], H)
    b = np.vdot(out["grad_W"], W)
    assert abs(a - b) <= 1e-11 * (abs(a) + 1e-30)
    # masked rows: zero grad, and their data does not matter
    assert np.all(out["grad_hidden"][[2, 11]] == 0)
    H2 = H.copy(); H2[2] = 100.0
    logit2 = logit.copy(); logit2[11] = 7.0
    o5 = fused_kl(H2, W, idx, logit2, mask, tau)
    assert abs(o5["loss"] - out["loss"]) <= 1e-13 * out["loss"]
    np.testing.assert_allclose(o5["grad_W"], out["grad_W"], rtol=1e-12, atol=1e-15)


def test_all_masked_gives_zero():
    rng = np.random.default_rng(1)
    H, W, idx, logit, _, tau = _rand_case(rng, 5, 4, 10, 3, 1.0)
    out = fused_kl(H, W, idx, logit, np.zeros(5, dtype=np.uint8), tau)
    assert out["loss"] == 0.0 and out["N"] == 0
    assert np.all(out["grad_hidden"] == 0) and np.all(out["grad_W"] == 0)


def test_rows_variant_matches_full():
    rng = np.random.default_rng(4)
    H, W, idx, logit, mask, tau = _rand_case(rng, 40, 7, 90, 5, 1.1, masked_rows=(6,), dup_row=3)
    full = fused_kl(H, W, idx, logit, mask, tau)
    rows = [0, 3, 6, 39]
    r = fused_kl_rows(H, W, idx, logit, mask, tau, rows, vocab_block=17)
    np.testing.assert_allclose(r["row_lse"], full["row_lse"][rows], rtol=1e-13)
    np.testing.assert_allclose(r["row_kl"], full["row_kl"][rows], rtol=1e-12)
    np.testing.assert_allclose(r["grad_hidden_rows"], full["grad_hidden"][rows], rtol=1e-12, atol=1e-16)


def test_invalid_ids_contribute_nothing():
    rng = np.random.default_rng(6)
    H, W, idx, logit, mask, tau = _rand_case(rng, 8, 5, 20, 4, 1.0)
    bad = idx.copy(); bad[3, 2] = 20; bad[5, 0] = -1
    out = fused_kl(H, W, bad, logit, mask, tau)
    p, log_p = teacher_distribution(logit, tau)
    ref = fused_kl(H, W, idx, logit, mask, tau)
    S = H @ W.T
    lse = scipy.special.logsumexp(S, axis=1)
    d3 = p[3, 2] * (log_p[3, 2] - (S[3, idx[3, 2]] - lse[3]))
    d5 = p[5, 0] * (log_p[5, 0] - (S[5, idx[5, 0]] - lse[5]))
    assert abs(out["row_kl"][3] - (ref["row_kl"][3] - d3)) < 1e-12
    assert abs(out["row_kl"][5] - (ref["row_kl"][5] - d5)) < 1e-12

"""The offline top-K teacher-logit cache builder on the GPU, against the oracle.

Several answers are correct where logits differ by less than the kernels'
rounding (fp32 sums of exact products), so the checks compare what is unique
and verify the rest:
  - each row's ids are distinct and valid, the logits are non-increasing and
    equal logits come in increasing id order;
  - the logits equal the oracle's fp64 logits at the returned ids (to the
    rounding of an fp32 sum over d);
  - the returned set is a valid top-K: no id left out has an oracle logit
    larger than a returned one by more than that rounding; where the oracle's
    K-th and (K+1)-th logits are further apart, the ids equal the oracle's.
Cases: the 32-row-block threshold path, the collect-everything path (fewer
blocks than K), fp32 inputs, padded d, ragged chunks, exact ties (duplicated
head rows), fully tied rows (the exact fallback), K = V, K = 4096 (the
maximum, both paths), the full-size head at reduced T, the cache feeding
the loss, and 30 seeded random shapes.
"""
import numpy as np
import pytest

from oracle import fused_kl, teacher_logits, topk_cache
from tests.gpu_util import GRAD_TOL, LOSS_TOL, log, rel, rel_f

pytestmark = pytest.mark.gpu


def _bf16(a):
    from datagen import f32_to_bf16_bits
    return f32_to_bf16_bits(np.ascontiguousarray(a, dtype=np.float32))


def _dev(a, dtype):
    import torch
    from datagen import _host_tensor
    if dtype == "bf16":
        return _host_tensor(np.asarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return _host_tensor(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def _run(H, W, K, chunk, dtype):
    import torch
    import chunked_top_kl_lm_amd as kd
    idx, logit = kd.topk_cache(_dev(H, dtype), _dev(W, dtype), K=K, chunk=chunk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), logit.cpu().numpy()


def _check(H, W, K, chunk, dtype, tag, exact_ids=None):
    log(f"[gpu-cache] {tag}: T={H.shape[0]} d={H.shape[1]} V={W.shape[0]} K={K} chunk={chunk} {dtype}")
    idx, logit = _run(H, W, K, chunk, dtype)
    T, V = H.shape[0], W.shape[0]
    z = teacher_logits(H, W)                       # fp64, all rows (small cases)
    ref_idx, ref_val = topk_cache(H, W, K)
    worst = 0.0
    n_exact = 0
    for t in range(T):
        ids = idx[t]
        assert len(set(ids.tolist())) == K and ids.min() >= 0 and ids.max() < V
        assert np.all(np.diff(logit[t]) <= 0)
        eq = np.diff(logit[t]) == 0
        assert np.all(np.diff(ids)[eq] > 0), "equal logits must come in increasing id order"
        tol = 1e-5 * max(1.0, np.abs(z[t]).max())
        err = np.abs(logit[t] - z[t, ids]).max()
        worst = max(worst, err / tol)
        assert err <= tol
        out = np.ones(V, dtype=bool)
        out[ids] = False
        if out.any():
            assert z[t, ids].min() >= z[t, out].max() - 2 * tol, "not a top-K set"
        gap = ref_val[t, K - 1] - (np.sort(z[t])[::-1][K] if K < V else -np.inf)
        if gap > 4 * tol:
            assert sorted(ids.tolist()) == sorted(ref_idx[t].tolist())
            n_exact += 1
    if exact_ids is not None:
        assert np.array_equal(idx, exact_ids)
    log(f"[gpu-cache] {tag}: max |dz|/tol {worst:.2e}; rows with a clear K-th gap matching the oracle {n_exact}/{T}")
    return idx, logit


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_threshold_path(dtype):
    rng = np.random.default_rng(1)
    H = rng.standard_normal((300, 256)).astype(np.float32)
    W = (rng.standard_normal((5000, 256)) * 0.1).astype(np.float32)
    if dtype == "bf16":
        H, W = _bf16(H), _bf16(W)
    _check(H, W, 16, 128, dtype, "threshold path")


def test_collect_everything_path_small_vocab():
    rng = np.random.default_rng(2)
    H = _bf16(rng.standard_normal((70, 64)))
    W = _bf16(rng.standard_normal((300, 64)) * 0.2)
    _check(H, W, 100, 32, "bf16", "fewer blocks than K")


def test_padded_d_ragged_chunks_and_k_equals_v():
    rng = np.random.default_rng(3)
    H = _bf16(rng.standard_normal((45, 70)))
    W = _bf16(rng.standard_normal((64, 70)))
    _check(H, W, 64, 20, "bf16", "K = V, d = 70")
    H = rng.standard_normal((33, 100)).astype(np.float32)
    W = rng.standard_normal((4000, 100)).astype(np.float32)
    _check(H, W, 8, 16, "f32", "padded d, ragged chunk")


def test_exact_ties_by_lower_id():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((3000, 128)).astype(np.float32) * 0.1
    W[2000:2050] = W[10:60]                        # duplicated head rows tie exactly
    H = rng.standard_normal((50, 128)).astype(np.float32)
    H, W = _bf16(H), _bf16(W)
    idx, logit = _check(H, W, 32, 64, "bf16", "duplicated head rows")
    for t in range(H.shape[0]):
        ids = set(idx[t].tolist())
        for a in range(10, 60):
            if a + 1990 in ids:                    # a tie partner was taken: the lower id must be too
                assert a in ids


def test_fully_tied_rows_take_the_fallback():
    rng = np.random.default_rng(5)
    W = np.tile(rng.standard_normal((1, 96)).astype(np.float32), (6000, 1))   # every logit of a row equal
    H = rng.standard_normal((20, 96)).astype(np.float32)
    H, W = _bf16(H), _bf16(W)
    idx, logit = _check(H, W, 24, 16, "bf16", "all logits tied", exact_ids=np.tile(np.arange(24), (20, 1)))
    assert np.all(logit == logit[:, :1])


def test_maximum_cache_width():
    """K = KD_MAX_K = 4096: with V = 6000 every logit is a candidate and fits
    the 8192-entry list; with V = 10000 the list overflows and every row takes
    the exact fallback (a sorted top-4096 in LDS)."""
    rng = np.random.default_rng(8)
    H = _bf16(rng.standard_normal((6, 64)))
    _check(H, _bf16(rng.standard_normal((6000, 64)) * 0.3), 4096, 4, "bf16", "K = 4096, V = 6000")
    _check(H, _bf16(rng.standard_normal((10000, 64)) * 0.3), 4096, 4, "bf16", "K = 4096, V = 10000")


def test_full_size_head_reduced_rows():
    from datagen import config_for, make_inputs
    x = make_inputs(config_for(3, T=96), seed=7)   # the 32K workload's head: d=2880, V=201088
    _check(x["hidden"], x["W"], 100, 64, "bf16", "d=2880 V=201088 K=100")


def test_cache_feeds_the_loss():
    """Build a cache from a synthetic teacher head, then train-step the
    student against it: the loss and gradients match the oracle run on the
    same cache."""
    import torch
    import chunked_top_kl_lm_amd as kd
    rng = np.random.default_rng(6)
    T, d, V, K = 200, 256, 6000, 20
    Ht = _bf16(rng.standard_normal((T, d)))
    Wt = _bf16(rng.standard_normal((V, d)) * 0.1)
    idx, logit = kd.topk_cache(_dev(Ht, "bf16"), _dev(Wt, "bf16"), K=K, chunk=64)
    Hs = _bf16(rng.standard_normal((T, d)))
    Ws = _bf16(rng.standard_normal((V, d)) * 0.1)
    mask = (rng.random(T) > 0.05).astype(np.uint8)
    log("[gpu-cache] cache -> loss")
    loss, gH, gW = kd.fwd_bwd(_dev(Hs, "bf16"), _dev(Ws, "bf16"), idx, logit,
                              torch.from_numpy(mask).to("cuda:0"), tau=1.0, chunk=64)
    torch.cuda.synchronize()
    ref = fused_kl(Hs, Ws, idx.cpu().numpy(), logit.cpu().numpy(), mask, 1.0)
    assert rel(float(loss.item()), ref["loss"]) <= LOSS_TOL
    assert rel_f(gH.cpu().numpy(), ref["grad_hidden"]) <= GRAD_TOL
    assert rel_f(gW.cpu().numpy(), ref["grad_W"]) <= GRAD_TOL


def test_timed_build_matches_untimed():
    import torch
    import chunked_top_kl_lm_amd as kd
    rng = np.random.default_rng(9)
    H = _dev(_bf16(rng.standard_normal((100, 128))), "bf16")
    W = _dev(_bf16(rng.standard_normal((3000, 128)) * 0.1), "bf16")
    log("[gpu-cache] timed build")
    nslots = kd.KD_CACHE_PHASES * (-(-100 // 32)) + 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nslots)]
    for e in ev:
        e.record()
    a = kd.topk_cache(H, W, K=16, chunk=32)
    b = kd.topk_cache(H, W, K=16, chunk=32, events=ev)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert all(ev[2 * i].elapsed_time(ev[2 * i + 1]) >= 0 for i in range(nslots))


def _sweep_cases(n=30, seed=31):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 400))
        d = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 600)), int(rng.integers(600, 3000))]))
        K = int(rng.integers(1, 257))
        V = int(rng.integers(K, 12000))
        chunk = int(rng.integers(1, T + 64))
        dtype = "f32" if i % 4 == 3 else "bf16"
        out.append((T, d, V, K, chunk, dtype, i))
    return out


@pytest.mark.parametrize("T,d,V,K,chunk,dtype,i", _sweep_cases())
def test_random_shapes(T, d, V, K, chunk, dtype, i):
    """Seeded random shapes: ragged chunks and vocabularies, padded d, both
    paths (a 32-row block per candidate bound, or every logit when the
    vocabulary has fewer blocks than K), both input dtypes."""
    rng = np.random.default_rng(700 + i)
    H = rng.standard_normal((T, d)).astype(np.float32)
    W = (rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32) * 2
    if dtype == "bf16":
        H, W = _bf16(H), _bf16(W)
    _check(H, W, K, chunk, dtype, f"sweep {i}")

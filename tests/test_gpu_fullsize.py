"""Full-size workloads on the GPU, in the launch configuration bench.py times.

The 8K and 32K workloads are compared with the oracle element by element in
test_gpu_fullsize_oracle.py.  At T = 131072 / 262144 the whole oracle would
take tens of minutes, so these tests compare one chunk's rows in full (the
first 4096 rows at 128K, the last 4096 at 256K: row logsumexp, row KL and
grad_hidden element by element) and check (and, at 32K, check again on the
way to the split calls):
  - sampled rows (first, last, masked, random) of row_lse, row_kl and
    grad_hidden against the oracle's per-row results, element by element;
  - the loss against tau^2 * sum_t m_t KL_t / N recomputed in fp64 from the
    library's own per-row KL (the reduction), and finite/positive;
  - properties that hold at any size: zero column sums of grad_W
    (sum_v G[t,v] = 0), <grad_hidden, H> = <grad_W, W> (both equal sum G.Z),
    masked rows of grad_hidden exactly zero;
  - the workspace and the peak device memory beyond the O(T) buffers do not
    depend on T.
test_gpu_fullsize_oracle.py also runs the chunk-4096 path (their launch
configuration) against the oracle element by element at d = 2880.  At the
32K workload the split calls are checked against the fused call, and the
cache builder's sampled rows against the oracle.
"""
import numpy as np
import pytest

from datagen import config_for, make_inputs, to_device
from oracle import fused_kl_rows
from tests.gpu_util import GRAD_TOL, LOSS_TOL, ROW_KL_TOL, ROW_LSE_TOL, log, rel, rel_f, row_errors

pytestmark = pytest.mark.gpu


def _run_full(num, T=None):
    import torch
    import chunked_top_kl_lm_amd as kd
    cfg = config_for(num, **({"T": T} if T else {}))
    log(f"[gpu-full] generating {cfg.name} T={cfg.T}")
    x = make_inputs(cfg, seed=0, topk_backend="torch-cuda")
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    t = to_device(x)
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    log(f"[gpu-full] {cfg.name}: T={cfg.T} chunk={cfg.chunk} tau={cfg.tau}")
    loss, gH, gW, rl, rk = kd.fwd_bwd(t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"],
                                      tau=cfg.tau, chunk=cfg.chunk, row_stats=True, status=st)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    out = dict(loss=float(loss.item()), status=int(st.item()), peak=peak,
               gH=gH, gW=gW, row_lse=rl.cpu().numpy(), row_kl=rk.cpu().numpy(), t=t)
    return x, cfg, out


def _checks(x, cfg, out, n_random=6):
    import torch
    T = cfg.T
    assert out["status"] == 0
    mask = x["mask"]
    # the loss is the tau^2-scaled masked mean of the per-row KL
    m = mask.astype(np.float64)
    want = cfg.tau ** 2 * float((m * out["row_kl"].astype(np.float64)).sum()) / m.sum()
    assert np.isfinite(out["loss"]) and out["loss"] > 0
    assert rel(out["loss"], want) < 1e-5
    # sampled rows against the oracle
    rng = np.random.default_rng(123)
    masked = np.nonzero(mask == 0)[0]
    rows = sorted(set([0, T - 1, int(masked[0]), int(masked[-1])] + rng.integers(0, T, n_random).tolist()))
    log(f"[gpu-full] oracle rows {rows}")
    ref = fused_kl_rows(x["hidden"], x["W"], x["teacher_idx"], x["teacher_logit"], mask, cfg.tau, rows)
    gH_rows = out["gH"][torch.tensor(rows, device="cuda:0")].cpu().numpy()
    e_lse = np.max(np.abs(out["row_lse"][rows] - ref["row_lse"]))
    e_kl = np.max(np.abs(out["row_kl"][rows] - ref["row_kl"]) / np.maximum(1.0, np.abs(ref["row_kl"])))
    live = [i for i, r in enumerate(rows) if mask[r]]
    e_gh = rel_f(gH_rows[live], ref["grad_hidden_rows"][live])
    log(f"[gpu-full] max|dLSE| {e_lse:.2e}  max rel dKL {e_kl:.2e}  sampled dH relF {e_gh:.2e}")
    assert e_lse < 1e-3
    assert e_kl < LOSS_TOL
    assert e_gh < GRAD_TOL
    dead = [i for i, r in enumerate(rows) if not mask[r]]
    assert np.all(gH_rows[dead] == 0)
    # properties of the full gradients (fp64 reductions on the device)
    gW = out["gW"].double()
    colsum = gW.sum(0)
    cs = float(torch.linalg.norm(colsum) / torch.linalg.norm(gW.abs().sum(0)))
    hid = out["t"]["hidden"].double()
    Wd = out["t"]["W"].double()
    a = float((out["gH"].double() * hid).sum())
    b = float((gW * Wd).sum())
    log(f"[gpu-full] column-sum ratio {cs:.2e}  <dH,H> {a:.6e}  <dW,W> {b:.6e}")
    assert cs < 1e-2
    assert rel(a, b) < GRAD_TOL


def test_gptoss_32k_full():
    x, cfg, out = _run_full(3)
    _checks(x, cfg, out)
    # the split calls at the same size (bench.py --split): the forward's loss
    # and row statistics are the fused call's bit for bit, the gradients equal
    # them up to the rounding of the saved natural-log normaliser
    import torch
    import chunked_top_kl_lm_amd as kd
    t = out["t"]
    args = (t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"])
    log("[gpu-full] gptoss-32k (T=32768) through the split calls")
    loss_s, rl_s = kd.fwd(*args, tau=cfg.tau, chunk=cfg.chunk)
    gH_s, gW_s, _ = kd.bwd(*args, rl_s, tau=cfg.tau, chunk=cfg.chunk)
    torch.cuda.synchronize()
    assert float(loss_s.item()) == out["loss"]
    assert np.array_equal(rl_s.cpu().numpy(), out["row_lse"])
    e_h = float(torch.linalg.norm(gH_s - out["gH"]) / torch.linalg.norm(out["gH"]))
    e_w = float(torch.linalg.norm(gW_s - out["gW"]) / torch.linalg.norm(out["gW"]))
    log(f"[gpu-full] split vs fused: dH relF {e_h:.2e}  dW relF {e_w:.2e}")
    assert e_h < 1e-3 and e_w < 1e-3


def test_topk_cache_full_size_sampled_rows():
    """The cache builder at the full 32K head (bench.py --topk-cache): every
    row valid and sorted, and sampled rows against the oracle's fp64 logits."""
    import torch
    import chunked_top_kl_lm_amd as kd
    from oracle import teacher_logits, topk_cache
    cfg = config_for(3)
    log("[gpu-full] generating the 32K head for the cache builder")
    x = make_inputs(cfg, seed=0, topk_backend="torch-cuda")
    t = to_device(x)
    idx, logit = kd.topk_cache(t["hidden"], t["W"], K=cfg.K, chunk=cfg.chunk)
    torch.cuda.synchronize()
    idx, logit = idx.cpu().numpy(), logit.cpu().numpy()
    V = cfg.V
    assert idx.min() >= 0 and idx.max() < V
    assert np.all(np.diff(logit, axis=1) <= 0)
    rows = [0, 1, cfg.T // 2, cfg.T - 1] + np.random.default_rng(5).integers(0, cfg.T, 8).tolist()
    log(f"[gpu-full] cache rows {rows}")
    H = x["hidden"][rows]
    z = teacher_logits(H, x["W"])
    ref_idx, ref_val = topk_cache(H, x["W"], cfg.K)
    for i, r in enumerate(rows):
        ids = idx[r]
        assert len(set(ids.tolist())) == cfg.K
        tol = 1e-5 * max(1.0, np.abs(z[i]).max())
        assert np.abs(logit[r] - z[i, ids]).max() <= tol
        out_mask = np.ones(V, dtype=bool)
        out_mask[ids] = False
        assert z[i, ids].min() >= z[i, out_mask].max() - 2 * tol
        gap = ref_val[i, cfg.K - 1] - np.sort(z[i])[::-1][cfg.K]
        if gap > 4 * tol:
            assert sorted(ids.tolist()) == sorted(ref_idx[i].tolist())


def _rows_against_oracle(x, cfg, out, r0, r1, block=1024):
    """Every row of [r0, r1) against the oracle: row logsumexp, row KL and
    grad_hidden element by element (the oracle's per-row results take the
    gradient scale from the whole sequence's mask)."""
    import torch
    log(f"[gpu-full] oracle rows [{r0}, {r1}) in full")
    e_lse = e_kl = 0.0
    num = den = 0.0
    for b0 in range(r0, r1, block):
        rows = np.arange(b0, min(r1, b0 + block))
        ref = fused_kl_rows(x["hidden"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], cfg.tau, rows)
        a, k = row_errors(out["row_lse"][rows], out["row_kl"][rows], ref["row_lse"], ref["row_kl"])
        e_lse, e_kl = max(e_lse, a), max(e_kl, k)
        g = out["gH"][torch.from_numpy(rows).to("cuda:0")].cpu().numpy().astype(np.float64)
        num += float(((g - ref["grad_hidden_rows"]) ** 2).sum())
        den += float((ref["grad_hidden_rows"] ** 2).sum())
        log(f"[gpu-full]   rows up to {rows[-1] + 1} done")
    e_gh = (num / den) ** 0.5
    log(f"[gpu-full] rows [{r0}, {r1}): max|dLSE| {e_lse:.2e}  max rel|dKL| {e_kl:.2e}  dH relF {e_gh:.2e}")
    assert e_lse <= ROW_LSE_TOL and e_kl <= ROW_KL_TOL and e_gh <= GRAD_TOL


def test_long_128k_full_tau2():
    x, cfg, out = _run_full(4)
    _checks(x, cfg, out)
    # the first chunk (4096 rows, tau = 2, its peaked rows among them) in full
    _rows_against_oracle(x, cfg, out, 0, cfg.chunk)


def test_extreme_256k_full_and_memory_is_t_independent():
    import chunked_top_kl_lm_amd as kd
    x, cfg, out = _run_full(5)
    _checks(x, cfg, out, n_random=4)
    # the last chunk in full
    _rows_against_oracle(x, cfg, out, cfg.T - cfg.chunk, cfg.T)
    peak_256k = out["peak"]
    del out, x
    import torch
    torch.cuda.empty_cache()
    # the same head at T = 32768 with the same chunk
    x2, cfg2, out2 = _run_full(5, T=32768)
    peak_32k = out2["peak"]
    d, V, K = cfg.d, cfg.V, cfg.K
    # O(T) buffers: hidden (bf16) + grad_hidden (fp32) + idx + logit + mask + 2 row stats + loss/status
    per_token = 2 * d + 4 * d + 4 * K + 4 * K + 1 + 4 + 4
    extra = (peak_256k - peak_32k) - per_token * (cfg.T - cfg2.T)
    log(f"[gpu-full] peak {peak_32k / 2**30:.2f} GiB at T=32768, {peak_256k / 2**30:.2f} GiB at T=262144; "
        f"difference beyond the O(T) buffers {extra / 2**20:.1f} MiB")
    assert abs(extra) < 64 * 2**20
    assert kd.workspace_bytes(262144, d, V, K, cfg.chunk, kd.KD_BF16) == kd.workspace_bytes(32768, d, V, K, cfg.chunk, kd.KD_BF16)

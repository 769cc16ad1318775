"""Split forward / backward entry points and the autograd node, on the GPU.

The split calls run the same kernels as the fused call; the backward
recomputes each chunk's logits from the saved per-row logsumexp.  Checked:
  - the forward's loss and row statistics equal the fused call's bit for bit;
  - the backward's gradients match the fused call's (they differ only by the
    rounding of the saved natural-log normaliser) and the oracle's;
  - the options: the upstream gradient scale (a power of two scales the
    gradients exactly), accumulation into grad_W, bf16 outputs (equal to the
    round-to-nearest-even of the fp32 results), skipping either gradient,
    invalid ids reported by the backward;
  - torch.autograd end to end, with and without an fp32 grad_W accumulator,
    against the oracle;
  - 16 seeded random shapes through the split calls.
"""
import numpy as np
import pytest

from datagen import config_for, make_inputs
from oracle import fused_kl
from tests.gpu_util import GRAD_TOL, LOSS_TOL, log, rel, rel_f, to_device

pytestmark = pytest.mark.gpu


def _inputs(num=3, T=520, d=None, V=None, seed=0):
    kw = {"T": T}
    if d:
        kw["d"] = d
    if V:
        kw["V"] = V
    return make_inputs(config_for(num, **kw), seed=seed)


def _bf16_round(a):
    """fp32 -> bf16 -> fp32, round to nearest even (numpy, for comparisons)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("num,T,chunk", [(3, 520, 256), (1, 512, 128)])
def test_split_matches_fused_and_oracle(num, T, chunk):
    import torch
    import chunked_top_kl_lm_amd as kd
    x = _inputs(num, T)
    log(f"[gpu-split] {config_for(num).name} T={T} chunk={chunk}")
    t = to_device(x)
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    loss_f, gH_f, gW_f, rl_f, rk_f = kd.fwd_bwd(t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"],
                                                t["mask"], tau=x["tau"], chunk=chunk, row_stats=True)
    loss_s, rl_s, rk_s = kd.fwd(t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"],
                                tau=x["tau"], chunk=chunk, row_kl=True, status=st)
    gH_s, gW_s, _ = kd.bwd(t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"], rl_s,
                           tau=x["tau"], chunk=chunk)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert float(loss_s.item()) == float(loss_f.item())
    assert torch.equal(rl_s, rl_f) and torch.equal(rk_s, rk_f)
    e_h = rel_f(gH_s.cpu().numpy(), gH_f.cpu().numpy())
    e_w = rel_f(gW_s.cpu().numpy(), gW_f.cpu().numpy())
    log(f"[gpu-split] split vs fused: dH relF {e_h:.2e} dW relF {e_w:.2e}")
    assert e_h < 1e-3 and e_w < 1e-3
    ref = fused_kl(x["hidden"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], x["tau"])
    assert rel(float(loss_s.item()), ref["loss"]) <= LOSS_TOL
    assert rel_f(gH_s.cpu().numpy(), ref["grad_hidden"]) <= GRAD_TOL
    assert rel_f(gW_s.cpu().numpy(), ref["grad_W"]) <= GRAD_TOL


def test_backward_options():
    import torch
    import chunked_top_kl_lm_amd as kd
    x = _inputs(2, 300, d=512, V=9000, seed=7)
    t = to_device(x)
    args = (t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"])
    chunk, tau = 128, x["tau"]
    log("[gpu-split] backward options")
    _, rl = kd.fwd(*args, tau=tau, chunk=chunk)
    gH, gW, _ = kd.bwd(*args, rl, tau=tau, chunk=chunk)
    # upstream gradient 0.5: exactly half (a power of two commutes with every rounding)
    half = torch.full((), 0.5, dtype=torch.float32, device="cuda:0")
    gH2, gW2, _ = kd.bwd(*args, rl, tau=tau, chunk=chunk, grad_loss=half)
    assert torch.equal(gH2, gH * 0.5) and torch.equal(gW2, gW * 0.5)
    # accumulation into an fp32 buffer
    acc = gW.clone()
    _, gW3, _ = kd.bwd(*args, rl, tau=tau, chunk=chunk, grad_hidden=None, accumulate_into=acc)
    assert gW3.data_ptr() == acc.data_ptr()
    assert rel_f(acc.cpu().numpy(), 2 * gW.cpu().numpy()) < 1e-6
    # bf16 outputs are the rounded fp32 results
    gHb, gW4, gWb = kd.bwd(*args, rl, tau=tau, chunk=chunk, grad_hidden="bfloat16", grad_W_bf16=True)
    torch.cuda.synchronize()
    assert gHb.dtype == torch.bfloat16 and gWb.dtype == torch.bfloat16
    assert np.array_equal(gHb.float().cpu().numpy(), _bf16_round(gH.cpu().numpy()))
    assert np.array_equal(gWb.float().cpu().numpy(), _bf16_round(gW4.cpu().numpy()))
    assert torch.equal(gW4, gW)
    # either gradient alone
    gH5, gW5, _ = kd.bwd(*args, rl, tau=tau, chunk=chunk, grad_W=False)
    assert gW5 is None and torch.equal(gH5, gH)
    gH6, gW6, _ = kd.bwd(*args, rl, tau=tau, chunk=chunk, grad_hidden=None)
    assert gH6 is None and torch.equal(gW6, gW)
    with pytest.raises(kd.KdError):
        kd.bwd(*args, rl, tau=tau, chunk=chunk, grad_hidden=None, grad_W=False)


def test_backward_reports_bad_index():
    import torch
    import chunked_top_kl_lm_amd as kd
    x = _inputs(3, 64, d=256, V=3000, seed=9)
    x["teacher_idx"][5, 1] = 3000
    t = to_device(x)
    args = (t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"])
    log("[gpu-split] bad index in backward")
    rl = torch.zeros(64, dtype=torch.float32, device="cuda:0")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    kd.bwd(*args, rl, tau=x["tau"], chunk=32, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 7


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_end_to_end(dtype):
    import torch
    import chunked_top_kl_lm_amd as kd
    if dtype == "bf16":
        x = _inputs(3, 300, d=256, V=5000, seed=11)
    else:
        x = make_inputs(config_for(1, T=200), seed=11)
    t = to_device(x)
    log(f"[gpu-split] autograd {dtype}")
    h = t["hidden"].clone().requires_grad_(True)
    w = t["W"].clone().requires_grad_(True)
    loss = kd.kd_topk_kl_loss(h, w, t["teacher_idx"], t["teacher_logit"], t["mask"], tau=x["tau"], chunk=128)
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    assert h.grad.dtype == h.dtype and w.grad.dtype == w.dtype
    ref = fused_kl(x["hidden"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], x["tau"])
    e_l = rel(float(loss.item()), ref["loss"])
    e_h = rel_f(h.grad.float().cpu().numpy(), 3 * ref["grad_hidden"])
    e_w = rel_f(w.grad.float().cpu().numpy(), 3 * ref["grad_W"])
    log(f"[gpu-split] autograd {dtype}: loss rel {e_l:.2e} dH relF {e_h:.2e} dW relF {e_w:.2e}")
    assert e_l <= LOSS_TOL and e_h <= GRAD_TOL and e_w <= GRAD_TOL
    # fp32 accumulator for the head gradient (twice: the sum of two backward passes)
    acc = torch.zeros(w.shape, dtype=torch.float32, device="cuda:0")
    h2 = t["hidden"].clone().requires_grad_(True)
    w2 = t["W"].clone().requires_grad_(True)
    for _ in range(2):
        loss2 = kd.kd_topk_kl_loss(h2, w2, t["teacher_idx"], t["teacher_logit"], t["mask"], tau=x["tau"],
                                   chunk=128, grad_W_accumulator=acc)
        loss2.backward()
    torch.cuda.synchronize()
    assert w2.grad is None
    e_acc = rel_f(acc.cpu().numpy(), 2 * ref["grad_W"])
    log(f"[gpu-split] accumulator relF {e_acc:.2e}")
    assert e_acc <= GRAD_TOL


def test_timed_split_calls_match_untimed():
    """The measurement entry points (events around every phase) give the
    same bits as the plain calls."""
    import torch
    import chunked_top_kl_lm_amd as kd
    x = _inputs(3, 520, d=256, V=3000, seed=13)
    t = to_device(x)
    args = (t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"])
    log("[gpu-split] timed split calls")
    nslots = kd.KD_NUM_PHASES * (-(-520 // 128)) + 2

    def events():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nslots)]
        for e in ev:
            e.record()
        return ev

    loss_a, rl_a = kd.fwd(*args, tau=x["tau"], chunk=128)
    loss_b, rl_b = kd.fwd(*args, tau=x["tau"], chunk=128, events=events())
    gH_a, gW_a, _ = kd.bwd(*args, rl_a, tau=x["tau"], chunk=128)
    eb = events()
    gH_b, gW_b, _ = kd.bwd(*args, rl_b, tau=x["tau"], chunk=128, events=eb)
    torch.cuda.synchronize()
    assert float(loss_a.item()) == float(loss_b.item()) and torch.equal(rl_a, rl_b)
    assert torch.equal(gH_a, gH_b) and torch.equal(gW_a, gW_b)
    assert all(eb[2 * i].elapsed_time(eb[2 * i + 1]) >= 0 for i in range(nslots))


def _split_cases(n=16, seed=53):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 600))
        d = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 700)), int(rng.integers(700, 3000))]))
        K = int(rng.integers(1, 129))
        V = int(rng.integers(K, 8000))
        chunk = int(rng.integers(1, T + 64))
        tau = float(np.round(rng.uniform(0.3, 3.0), 2))
        dtype = "f32" if i % 4 == 3 else "bf16"
        out.append((T, d, V, K, chunk, tau, dtype, i))
    return out


@pytest.mark.parametrize("T,d,V,K,chunk,tau,dtype,i", _split_cases())
def test_split_random_shapes(T, d, V, K, chunk, tau, dtype, i):
    """Seeded random shapes through the split calls: the forward equals the
    fused call bit for bit, the backward (its own hit lists and teacher
    probabilities) matches the fused gradients and the oracle."""
    import torch
    import chunked_top_kl_lm_amd as kd
    from tests.gpu_util import run_gpu
    from tests.test_gpu_parity import _small
    x = _small(T, d, V, K, dtype, seed=900 + i, tau=tau, masked=tuple(range(0, T, 6)) if T > 3 else (),
               dup_row=(T // 2 if K >= 2 else None))
    log(f"[gpu-split] sweep {i}: T={T} d={d} V={V} K={K} chunk={chunk} tau={tau} {dtype}")
    fused = run_gpu(x, chunk=chunk)
    t = to_device(x)
    args = (t["hidden"], t["W"], t["teacher_idx"], t["teacher_logit"], t["mask"])
    loss_s, rl_s, rk_s = kd.fwd(*args, tau=tau, chunk=chunk, row_kl=True)
    gH_s, gW_s, _ = kd.bwd(*args, rl_s, tau=tau, chunk=chunk)
    torch.cuda.synchronize()
    assert float(loss_s.item()) == fused["loss"]
    assert np.array_equal(rl_s.cpu().numpy(), fused["row_lse"]) and np.array_equal(rk_s.cpu().numpy(), fused["row_kl"])
    gH, gW = gH_s.float().cpu().numpy(), gW_s.float().cpu().numpy()
    tight = dtype == "f32"
    assert rel_f(gH, fused["grad_hidden"]) < (1e-5 if tight else 1e-3)
    assert rel_f(gW, fused["grad_W"]) < (1e-5 if tight else 1e-3)
    ref = fused_kl(x["hidden"], x["W"], x["teacher_idx"], x["teacher_logit"], x["mask"], tau)
    assert rel_f(gH, ref["grad_hidden"]) <= (1e-4 if tight else GRAD_TOL)
    assert rel_f(gW, ref["grad_W"]) <= (1e-4 if tight else GRAD_TOL)

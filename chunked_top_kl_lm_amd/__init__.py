"""MI355X fused chunked top-K KL distillation loss: thin Python binding.

The computation runs entirely in the HIP library libkdtopk.so (C ABI in
include/kd_topk_kl.h).  This module only marshals arguments: PyTorch supplies
device memory (torch.empty) and the current stream.  If the library is not
built, every entry point raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["KD_BF16", "KD_F32", "KD_NUM_PHASES", "PHASES", "KD_CACHE_PHASES", "CACHE_PHASES", "KdError", "lib", "workspace_bytes", "fwd_bwd",
           "fwd", "bwd", "fwd_workspace_bytes", "bwd_workspace_bytes", "dw_chunks", "KdTopKKLFunction",
           "kd_topk_kl_loss", "topk_cache", "mfma_probe", "topk_cache_workspace_bytes",
           "fwd_bwd_noalloc", "NOALLOC_SCRATCH_BYTES",
           "status_str", "STATUS"]

KD_BF16 = 0
KD_F32 = 1
KD_NUM_PHASES = 8
KD_CACHE_PHASES = 4
CACHE_PHASES = ("gemm_block_max", "threshold", "collect", "select")
PHASES = ("chunk_prep", "gemm_fwd_lse", "kl_rows", "gemm_bwd_grad", "teacher_p",
          "gemm_dhidden", "dhidden_reduce", "gemm_dW")
STATUS = {0: "KD_OK", 1: "KD_ERR_NULL_ARG", 2: "KD_ERR_BAD_SHAPE", 3: "KD_ERR_BAD_TAU",
          4: "KD_ERR_BAD_CHUNK", 5: "KD_ERR_DTYPE", 6: "KD_ERR_WORKSPACE",
          7: "KD_ERR_BAD_INDEX", 8: "KD_ERR_HIP", 9: "KD_ERR_NOALLOC_SIZE"}
NOALLOC_SCRATCH_BYTES = 256 << 20     # KD_NOALLOC_SCRATCH_BYTES

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdtopk.so")
_lib = None


class KdError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"{STATUS.get(code, code)}: {status_str(code)}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libkdtopk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m chunked_top_kl_lm_amd._build`")
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        L.kd_topk_kl_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        L.kd_topk_kl_workspace_bytes.restype = ctypes.c_size_t
        L.kd_topk_kl_fwd_bwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, f32, i64,
                                         vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
        L.kd_topk_kl_fwd_bwd.restype = i32
        L.kd_topk_kl_fwd_bwd_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, f32, i64,
                                                 vp, vp, vp, vp, vp, vp, vp]
        L.kd_topk_kl_fwd_bwd_noalloc.restype = i32
        L.kd_topk_kl_fwd_bwd_timed.argtypes = L.kd_topk_kl_fwd_bwd.argtypes + [vp]
        L.kd_topk_kl_fwd_bwd_timed.restype = i32
        L.kd_topk_kl_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        L.kd_topk_kl_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.kd_topk_kl_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        L.kd_topk_kl_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.kd_topk_kl_dw_chunks.argtypes = [i64, i64, i64, i64, i64, i32]
        L.kd_topk_kl_dw_chunks.restype = i32
        L.kd_topk_kl_fwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, f32, i64,
                                     vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
        L.kd_topk_kl_fwd.restype = i32
        L.kd_topk_kl_bwd.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, f32, i64,
                                     vp, vp, vp, i32, vp, i32, vp, vp, ctypes.c_size_t, vp, vp]
        L.kd_topk_kl_bwd.restype = i32
        L.kd_topk_cache_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
        L.kd_topk_cache_workspace_bytes.restype = ctypes.c_size_t
        L.kd_topk_cache_build.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
        L.kd_topk_cache_build.restype = i32
        L.kd_topk_kl_fwd_timed.argtypes = L.kd_topk_kl_fwd.argtypes + [vp]
        L.kd_topk_kl_fwd_timed.restype = i32
        L.kd_topk_kl_bwd_timed.argtypes = L.kd_topk_kl_bwd.argtypes + [vp]
        L.kd_topk_kl_bwd_timed.restype = i32
        L.kd_topk_cache_build_timed.argtypes = L.kd_topk_cache_build.argtypes + [vp]
        L.kd_topk_cache_build_timed.restype = i32
        L.kd_mfma_probe.argtypes = [i32, i32, i32, vp, vp]
        L.kd_mfma_probe.restype = i32
        L.kd_status_str.argtypes = [i32]
        L.kd_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().kd_status_str(int(code)).decode()


def workspace_bytes(T: int, d: int, V: int, K: int, chunk: int, dtype: int) -> int:
    return int(lib().kd_topk_kl_workspace_bytes(T, d, V, K, chunk, dtype))


def fwd_workspace_bytes(T: int, d: int, V: int, K: int, chunk: int, dtype: int) -> int:
    return int(lib().kd_topk_kl_fwd_workspace_bytes(T, d, V, K, chunk, dtype))


def bwd_workspace_bytes(T: int, d: int, V: int, K: int, chunk: int, dtype: int) -> int:
    return int(lib().kd_topk_kl_bwd_workspace_bytes(T, d, V, K, chunk, dtype))


def dw_chunks(T: int, d: int, V: int, K: int, chunk: int, dtype: int) -> int:
    """Chunks contracted by one launch of the head-gradient GEMM (0: invalid sizes)."""
    return int(lib().kd_topk_kl_dw_chunks(T, d, V, K, chunk, dtype))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nchunks(T: int, chunk: int) -> int:
    c = min(int(chunk), int(T))
    return -(-int(T) // c) if c > 0 else 0


def _events(events, needed: int):
    """ctypes array of the hipEvent_t handles of already-recorded
    torch.cuda.Event objects; the library records into exactly `needed` of
    them, so any other count is refused before the call."""
    if len(events) != needed:
        raise ValueError(f"events: expected {needed} recorded torch.cuda.Event objects, got {len(events)}")
    return (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])


def _loss_events(events, T: int, chunk: int):
    return _events(events, 2 * (KD_NUM_PHASES * _nchunks(T, chunk) + 2))


def _check_device(dev, **tensors):
    """Every given tensor must live on the CUDA device `dev` (the library
    dereferences the pointers on that GPU)."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"{name} must be a CUDA tensor on {dev}")


def _check_workspace(workspace, status):
    import torch
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1):
        raise ValueError("status must be an int32 tensor of at least one element")


def _check_inputs(hidden, W, teacher_idx, teacher_logit, mask):
    import torch
    if not hidden.is_cuda:
        raise ValueError("hidden must be a CUDA tensor")
    _check_device(hidden.device, W=W, teacher_idx=teacher_idx, teacher_logit=teacher_logit, mask=mask)
    if hidden.dim() != 2 or W.dim() != 2 or teacher_idx.dim() != 2:
        raise ValueError("shapes: hidden [T,d], W [V,d], teacher_idx and teacher_logit [T,K]")
    T, d = hidden.shape
    V = W.shape[0]
    K = teacher_idx.shape[1]
    if hidden.dtype == torch.bfloat16:
        dt = KD_BF16
    elif hidden.dtype == torch.float32:
        dt = KD_F32
    else:
        raise TypeError("hidden must be bfloat16 or float32")
    for name, tns in (("hidden", hidden), ("W", W), ("teacher_idx", teacher_idx),
                      ("teacher_logit", teacher_logit), ("mask", mask)):
        if tns is not None and not tns.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if W.dtype != hidden.dtype or teacher_idx.dtype != torch.int32 or teacher_logit.dtype != torch.float32:
        raise TypeError("W must match hidden's dtype; teacher_idx int32; teacher_logit float32")
    if W.shape[1] != d or tuple(teacher_logit.shape) != (T, K) or teacher_idx.shape[0] != T:
        raise ValueError("shapes: hidden [T,d], W [V,d], teacher_idx and teacher_logit [T,K]")
    if mask is not None and (mask.dtype != torch.uint8 or tuple(mask.shape) != (T,)):
        raise TypeError("mask must be uint8 [T]")
    return T, d, V, K, dt


def fwd_bwd(hidden, W, teacher_idx, teacher_logit, mask=None, tau: float = 1.0,
            chunk: int = 2048, row_stats: bool = False, workspace=None, status=None,
            out=None, events=None):
    """Loss and gradients of the top-K KL distillation loss on the GPU.

    hidden [T,d] and W [V,d]: torch bfloat16 or float32 CUDA tensors
    (contiguous); teacher_idx [T,K] int32; teacher_logit [T,K] float32;
    mask [T] uint8 (nonzero = counts) or None.  Returns (loss [0-d float32],
    grad_hidden [T,d] float32, grad_W [V,d] float32) and, with row_stats,
    also (row_lse [T], row_kl [T]).  `out` may hold preallocated
    (loss, grad_hidden, grad_W[, row_lse, row_kl]); `workspace` a uint8 CUDA
    tensor of at least workspace_bytes(...) bytes; `status` an int32 CUDA
    tensor of one element that receives the device status.  `events`, for
    measurement only, is a sequence of 2 * (KD_NUM_PHASES * nchunks + 2)
    already-recorded torch.cuda.Event objects (see kd_topk_kl_fwd_bwd_timed).
    """
    import torch
    L = lib()
    T, d, V, K, dt = _check_inputs(hidden, W, teacher_idx, teacher_logit, mask)
    dev = hidden.device
    if out is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
        gH = torch.empty((T, d), dtype=torch.float32, device=dev)
        gW = torch.empty((V, d), dtype=torch.float32, device=dev)
        rl = torch.empty(T, dtype=torch.float32, device=dev) if row_stats else None
        rk = torch.empty(T, dtype=torch.float32, device=dev) if row_stats else None
    else:
        loss, gH, gW = out[:3]
        rl, rk = (out[3], out[4]) if row_stats else (None, None)
        for name, t, shape in (("loss", loss, ()), ("grad_hidden", gH, (T, d)), ("grad_W", gW, (V, d)),
                               ("row_lse", rl, (T,)), ("row_kl", rk, (T,))):
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()):
                raise ValueError(f"out: {name} must be a contiguous float32 tensor of shape {shape}")
        _check_device(dev, loss=loss, grad_hidden=gH, grad_W=gW, row_lse=rl, row_kl=rk)
    _check_device(dev, workspace=workspace, status=status)
    _check_workspace(workspace, status)
    nbytes = workspace_bytes(T, d, V, K, chunk, dt)
    if nbytes == 0:
        raise KdError(2)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (_ptr(hidden), _ptr(W), dt, _ptr(teacher_idx), _ptr(teacher_logit),
            _ptr(mask), T, d, V, K, float(tau), int(chunk), _ptr(loss), _ptr(gH),
            _ptr(gW), _ptr(rl), _ptr(rk), _ptr(workspace), workspace.numel(),
            _ptr(status), ctypes.c_void_p(stream))
    if events is None:
        rc = L.kd_topk_kl_fwd_bwd(*args)
    else:
        rc = L.kd_topk_kl_fwd_bwd_timed(*args, _loss_events(events, T, chunk))
    if rc != 0:
        raise KdError(rc)
    if row_stats:
        return loss, gH, gW, rl, rk
    return loss, gH, gW


def fwd_bwd_noalloc(hidden, W, teacher_idx, teacher_logit, mask=None, tau: float = 1.0,
                    chunk: int = 2048, out=None, row_stats: bool = False, status=None):
    """fwd_bwd through kd_topk_kl_fwd_bwd_noalloc: the library allocates
    nothing and uses its fixed device scratch (NOALLOC_SCRATCH_BYTES per
    GPU) as the workspace.  `out` = (loss, grad_hidden, grad_W[, row_lse,
    row_kl]) preallocated by the caller (allocated here if None, which a
    caller that cannot allocate does not do).  Calls that overlap on one GPU
    race on the scratch."""
    import torch
    L = lib()
    T, d, V, K, dt = _check_inputs(hidden, W, teacher_idx, teacher_logit, mask)
    dev = hidden.device
    if out is None:
        out = (torch.empty((), dtype=torch.float32, device=dev), torch.empty((T, d), dtype=torch.float32, device=dev),
               torch.empty((V, d), dtype=torch.float32, device=dev))
        if row_stats:
            out = out + (torch.empty(T, dtype=torch.float32, device=dev), torch.empty(T, dtype=torch.float32, device=dev))
    loss, gH, gW = out[:3]
    rl, rk = (out[3], out[4]) if row_stats else (None, None)
    for name, t, shape in (("loss", loss, ()), ("grad_hidden", gH, (T, d)), ("grad_W", gW, (V, d)),
                           ("row_lse", rl, (T,)), ("row_kl", rk, (T,))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()):
            raise ValueError(f"out: {name} must be a contiguous float32 tensor of shape {shape}")
    _check_device(dev, loss=loss, grad_hidden=gH, grad_W=gW, row_lse=rl, row_kl=rk, status=status)
    _check_workspace(None, status)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = L.kd_topk_kl_fwd_bwd_noalloc(_ptr(hidden), _ptr(W), dt, _ptr(teacher_idx), _ptr(teacher_logit),
                                      _ptr(mask), T, d, V, K, float(tau), int(chunk), _ptr(loss), _ptr(gH),
                                      _ptr(gW), _ptr(rl), _ptr(rk), _ptr(status), ctypes.c_void_p(stream))
    if rc != 0:
        raise KdError(rc)
    return (loss, gH, gW, rl, rk) if row_stats else (loss, gH, gW)


def mfma_probe(out, blocks: int, iters: int, zero_operands: bool = False) -> None:
    """Enqueue the sustained-MFMA-ceiling probe (kd_mfma_probe) on the
    current stream; `out` is a float32 device tensor of blocks * 512
    elements.  64 * iters MFMAs of 32768 FLOPs per wave, 8 waves per block."""
    import torch
    if out.dtype != torch.float32 or out.numel() < blocks * 512 or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out: contiguous float32 CUDA tensor with blocks * 512 elements")
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib().kd_mfma_probe(int(blocks), int(iters), 1 if zero_operands else 0, _ptr(out), ctypes.c_void_p(stream))
    if rc != 0:
        raise KdError(rc)


def topk_cache_workspace_bytes(T: int, d: int, V: int, K: int, chunk: int, dtype: int) -> int:
    return int(lib().kd_topk_cache_workspace_bytes(T, d, V, K, chunk, dtype))


def topk_cache(hidden, W, K: int = 100, chunk: int = 2048, workspace=None, events=None):
    """Offline top-K cache of a teacher head (kd_topk_cache_build): returns
    (idx [T,K] int32, logit [T,K] float32), per row the K largest logits of
    hidden @ W^T in descending order (equal logits: lower id first).
    `events`, for measurement only: 2 * (KD_CACHE_PHASES * nchunks + 1)
    already-recorded torch.cuda.Event objects (kd_topk_cache_build_timed)."""
    import torch
    T, d = hidden.shape
    V = W.shape[0]
    if hidden.dtype == torch.bfloat16:
        dt = KD_BF16
    elif hidden.dtype == torch.float32:
        dt = KD_F32
    else:
        raise TypeError("hidden must be bfloat16 or float32")
    if W.dtype != hidden.dtype or W.shape[1] != d or not (hidden.is_contiguous() and W.is_contiguous()):
        raise ValueError("hidden [T,d] and W [V,d]: contiguous, same dtype")
    if not hidden.is_cuda:
        raise ValueError("hidden must be a CUDA tensor")
    dev = hidden.device
    _check_device(dev, W=W, workspace=workspace)
    _check_workspace(workspace, None)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    logit = torch.empty((T, K), dtype=torch.float32, device=dev)
    nbytes = topk_cache_workspace_bytes(T, d, V, K, chunk, dt)
    if nbytes == 0:
        raise KdError(2)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (_ptr(hidden), _ptr(W), dt, T, d, V, K, int(chunk), _ptr(idx), _ptr(logit), _ptr(workspace),
            workspace.numel(), ctypes.c_void_p(stream))
    if events is None:
        rc = lib().kd_topk_cache_build(*args)
    else:
        rc = lib().kd_topk_cache_build_timed(*args, _events(events, 2 * (KD_CACHE_PHASES * _nchunks(T, chunk) + 1)))
    if rc != 0:
        raise KdError(rc)
    return idx, logit


def fwd(hidden, W, teacher_idx, teacher_logit, mask=None, tau: float = 1.0, chunk: int = 2048,
        row_kl: bool = False, workspace=None, status=None, events=None):
    """Forward only (kd_topk_kl_fwd).  Returns (loss [0-d float32], row_lse
    [T] float32) and, with row_kl, also the per-row KL [T].  row_lse is what
    bwd() needs.  `events`: as for fwd_bwd (kd_topk_kl_fwd_timed)."""
    import torch
    T, d, V, K, dt = _check_inputs(hidden, W, teacher_idx, teacher_logit, mask)
    dev = hidden.device
    _check_device(dev, workspace=workspace, status=status)
    _check_workspace(workspace, status)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    rl = torch.empty(T, dtype=torch.float32, device=dev)
    rk = torch.empty(T, dtype=torch.float32, device=dev) if row_kl else None
    nbytes = fwd_workspace_bytes(T, d, V, K, chunk, dt)
    if nbytes == 0:
        raise KdError(2)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (_ptr(hidden), _ptr(W), dt, _ptr(teacher_idx), _ptr(teacher_logit), _ptr(mask), T, d, V, K,
            float(tau), int(chunk), _ptr(loss), _ptr(rl), _ptr(rk), _ptr(workspace), workspace.numel(),
            _ptr(status), ctypes.c_void_p(stream))
    if events is None:
        rc = lib().kd_topk_kl_fwd(*args)
    else:
        rc = lib().kd_topk_kl_fwd_timed(*args, _loss_events(events, T, chunk))
    if rc != 0:
        raise KdError(rc)
    return (loss, rl, rk) if row_kl else (loss, rl)


def bwd(hidden, W, teacher_idx, teacher_logit, mask, row_lse, tau: float = 1.0, chunk: int = 2048,
        grad_loss=None, grad_hidden="float32", grad_W=True, accumulate_into=None, grad_W_bf16: bool = False,
        workspace=None, status=None, events=None):
    """Backward only (kd_topk_kl_bwd): gradients of grad_loss * loss.

    grad_loss: 0-d float32 CUDA tensor or None (= 1).  grad_hidden:
    "float32", "bfloat16" or None (not computed).  grad_W: True (a new fp32
    [V,d] tensor), False (not computed); accumulate_into: an fp32 [V,d] CUDA
    tensor that the head gradient is added to instead (returned as grad_W).
    grad_W_bf16: also return a bf16 copy of the final grad_W.  Returns
    (grad_hidden, grad_W, grad_W_bf16), with None for what was not asked.
    `events`: as for fwd_bwd (kd_topk_kl_bwd_timed)."""
    import torch
    T, d, V, K, dt = _check_inputs(hidden, W, teacher_idx, teacher_logit, mask)
    dev = hidden.device
    _check_device(dev, row_lse=row_lse, grad_loss=grad_loss, accumulate_into=accumulate_into,
                  workspace=workspace, status=status)
    _check_workspace(workspace, status)
    if row_lse.dtype != torch.float32 or tuple(row_lse.shape) != (T,) or not row_lse.is_contiguous():
        raise ValueError("row_lse must be a contiguous float32 [T] tensor")
    if grad_loss is not None and (grad_loss.dtype != torch.float32 or grad_loss.numel() != 1):
        raise ValueError("grad_loss must be a one-element float32 tensor")
    gh_dt = {"float32": (KD_F32, torch.float32), "bfloat16": (KD_BF16, torch.bfloat16), None: (KD_F32, None)}
    if grad_hidden not in gh_dt:
        raise ValueError("grad_hidden must be 'float32', 'bfloat16' or None")
    gh_code, gh_torch = gh_dt[grad_hidden]
    gH = torch.empty((T, d), dtype=gh_torch, device=dev) if gh_torch is not None else None
    if accumulate_into is not None:
        if accumulate_into.dtype != torch.float32 or tuple(accumulate_into.shape) != (V, d) \
                or not accumulate_into.is_contiguous():
            raise ValueError("accumulate_into must be a contiguous float32 [V,d] tensor")
        gW, acc = accumulate_into, 1
    else:
        gW, acc = (torch.empty((V, d), dtype=torch.float32, device=dev) if grad_W else None), 0
    gWb = torch.empty((V, d), dtype=torch.bfloat16, device=dev) if (grad_W_bf16 and gW is not None) else None
    nbytes = bwd_workspace_bytes(T, d, V, K, chunk, dt)
    if nbytes == 0:
        raise KdError(2)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (_ptr(hidden), _ptr(W), dt, _ptr(teacher_idx), _ptr(teacher_logit), _ptr(mask), T, d, V, K,
            float(tau), int(chunk), _ptr(row_lse), _ptr(grad_loss), _ptr(gH), gh_code, _ptr(gW), acc, _ptr(gWb),
            _ptr(workspace), workspace.numel(), _ptr(status), ctypes.c_void_p(stream))
    if events is None:
        rc = lib().kd_topk_kl_bwd(*args)
    else:
        rc = lib().kd_topk_kl_bwd_timed(*args, _loss_events(events, T, chunk))
    if rc != 0:
        raise KdError(rc)
    return gH, gW, gWb


def _autograd_function():
    import torch

    class KdTopKKLFunction(torch.autograd.Function):
        """The fused chunked top-K KL loss as an autograd node.

        forward(hidden, W, teacher_idx, teacher_logit, mask, tau, chunk,
        grad_W_accumulator) -> loss (0-d float32).  Only the per-row
        logsumexp is saved besides the inputs; the backward recomputes each
        chunk's logits.  The hidden gradient comes back in hidden's dtype.
        The head gradient: with a grad_W_accumulator (fp32 [V,d], e.g. a
        master-weight gradient buffer) it is added there in fp32 and W gets
        no .grad; otherwise it is returned in W's dtype."""

        @staticmethod
        def forward(ctx, hidden, W, teacher_idx, teacher_logit, mask, tau, chunk, grad_W_accumulator):
            loss, row_lse = fwd(hidden, W, teacher_idx, teacher_logit, mask, tau, chunk)
            ctx.save_for_backward(hidden, W, teacher_idx, teacher_logit, mask, row_lse)
            ctx.tau, ctx.chunk, ctx.acc = tau, chunk, grad_W_accumulator
            return loss

        @staticmethod
        def backward(ctx, grad_loss):
            hidden, W, teacher_idx, teacher_logit, mask, row_lse = ctx.saved_tensors
            need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
            if not (need_h or need_w):
                return (None,) * 8
            g = grad_loss.reshape(()).to(torch.float32).contiguous()
            gh_kind = ("bfloat16" if hidden.dtype == torch.bfloat16 else "float32") if need_h else None
            use_acc = need_w and ctx.acc is not None
            gH, gW, gWb = bwd(hidden, W, teacher_idx, teacher_logit, mask, row_lse, ctx.tau, ctx.chunk,
                              grad_loss=g, grad_hidden=gh_kind, grad_W=need_w and not use_acc,
                              accumulate_into=ctx.acc if use_acc else None,
                              grad_W_bf16=need_w and not use_acc and W.dtype == torch.bfloat16)
            if not need_w or use_acc:
                dW = None
            else:
                dW = gWb if W.dtype == torch.bfloat16 else gW
            return gH, dW, None, None, None, None, None, None

    return KdTopKKLFunction


_FN = None


def __getattr__(name):
    global _FN
    if name == "KdTopKKLFunction":
        if _FN is None:
            _FN = _autograd_function()
        return _FN
    raise AttributeError(name)


def kd_topk_kl_loss(hidden, W, teacher_idx, teacher_logit, mask=None, tau: float = 1.0, chunk: int = 2048,
                    grad_W_accumulator=None):
    """Differentiable loss: tau^2 * masked mean over positions of
    KL(teacher top-K softmax || student full-vocabulary softmax), computed
    and differentiated by the HIP library."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    return _FN.apply(hidden, W, teacher_idx, teacher_logit, mask, tau, chunk, grad_W_accumulator)

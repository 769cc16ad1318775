"""MI355X fused chunked top-K KL distillation loss: thin Python binding.

The computation runs entirely in the HIP library libkdtopk.so (C ABI in
include/kd_topk_kl.h).  This module only marshals arguments: PyTorch supplies
device memory (torch.empty) and the current stream.  If the library is not
built, every entry point raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["KD_BF16", "KD_F32", "KD_NUM_PHASES", "PHASES", "KdError", "lib", "workspace_bytes", "fwd_bwd",
           "status_str", "STATUS"]

KD_BF16 = 0
KD_F32 = 1
KD_NUM_PHASES = 8
PHASES = ("chunk_prep", "gemm_fwd_lse", "kl_rows", "gemm_bwd_grad", "scatter_sparse",
          "gemm_dhidden", "dhidden_reduce", "gemm_dW")
STATUS = {0: "KD_OK", 1: "KD_ERR_NULL_ARG", 2: "KD_ERR_BAD_SHAPE", 3: "KD_ERR_BAD_TAU",
          4: "KD_ERR_BAD_CHUNK", 5: "KD_ERR_DTYPE", 6: "KD_ERR_WORKSPACE",
          7: "KD_ERR_BAD_INDEX", 8: "KD_ERR_HIP"}

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
        L.kd_topk_kl_fwd_bwd_timed.argtypes = L.kd_topk_kl_fwd_bwd.argtypes + [vp]
        L.kd_topk_kl_fwd_bwd_timed.restype = i32
        L.kd_status_str.argtypes = [i32]
        L.kd_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().kd_status_str(int(code)).decode()


def workspace_bytes(T: int, d: int, V: int, K: int, chunk: int, dtype: int) -> int:
    return int(lib().kd_topk_kl_workspace_bytes(T, d, V, K, chunk, dtype))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


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
    if mask is not None and mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8")
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
        arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        rc = L.kd_topk_kl_fwd_bwd_timed(*args, arr)
    if rc != 0:
        raise KdError(rc)
    if row_stats:
        return loss, gH, gW, rl, rk
    return loss, gH, gW

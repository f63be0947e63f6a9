"""ctypes binding of the KDA C ABI (include/kda.h).

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity, their device pointers and the current HIP stream are passed to
libkda.so, and a non-OK status raises.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1

_vp = ctypes.c_void_p
_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by gated_delta_rule_81_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gated_delta_rule_81_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.kda_fwd_workspace_bytes.argtypes = [ctypes.c_int] * 6
    L.kda_fwd_chunked.restype = ctypes.c_int
    L.kda_fwd_chunked.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, device, dtype=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, num_seqs: int) -> int:
    return int(lib().kda_fwd_workspace_bytes(B, T, H, dk, dv, num_seqs))


def fwd_chunked(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *,
                output_final_state: bool = True, o=None, S_T=None,
                workspace=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA forward (kda_fwd_chunked).

    q, k, log_alpha: (B, T, H, dk); v: (B, T, H, dv); beta: (B, T, H), all of
    one dtype (bf16 or fp32) on one GPU.  S0: (N, H, dk, dv) fp32 or None.
    cu_seqlens: int32 (N+1,) on the same GPU (requires B == 1) or None.
    Returns (o, S_T); S_T is None when output_final_state is False.
    """
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        _check(t, name, dev, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (B, T, H, dv) \
            or beta.shape != (B, T, H):
        raise ValueError("inconsistent input shapes")
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    if S0 is not None:
        _check(S0, "S0", dev, torch.float32)
        if S0.shape != (N, H, dk, dv):
            raise ValueError(f"S0 must have shape {(N, H, dk, dv)}")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt)
    if output_final_state and S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if S_T is not None:
        _check(S_T, "S_T", dev, torch.float32)
    need = workspace_bytes(B, T, H, dk, dv, N) if cu_seqlens is not None else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().kda_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                               _ptr(S0), _ptr(cu_seqlens), N, B, T, H, dk, dv,
                               _dtype_code(q), _ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes,
                               _stream(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_fwd_chunked")
    return o, S_T


def decode_step(q, k, v, log_alpha, beta, S_cache, *, o=None) -> torch.Tensor:
    """One-token KDA update of S_cache in place (kda_decode_step); returns o.

    q, k, log_alpha: (N, H, dk); v: (N, H, dv); beta: (N, H) of one dtype;
    S_cache: (N, H, dk, dv) fp32.
    """
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        _check(t, name, dev, dt)
    _check(S_cache, "S_cache", dev, torch.float32)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape != (N, H, dv) \
            or beta.shape != (N, H) or S_cache.shape != (N, H, dk, dv):
        raise ValueError("inconsistent input shapes")
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt)
    st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                               _ptr(S_cache), N, H, dk, dv, _dtype_code(q), _ptr(o),
                               _stream(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return o

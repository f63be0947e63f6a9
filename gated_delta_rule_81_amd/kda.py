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
KDA_ERR_SCRATCH_LIMIT = 4
NOALLOC_MAX_SEQS = 65536
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_CHANNEL, KDA_GATE_HEAD, KDA_GATE_NONE = 0, 1, 2
_GATES = {"channel": KDA_GATE_CHANNEL, "head": KDA_GATE_HEAD, "none": KDA_GATE_NONE}
KDA_FLAG_L2NORM_QK, KDA_FLAG_GATE_SOFTPLUS = 1, 2
KDA_DEVERR_WAIT_TIMEOUT = 1
WAIT_LIMIT_DEFAULT = 1 << 20

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
    L.kda_fwd_chunked_ex.restype = ctypes.c_int
    L.kda_fwd_chunked_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_uint, _vp, _vp, _vp,
                                     ctypes.c_int, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp,
                                     _vp, ctypes.c_size_t, _vp]
    L.kda_decode_step_ex.restype = ctypes.c_int
    L.kda_decode_step_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_uint, _vp, _vp,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]
    L.kda_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.kda_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 6
    L.kda_bwd_chunked.restype = ctypes.c_int
    L.kda_bwd_chunked.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.kda_fwd_chunked_noalloc.restype = ctypes.c_int
    L.kda_fwd_chunked_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_uint, _vp,
                                          _vp, _vp, ctypes.c_int, _vp, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, _vp, _vp]
    L.kda_device_errors.restype = ctypes.c_int
    L.kda_device_errors.argtypes = [ctypes.POINTER(ctypes.c_uint), ctypes.c_int, _vp]
    L.kda_set_wait_limit.restype = ctypes.c_int
    L.kda_set_wait_limit.argtypes = [ctypes.c_int]
    # measurement kernels (include/kda_measure.h)
    L.kda_measure_copy.restype = ctypes.c_int
    L.kda_measure_copy.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
    L.kda_measure_rmw.restype = ctypes.c_int
    L.kda_measure_rmw.argtypes = [_vp, ctypes.c_size_t, _vp]
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


def _gate_code(gate: str) -> int:
    if gate not in _GATES:
        raise ValueError(f"gate must be one of {sorted(_GATES)}, got {gate!r}")
    return _GATES[gate]


def _check_gate(log_alpha, gate: str, shape_k, dev, dt):
    """log_alpha's expected shape: per key channel, per (token, head), or unused."""
    code = _gate_code(gate)
    if code == KDA_GATE_NONE:
        return code
    if log_alpha is None:
        raise ValueError(f"log_alpha is required for gate={gate!r}")
    _check(log_alpha, "log_alpha", dev, dt)
    want = tuple(shape_k) if code == KDA_GATE_CHANNEL else tuple(shape_k[:-1])
    if tuple(log_alpha.shape) != want:
        raise ValueError(f"log_alpha must have shape {want} for gate={gate!r}")
    return code


def fwd_chunked(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *,
                output_final_state: bool = True, o=None, S_T=None,
                workspace=None, gate: str = "channel", state_idx=None,
                pool_size: Optional[int] = None,
                flags: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA forward (kda_fwd_chunked / kda_fwd_chunked_ex).

    q, k: (B, T, H, dk); v: (B, T, H, dv); beta: (B, T, H), all of one dtype
    (bf16 or fp32) on one GPU.  log_alpha: (B, T, H, dk) for gate="channel",
    (B, T, H) for gate="head", ignored (may be None) for gate="none".
    S0: (N, H, dk, dv) fp32 or None.  cu_seqlens: int32 (N+1,) on the same GPU
    (requires B == 1) or None.  With state_idx (int32 (N,), on the GPU), S0 and
    S_T are pools of pool_size rows (default: S0's or S_T's first dimension)
    and sequence s reads and writes row state_idx[s]; S_T is then never
    allocated here (pass S_T=S0 to continue a pool in place).  flags: input
    preparation, KDA_FLAG_L2NORM_QK | KDA_FLAG_GATE_SOFTPLUS (kda.h kda_flags).
    Returns (o, S_T); S_T is None when output_final_state is False.
    """
    _gate_code(gate)
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _check(t, name, dev, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gcode = _check_gate(log_alpha, gate, q.shape, dev, dt)
    if k.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("inconsistent input shapes")
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    if state_idx is not None:
        _check(state_idx, "state_idx", dev, torch.int32)
        if state_idx.shape != (N,):
            raise ValueError(f"state_idx must have shape {(N,)}")
        if pool_size is None:
            ref = S0 if S0 is not None else S_T
            pool_size = ref.shape[0] if ref is not None else 0
        rows = pool_size
    else:
        rows = N
    if S0 is not None:
        _check(S0, "S0", dev, torch.float32)
        if S0.shape != (rows, H, dk, dv):
            raise ValueError(f"S0 must have shape {(rows, H, dk, dv)}")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt)
    if output_final_state and S_T is None and state_idx is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if S_T is not None:
        _check(S_T, "S_T", dev, torch.float32)
        if S_T.shape != (rows, H, dk, dv):
            raise ValueError(f"S_T must have shape {(rows, H, dk, dv)}")
    need = workspace_bytes(B, T, H, dk, dv, N) if cu_seqlens is not None else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ga = None if gcode == KDA_GATE_NONE else log_alpha
    if gcode == KDA_GATE_CHANNEL and state_idx is None and not flags:
        st = lib().kda_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(beta),
                                   _ptr(S0), _ptr(cu_seqlens), N, B, T, H, dk, dv,
                                   _dtype_code(q), _ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes,
                                   _stream(dev))
        where = "kda_fwd_chunked"
    else:
        st = lib().kda_fwd_chunked_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(beta), gcode,
                                      int(flags), _ptr(S0), _ptr(S_T), _ptr(state_idx), int(rows),
                                      _ptr(cu_seqlens), N, B, T, H, dk, dv, _dtype_code(q),
                                      _ptr(o), _ptr(workspace), ws_bytes, _stream(dev))
        where = "kda_fwd_chunked_ex"
    if st != KDA_OK:
        raise KdaError(st, where)
    return o, S_T


def decode_step(q, k, v, log_alpha, beta, S_cache, *, o=None, gate: str = "channel",
                state_idx=None, flags: int = 0) -> torch.Tensor:
    """KDA decode of S_cache in place (kda_decode_step / _ex); returns o.

    One token per sequence: q, k: (N, H, dk); v: (N, H, dv); beta: (N, H);
    or L consecutive tokens per sequence: q, k: (N, L, H, dk); v: (N, L, H, dv);
    beta: (N, L, H), all of one dtype.  log_alpha has q's shape for
    gate="channel", beta's for gate="head", and is ignored for gate="none".
    S_cache: (N, H, dk, dv) fp32, or with state_idx (int32 (N,) on the GPU) a
    pool (P, H, dk, dv) whose row state_idx[n] sequence n updates.  flags: input
    preparation (kda.h kda_flags).
    """
    _gate_code(gate)
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _check(t, name, dev, dt)
    _check(S_cache, "S_cache", dev, torch.float32)
    if q.dim() == 4:
        N, L, H, dk = q.shape
    else:
        (N, H, dk), L = q.shape, 1
    dv = v.shape[-1]
    gcode = _check_gate(log_alpha, gate, q.shape, dev, dt)
    tok = (N, L, H) if q.dim() == 4 else (N, H)
    rows = N
    if state_idx is not None:
        _check(state_idx, "state_idx", dev, torch.int32)
        if state_idx.shape != (N,):
            raise ValueError(f"state_idx must have shape {(N,)}")
        rows = S_cache.shape[0]
    if k.shape != q.shape or v.shape != tok + (dv,) or beta.shape != tok \
            or S_cache.shape != (rows, H, dk, dv):
        raise ValueError("inconsistent input shapes")
    if o is None:
        o = torch.empty(tok + (dv,), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt)
    ga = None if gcode == KDA_GATE_NONE else log_alpha
    if gcode == KDA_GATE_CHANNEL and state_idx is None and L == 1 and not flags:
        st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(beta),
                                   _ptr(S_cache), N, H, dk, dv, _dtype_code(q), _ptr(o),
                                   _stream(dev))
        where = "kda_decode_step"
    else:
        st = lib().kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(beta), gcode,
                                      int(flags), _ptr(S_cache), _ptr(state_idx), int(rows), N, L, H, dk, dv,
                                      _dtype_code(q), _ptr(o), _stream(dev))
        where = "kda_decode_step_ex"
    if st != KDA_OK:
        raise KdaError(st, where)
    return o


def bwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, num_seqs: int) -> int:
    return int(lib().kda_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs))


def bwd_chunked(q, k, v, log_alpha, beta, dO, S0=None, dS_T=None, cu_seqlens=None, *,
                gate: str = "channel", workspace=None, out=None):
    """Gradients through fwd_chunked (kda_bwd_chunked).

    Inputs exactly as given to fwd_chunked (no flags, no slot map), plus dO
    (like o) and dS_T ((N, H, dk, dv) fp32 or None).  workspace: a uint8 GPU
    tensor of at least bwd_workspace_bytes(...) bytes (allocated here when
    None).  out: optional preallocated (dq, dk, dv, dlog_alpha, dbeta, dS0).
    Returns (dq, dk, dv, dlog_alpha, dbeta, dS0); dlog_alpha is None for
    gate="none" and has log_alpha's shape otherwise.
    """
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("dO", dO)):
        _check(t, name, dev, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gcode = _check_gate(log_alpha, gate, q.shape, dev, dt)
    if (k.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H)
            or dO.shape != v.shape):
        raise ValueError("inconsistent input shapes")
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _check(t, name, dev, torch.float32)
            if t.shape != (N, H, dk, dv):
                raise ValueError(f"{name} must have shape {(N, H, dk, dv)}")
    if out is None:
        dq = torch.empty_like(q)
        dk_ = torch.empty_like(k)
        dv_ = torch.empty_like(v)
        dg = None if gcode == KDA_GATE_NONE else torch.empty_like(log_alpha)
        db = torch.empty_like(beta)
        dS0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        dq, dk_, dv_, dg, db, dS0 = out
        for name, t, like in (("dq", dq, q), ("dk", dk_, k), ("dv", dv_, v), ("dbeta", db, beta)):
            _check(t, name, dev, dt)
            if t.shape != like.shape:
                raise ValueError(f"{name} must have shape {tuple(like.shape)}")
        if gcode != KDA_GATE_NONE:
            _check(dg, "dlog_alpha", dev, dt)
            if dg.shape != log_alpha.shape:
                raise ValueError("dlog_alpha must have log_alpha's shape")
        if dS0 is not None:
            _check(dS0, "dS0", dev, torch.float32)
            if dS0.shape != (N, H, dk, dv):
                raise ValueError(f"dS0 must have shape {(N, H, dk, dv)}")
    need = bwd_workspace_bytes(B, T, H, dk, dv, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    ga = None if gcode == KDA_GATE_NONE else log_alpha
    st = lib().kda_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(beta), gcode, _ptr(S0),
                               _ptr(dO), _ptr(dS_T), _ptr(cu_seqlens), N, B, T, H, dk, dv,
                               _dtype_code(q), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db),
                               _ptr(dS0), _ptr(workspace), ws_bytes, _stream(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_bwd_chunked")
    return dq, dk_, dv_, dg, db, dS0


def device_errors(clear: bool = False, device=None) -> int:
    """The current device's sticky error bits (kda_device_errors), after
    synchronising the current stream; KDA_DEVERR_WAIT_TIMEOUT when a bounded
    wait inside a kernel ran out.  clear=True resets them."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    bits = ctypes.c_uint(0)
    with torch.cuda.device(dev):
        st = lib().kda_device_errors(ctypes.byref(bits), int(bool(clear)), _stream(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_device_errors")
    return int(bits.value)


def set_wait_limit(polls: int) -> None:
    """Diagnostics (kda_set_wait_limit): polls a bounded wait makes before it
    gives up, process-wide, for launches after the call."""
    st = lib().kda_set_wait_limit(int(polls))
    if st != KDA_OK:
        raise KdaError(st, "kda_set_wait_limit")


def measure_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """kda_measure_copy: dst = src byte for byte with the decode step's access
    pattern (include/kda_measure.h); both contiguous GPU tensors of equal size."""
    _check(src, "src", src.device)
    _check(dst, "dst", src.device)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst sizes differ")
    st = lib().kda_measure_copy(_ptr(src), _ptr(dst), n, _stream(src.device))
    if st != KDA_OK:
        raise KdaError(st, "kda_measure_copy")


def measure_rmw(buf: torch.Tensor) -> None:
    """kda_measure_rmw: every 16 bytes of buf read and written back in place."""
    _check(buf, "buf", buf.device)
    st = lib().kda_measure_rmw(_ptr(buf), buf.numel() * buf.element_size(), _stream(buf.device))
    if st != KDA_OK:
        raise KdaError(st, "kda_measure_rmw")


def fwd_chunked_noalloc(q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T=None, *,
                        gate: str = "channel", state_idx=None, pool_size: Optional[int] = None,
                        flags: int = 0) -> None:
    """kda_fwd_chunked_noalloc: the chunked forward into caller-given outputs
    (o, and S_T or None) with no workspace; nothing is allocated here or in
    the library.  Arguments as in fwd_chunked.  Calls that overlap on one GPU
    must not be issued (they share that GPU's scratch)."""
    dev = q.device
    dt = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("o", o)):
        _check(t, name, dev, dt)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gcode = _check_gate(log_alpha, gate, q.shape, dev, dt)
    if k.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H) \
            or o.shape != v.shape:
        raise ValueError("inconsistent input shapes")
    N = B
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
        N = cu_seqlens.shape[0] - 1
    rows = N
    if state_idx is not None:
        _check(state_idx, "state_idx", dev, torch.int32)
        if pool_size is None:
            ref = S0 if S0 is not None else S_T
            pool_size = ref.shape[0] if ref is not None else 0
        rows = pool_size
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None:
            _check(t, name, dev, torch.float32)
            if t.shape != (rows, H, dk, dv):
                raise ValueError(f"{name} must have shape {(rows, H, dk, dv)}")
    ga = None if gcode == KDA_GATE_NONE else log_alpha
    st = lib().kda_fwd_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(ga), _ptr(beta), gcode,
                                       int(flags), _ptr(S0), _ptr(S_T), _ptr(state_idx), int(rows),
                                       _ptr(cu_seqlens), N, B, T, H, dk, dv, _dtype_code(q), _ptr(o),
                                       _stream(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_fwd_chunked_noalloc")

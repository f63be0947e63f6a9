"""Python front end of the fp64 KDA oracle (test infrastructure only).

Two independent routes to the same result live here:

* ``fwd`` / ``decode`` call the literal token-by-token recurrence in
  ``kda_oracle.c`` (fp64, OpenMP over independent (sequence, head) units).
* ``brute_force`` builds, for tiny T, each token's full d_k x d_k transition
  matrix  M_t = (I - beta_t k_t k_t^T) Diag(alpha_t)  and multiplies them out:
  S_t = M_t S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.  That is the
  closed matrix form of the same update ("Diagonal-Plus-Low-Rank" transition,
  akshathtiwari.co.in "Kimi Delta Attention" explainer; per-key-channel
  diagonal gate, daily.dev summary of "You Could Have Come Up with Kimi Delta
  Attention").  It shares no code with the C loop.

Every function here is pinned by tests/test_oracle_pins.py (values the pages
print, closed forms, special cases that reduce to published recurrences, brute
force), and tests/test_oracle_mutants.py checks that planted mistakes in the C
loop fail those pins.

Inputs are numpy arrays of any float dtype; they are widened to float64
exactly (bf16 and fp32 values are exactly representable in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile kda_oracle.c with gcc into oracle/libkda_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    _lib = load_path(_LIB)
    return _lib


def load_path(path: str):
    """Load and bind an oracle library built from kda_oracle.c at ``path``."""
    lib = ctypes.CDLL(path)
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i64p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, _dp, _dp, ctypes.c_int]
    lib.kda_oracle_decode.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp,
                                      ctypes.c_int]
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    return lib


def max_threads() -> int:
    return int(load().kda_oracle_max_threads())


def default_threads() -> int:
    """OMP_NUM_THREADS when set (the host's CPU share), else the affinity mask size."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, len(os.sched_getaffinity(0)))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _dp)
    return a.ctypes.data_as(_dp)


def fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None,
        nthreads: Optional[int] = None, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Literal recurrence over whole sequences.

    q, k, log_alpha: (B, T, H, dk); v: (B, T, H, dv); beta: (B, T, H);
    S0: (N, H, dk, dv) or None (zeros); cu_seqlens: (N+1,) ints or None.
    Returns (o (B, T, H, dv), S_T (N, H, dk, dv)) as float64.
    """
    q, k, v, log_alpha, beta = map(_f64, (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and log_alpha.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        assert B == 1
    else:
        cu = None
        N = B
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_T = np.zeros((N, H, dk, dv), dtype=np.float64)
    lib = lib if lib is not None else load()
    nt = nthreads if nthreads else default_threads()
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                            _ptr(S0), cu.ctypes.data_as(_i64p) if cu is not None
                            else ctypes.cast(None, _i64p), N, B, T, H, dk, dv,
                            _ptr(o), _ptr(S_T), nt)
    if rc != 0:
        raise ValueError(f"kda_oracle_fwd rejected its arguments (rc={rc})")
    return o, S_T


def decode(q, k, v, log_alpha, beta, S, nthreads: Optional[int] = None, lib=None):
    """One token for each of N independent states.

    q, k, log_alpha: (N, H, dk); v: (N, H, dv); beta: (N, H); S: (N, H, dk, dv).
    Returns (o (N, H, dv), S_new (N, H, dk, dv)); the input S is not modified.
    """
    q, k, v, log_alpha, beta = map(_f64, (q, k, v, log_alpha, beta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    S_new = np.array(S, dtype=np.float64, copy=True, order="C")
    assert S_new.shape == (N, H, dk, dv)
    o = np.zeros((N, H, dv), dtype=np.float64)
    nt = nthreads if nthreads else default_threads()
    lib = lib if lib is not None else load()
    rc = lib.kda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  _ptr(S_new), N, H, dk, dv, _ptr(o), nt)
    if rc != 0:
        raise ValueError(f"kda_oracle_decode rejected its arguments (rc={rc})")
    return o, S_new


def brute_force(q, k, v, log_alpha, beta, S0=None):
    """Explicit transition-matrix products for tiny T (T <= 8).

    Same shapes as ``fwd`` without varlen.  For each (b, h):
      M_t = (I - beta_t k_t k_t^T) Diag(exp(log_alpha_t))      (d_k x d_k)
      S_t = M_t S_{t-1} + beta_t k_t v_t^T ,   o_t = S_t^T q_t
    """
    q, k, v, log_alpha, beta = map(_f64, (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if T > 8:
        raise ValueError("brute_force is meant for T <= 8")
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h].copy()
            for t in range(T):
                kt = k[b, t, h][:, None]
                M = (eye - beta[b, t, h] * (kt @ kt.T)) @ np.diag(np.exp(log_alpha[b, t, h]))
                S = M @ S + beta[b, t, h] * (kt @ v[b, t, h][None, :])
                o[b, t, h] = S.T @ q[b, t, h]
            S_T[b, h] = S
    return o, S_T

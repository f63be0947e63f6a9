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

``prepare`` applies the optional input preparation (L2-normalising q and k,
the softplus form of the gate), ``channel_gate`` restates the two narrower
gate layouts (one decay per head,
or none) as the per-channel gate they stand for, and ``fwd_pooled`` /
``decode_pooled`` read and write states as rows of a pool through a slot map;
both only rearrange inputs and outputs around ``fwd`` / ``decode``.

``bwd`` differentiates the token loop in reverse (kda_oracle_bwd); it is
pinned by tests/test_oracle_bwd.py (exact adjoint identities where the
forward is linear, central differences of ``fwd``, a closed form at beta = 0,
planted mistakes).

Every other function here is pinned by tests/test_oracle_pins.py (values the pages
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
    lib.kda_oracle_bwd.restype = ctypes.c_int
    lib.kda_oracle_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
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


GATES = ("channel", "head", "none")

# input preparation folded into the operator (flags of the *_ex entry points)
FLAG_L2NORM_QK = 1
FLAG_GATE_SOFTPLUS = 2


def prepare(q, k, gate_in, flags: int):
    """Inputs as the operator sees them after the optional preparation steps.

    FLAG_L2NORM_QK: q and k divided by their Euclidean norm over d_k, per token
    and head (a zero vector stays zero) -- the normalisation the workloads'
    generator applies before the operator.
    FLAG_GATE_SOFTPLUS: the gate tensor holds x and log_alpha = -softplus(x) =
    -log(1 + e^x), the forget-gate form of the workloads' generator; alpha =
    e^{-softplus(x)} lies in (0, 1).  None (no gate) stays None.
    Returns (q, k, log_alpha) as float64.
    """
    q = _f64(q)
    k = _f64(k)
    if flags & FLAG_L2NORM_QK:
        def unit(x):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)
        q, k = unit(q), unit(k)
    g = None if gate_in is None else _f64(gate_in)
    if g is not None and flags & FLAG_GATE_SOFTPLUS:
        g = -np.logaddexp(0.0, g)
    return q, k, g


def prepare_vjp(q_in, k_in, gate_in, flags: int, dq, dk, dg):
    """Gradients with respect to the raw inputs of ``prepare`` from those with
    respect to its outputs (the chain rule through each step):

    FLAG_L2NORM_QK: y = x / |x| gives dx = (dy - y (y . dy)) / |x| (zero for a
    zero row, where the step is the constant 0).
    FLAG_GATE_SOFTPLUS: g = -softplus(x) gives dx = -sigmoid(x) dg.
    Returns (dq_in, dk_in, dgate_in) as float64 (dgate_in None without a gate).
    """
    dq, dk = _f64(dq), _f64(dk)
    if flags & FLAG_L2NORM_QK:
        def back(x, dy):
            x = _f64(x)
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            safe = np.where(n > 0, n, 1.0)
            y = x / safe
            dx = (dy - y * np.sum(y * dy, axis=-1, keepdims=True)) / safe
            return np.where(n > 0, dx, 0.0)
        dq, dk = back(q_in, dq), back(k_in, dk)
    if dg is None:
        return dq, dk, None
    dg = _f64(dg)
    if flags & FLAG_GATE_SOFTPLUS:
        x = _f64(gate_in)
        dg = -np.exp(-np.logaddexp(0.0, -x)) * dg      # sigmoid(x), overflow-free
    return dq, dk, dg


def channel_gate(log_alpha, gate: str, shape_k) -> np.ndarray:
    """The per-key-channel log-gate that a gate layout stands for.

    "channel": log_alpha itself, shape (..., dk).
    "head": one value per (token, head), shape (...,), the same on every key
    channel -- the single decay per head and token of Gated DeltaNet, which
    KDA turns into one per key channel ("The fourth layer remembers",
    paragraph on the forget gate): repeated over dk.
    "none": alpha = 1, the plain delta rule of DeltaNet (akshathtiwari.co.in
    "Kimi Delta Attention" explainer, delta-rule paragraph): zeros.
    """
    shape_k = tuple(shape_k)
    if gate == "channel":
        g = _f64(log_alpha)
        assert g.shape == shape_k
        return g
    if gate == "head":
        g = _f64(log_alpha)
        assert g.shape == shape_k[:-1]
        return np.ascontiguousarray(np.repeat(g[..., None], shape_k[-1], axis=-1))
    if gate == "none":
        return np.zeros(shape_k)
    raise ValueError(f"unknown gate layout {gate!r}")


def fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None,
        nthreads: Optional[int] = None, lib=None, gate: str = "channel",
        flags: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Literal recurrence over whole sequences.

    q, k: (B, T, H, dk); v: (B, T, H, dv); beta: (B, T, H); log_alpha in the
    layout ``gate`` names (see channel_gate), or the softplus input with
    FLAG_GATE_SOFTPLUS (see prepare);
    S0: (N, H, dk, dv) or None (zeros); cu_seqlens: (N+1,) ints or None.
    Returns (o (B, T, H, dv), S_T (N, H, dk, dv)) as float64.
    """
    if flags:
        q, k, log_alpha = prepare(q, k, log_alpha, flags)
    log_alpha = channel_gate(log_alpha, gate, np.shape(q))
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


def decode(q, k, v, log_alpha, beta, S, nthreads: Optional[int] = None, lib=None,
           gate: str = "channel", flags: int = 0):
    """One token for each of N independent states.

    q, k: (N, H, dk); v: (N, H, dv); beta: (N, H); S: (N, H, dk, dv);
    log_alpha in the layout ``gate`` names (see channel_gate), prepared per
    ``flags`` (see prepare).
    Returns (o (N, H, dv), S_new (N, H, dk, dv)); the input S is not modified.
    """
    if flags:
        q, k, log_alpha = prepare(q, k, log_alpha, flags)
    log_alpha = channel_gate(log_alpha, gate, np.shape(q))
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


def bwd(q, k, v, log_alpha, beta, S0, dO, dS_T=None, cu_seqlens=None,
        nthreads: Optional[int] = None, lib=None, gate: str = "channel", flags: int = 0):
    """Gradients of L = <dO, o> + <dS_T, S_T> through ``fwd`` (same arguments).

    The token loop differentiated in reverse (kda_oracle_bwd in
    kda_oracle.c), then, for the narrower gate layouts, the per-channel gate
    gradient summed over the channels a per-head value stands for (none: no
    gate gradient), and the chain rule through the optional preparation.
    dO: like o (B, T, H, dv); dS_T: (N, H, dk, dv) or None (zero).
    Returns (dq, dk, dv, dlog_alpha, dbeta, dS0) as float64; dlog_alpha has
    the gate input's shape (None for gate "none"); dS0 has S_T's shape.
    """
    q_in, k_in, g_in = q, k, log_alpha
    if flags:
        q, k, log_alpha = prepare(q, k, log_alpha, flags)
    log_alpha = channel_gate(log_alpha, gate, np.shape(q))
    q, k, v, log_alpha, beta, dO = map(_f64, (q, k, v, log_alpha, beta, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert dO.shape == (B, T, H, dv)
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
    if dS_T is not None:
        dS_T = _f64(dS_T)
        assert dS_T.shape == (N, H, dk, dv)
    gq, gk, glog = (np.zeros((B, T, H, dk)) for _ in range(3))
    gv = np.zeros((B, T, H, dv))
    gb = np.zeros((B, T, H))
    gS0 = np.zeros((N, H, dk, dv))
    lib = lib if lib is not None else load()
    nt = nthreads if nthreads else default_threads()
    rc = lib.kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                            _ptr(dO), _ptr(dS_T), cu.ctypes.data_as(_i64p) if cu is not None
                            else ctypes.cast(None, _i64p), N, B, T, H, dk, dv,
                            _ptr(gq), _ptr(gk), _ptr(gv), _ptr(glog), _ptr(gb), _ptr(gS0), nt)
    if rc != 0:
        raise ValueError(f"kda_oracle_bwd rejected its arguments (rc={rc})")
    if gate == "head":
        glog = glog.sum(axis=-1)
    elif gate == "none":
        glog = None
    if flags:
        gq, gk, glog = prepare_vjp(q_in, k_in, g_in, flags, gq, gk, glog)
    return gq, gk, gv, glog, gb, gS0


def pool_rows(state_idx, pool_size: int) -> np.ndarray:
    """Pool row of each sequence, or -1 (no state) for an index outside [0, pool_size)."""
    idx = np.asarray(state_idx, dtype=np.int64)
    return np.where((idx >= 0) & (idx < pool_size), idx, -1)


def fwd_pooled(q, k, v, log_alpha, beta, S0_pool, state_idx, cu_seqlens=None, gate="channel",
               S_T_pool=None, pool_size: Optional[int] = None, nthreads: Optional[int] = None,
               lib=None, flags: int = 0):
    """Sequences continued from and into rows of state pools (slot-indexed states).

    Sequence s starts from row state_idx[s] of S0_pool (zeros when S0_pool is
    None or the index is outside the pool) and its final state replaces row
    state_idx[s] of a copy of S_T_pool; other rows are kept.  Pools have shape
    (P, H, dk, dv); P = pool_size, else the pools' first dimension.
    Returns (o, new S_T pool or None).
    """
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    if pool_size is None:
        ref = S0_pool if S0_pool is not None else S_T_pool
        pool_size = 0 if ref is None else np.shape(ref)[0]
    rows = pool_rows(state_idx, pool_size)
    N = rows.shape[0]
    S0 = np.zeros((N, H, dk, dv))
    if S0_pool is not None:
        pool0 = _f64(S0_pool)
        for s in range(N):
            if rows[s] >= 0:
                S0[s] = pool0[rows[s]]
    o, S_T = fwd(q, k, v, log_alpha, beta, S0, cu_seqlens, nthreads=nthreads, lib=lib, gate=gate,
                 flags=flags)
    if S_T_pool is None:
        return o, None
    new = np.array(S_T_pool, dtype=np.float64, copy=True)
    for s in range(N):
        if rows[s] >= 0:
            new[rows[s]] = S_T[s]
    return o, new


def decode_pooled(q, k, v, log_alpha, beta, pool, state_idx, gate="channel",
                  nthreads: Optional[int] = None, lib=None, flags: int = 0):
    """One token per sequence on rows of a state pool; returns (o, new pool).

    Sequence n updates row state_idx[n]; for an index outside the pool it
    starts from a zero state and writes nothing.
    """
    pool = np.array(pool, dtype=np.float64, copy=True)
    rows = pool_rows(state_idx, pool.shape[0])
    N = rows.shape[0]
    S = np.zeros((N,) + pool.shape[1:])
    for n in range(N):
        if rows[n] >= 0:
            S[n] = pool[rows[n]]
    o, S_new = decode(q, k, v, log_alpha, beta, S, nthreads=nthreads, lib=lib, gate=gate,
                      flags=flags)
    for n in range(N):
        if rows[n] >= 0:
            pool[rows[n]] = S_new[n]
    return o, pool


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

"""Pins for the oracle's backward (oracle.bwd), each independent of its code.

The backward is the gradient of L = <dO, o> + <dS_T, S_T> through the forward
token loop.  What fixes it without re-deriving its formulas:

* exact adjoint identities where the forward is linear: o is linear in q
  (S_T does not depend on q), and (o, S_T) are jointly linear in (v, S0) --
  with nothing written and nothing carried in the state is zero -- so
  <dO, o> = <dq, q>, and L = <dv, v> when S0 = 0, L = <dS0, S0> when v = 0;
* central differences of the (separately pinned) forward along random
  directions, for every input, across several checkpoint segments, with
  varlen sequences (one empty) and every gate layout and preparation flag;
* a closed form at beta = 0, where the state only decays,
  S_t = Diag(e^{G_t}) S0 with G_t the running sum of log_alpha:
  o_t = S_t^T q_t, so dq_t = S_t dO_t, dv = dk = 0, dS0 and dlog_alpha follow
  from sums over later tokens, and dbeta_t = (Lam_t^T k_t) . (v_t - S_t^T k_t)
  with Lam_t the gradient of the state after token t.

Each pin takes the oracle library (so planted mistakes can be run against
it) and raises AssertionError on a mismatch.
"""
import numpy as np

import oracle


def _inputs(rng, B, T, H, dk, dv, N=None, gate_mu=-0.3):
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk)) / np.sqrt(dk)
    v = rng.normal(size=(B, T, H, dv))
    g = -np.log1p(np.exp(rng.normal(gate_mu, 1.0, size=(B, T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.normal(size=(B, T, H))))
    N = B if N is None else N
    S0 = rng.normal(size=(N, H, dk, dv))
    dO = rng.normal(size=(B, T, H, dv))
    dST = rng.normal(size=(N, H, dk, dv))
    return q, k, v, g, beta, S0, dO, dST


def _loss(lib, q, k, v, g, beta, S0, dO, dST, cu=None, gate="channel", flags=0):
    o, ST = oracle.fwd(q, k, v, g, beta, S0, cu, lib=lib, gate=gate, flags=flags, nthreads=4)
    return float(np.sum(dO * o) + np.sum(dST * ST))


def _rel(a, b):
    return abs(a - b) / max(abs(a), abs(b), 1e-30)


def pin_adjoint_q(lib):
    """<dO, o> = <dq, q>: o is linear in q and S_T does not depend on it."""
    rng = np.random.default_rng(11)
    q, k, v, g, b, S0, dO, dST = _inputs(rng, 2, 70, 2, 5, 3)
    o, _ = oracle.fwd(q, k, v, g, b, S0, lib=lib, nthreads=4)
    dq = oracle.bwd(q, k, v, g, b, S0, dO, None, lib=lib, nthreads=4)[0]
    lhs, rhs = float(np.sum(dO * o)), float(np.sum(dq * q))
    assert _rel(lhs, rhs) < 1e-11, (lhs, rhs)


def pin_adjoint_v_s0(lib):
    """L = <dv, v> at S0 = 0 and L = <dS0, S0> at v = 0 (joint linearity)."""
    rng = np.random.default_rng(12)
    q, k, v, g, b, S0, dO, dST = _inputs(rng, 2, 70, 2, 5, 3)
    L = _loss(lib, q, k, v, g, b, None, dO, dST)
    dv = oracle.bwd(q, k, v, g, b, None, dO, dST, lib=lib, nthreads=4)[2]
    assert _rel(L, float(np.sum(dv * v))) < 1e-11, (L, float(np.sum(dv * v)))
    z = np.zeros_like(v)
    L = _loss(lib, q, k, z, g, b, S0, dO, dST)
    dS0 = oracle.bwd(q, k, z, g, b, S0, dO, dST, lib=lib, nthreads=4)[5]
    assert _rel(L, float(np.sum(dS0 * S0))) < 1e-11, (L, float(np.sum(dS0 * S0)))


def _check_fd(lib, args, grads, cu=None, gate="channel", flags=0, h=1e-5, tol=1e-6, seed=0):
    """Central difference of L along a random direction for each input."""
    rng = np.random.default_rng(seed)
    names = ("q", "k", "v", "log_alpha", "beta", "S0")
    for i, name in enumerate(names):
        x = args[i]
        if x is None or grads[i] is None:
            continue
        d = rng.normal(size=np.shape(x))
        plus = list(args)
        minus = list(args)
        plus[i] = x + h * d
        minus[i] = x - h * d
        fd = (_loss(lib, *plus, cu=cu, gate=gate, flags=flags)
              - _loss(lib, *minus, cu=cu, gate=gate, flags=flags)) / (2 * h)
        an = float(np.sum(grads[i] * d))
        scale = max(abs(fd), abs(an), 1.0)
        assert abs(fd - an) / scale < tol, (name, fd, an)


def pin_fd_dense(lib):
    """Every input's gradient against central differences (T spans 3 segments)."""
    rng = np.random.default_rng(13)
    q, k, v, g, b, S0, dO, dST = _inputs(rng, 2, 150, 2, 4, 3)
    grads = oracle.bwd(q, k, v, g, b, S0, dO, dST, lib=lib, nthreads=4)
    _check_fd(lib, (q, k, v, g, b, S0, dO, dST), grads, seed=1)


def pin_fd_varlen(lib):
    """Packed sequences (one empty, one a single token) against central differences."""
    rng = np.random.default_rng(14)
    lens = [37, 0, 1, 90]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, b, S0, dO, dST = _inputs(rng, 1, int(cu[-1]), 2, 4, 3, N=len(lens))
    grads = oracle.bwd(q, k, v, g, b, S0, dO, dST, cu_seqlens=cu, lib=lib, nthreads=4)
    _check_fd(lib, (q, k, v, g, b, S0, dO, dST), grads, cu=cu, seed=2)
    # the empty sequence passes dS_T straight through to dS0
    assert np.array_equal(grads[5][1], dST[1])


def pin_fd_gates_and_flags(lib):
    """Per-head and absent gates, and the fused preparation, against central differences."""
    rng = np.random.default_rng(15)
    q, k, v, g, b, S0, dO, dST = _inputs(rng, 1, 40, 2, 4, 3)
    gh = g[..., 0].copy()
    grads = oracle.bwd(q, k, v, gh, b, S0, dO, dST, lib=lib, gate="head", nthreads=4)
    assert grads[3].shape == gh.shape
    _check_fd(lib, (q, k, v, gh, b, S0, dO, dST), grads, gate="head", seed=3)
    grads = oracle.bwd(q, k, v, None, b, S0, dO, dST, lib=lib, gate="none", nthreads=4)
    assert grads[3] is None
    _check_fd(lib, (q, k, v, None, b, S0, dO, dST), grads, gate="none", seed=4)
    flags = oracle.FLAG_L2NORM_QK | oracle.FLAG_GATE_SOFTPLUS
    x = rng.normal(-1.0, 1.5, size=g.shape)             # raw gate input
    qs, ks = q * 3.0, k * 0.2                            # rows far from unit norm
    grads = oracle.bwd(qs, ks, v, x, b, S0, dO, dST, lib=lib, flags=flags, nthreads=4)
    _check_fd(lib, (qs, ks, v, x, b, S0, dO, dST), grads, flags=flags, seed=5)


def pin_closed_form_beta0(lib):
    """beta = 0: decay only; every gradient in closed form."""
    rng = np.random.default_rng(16)
    B, T, H, dk, dv = 1, 12, 1, 3, 2
    q, k, v, g, _, S0, dO, dST = _inputs(rng, B, T, H, dk, dv)
    b = np.zeros((B, T, H))
    dq, dk_, dv_, dg, db, dS0 = oracle.bwd(q, k, v, g, b, S0, dO, dST, lib=lib, nthreads=1)
    G = np.cumsum(g[0, :, 0], axis=0)                   # (T, dk), G_t = sum_{j<=t} g_j
    S = [np.exp(G[t])[:, None] * S0[0, 0] for t in range(T)]
    # gradient of the state after token t: later outputs and the final state
    Lam = [None] * T
    acc = dST[0, 0].copy()
    for t in range(T - 1, -1, -1):
        acc = acc + np.outer(q[0, t, 0], dO[0, t, 0])
        Lam[t] = acc.copy()
        if t > 0:
            acc = np.exp(g[0, t, 0])[:, None] * acc
    ref_dq = np.stack([S[t] @ dO[0, t, 0] for t in range(T)])
    ref_dS0 = np.exp(g[0, 0, 0])[:, None] * Lam[0]
    # d/dg_j of sum_t <Lam-part> : every later state scales by e^{g_j}
    contrib = [np.sum(np.outer(q[0, t, 0], dO[0, t, 0]) * S[t], axis=1) for t in range(T)]
    final = np.sum(dST[0, 0] * S[T - 1], axis=1)
    ref_dg = np.stack([sum(contrib[t] for t in range(j, T)) + final for j in range(T)])
    ref_db = np.stack([(Lam[t].T @ k[0, t, 0]) @ (v[0, t, 0] - S[t].T @ k[0, t, 0])
                       for t in range(T)])
    np.testing.assert_allclose(dq[0, :, 0], ref_dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dS0[0, 0], ref_dS0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dg[0, :, 0], ref_dg, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db[0, :, 0], ref_db, rtol=1e-12, atol=1e-12)
    assert np.all(dk_ == 0) and np.all(dv_ == 0)


BWD_PINS = [pin_adjoint_q, pin_adjoint_v_s0, pin_fd_dense, pin_fd_varlen,
            pin_fd_gates_and_flags, pin_closed_form_beta0]

"""The chunkwise (WY / UT-transform) form of the KDA recurrence, in fp64 numpy.

Test-side derivation, used as an independent route to the oracle's result
(pin_chunk_form) and as a readable statement of the algebra the GPU kernel
implements.  The pages name a chunkwise algorithm built on a
Diagonal-Plus-Low-Rank transition (akshathtiwari.co.in "Kimi Delta Attention"
explainer) and say the chunkwise form regroups the recurrence into matrix
products (daily.dev summary of "You Could Have Come Up with Kimi Delta
Attention"); the pseudocode itself is not on the pages, so this is derived
from the recurrence:

Within a chunk of c tokens starting from state S (d_k x d_v), let
Gamma_r = sum_{j<=r} log_alpha_j (per key channel, inclusive).  Then the state
after token r is
    S_r = Diag(e^{Gamma_r}) S + sum_{i<=r} Diag(e^{Gamma_r - Gamma_i}) k_i u_i^T
and the per-token corrections u_r satisfy
    u_r + beta_r sum_{i<r} [sum_c k_rc k_ic e^{Gamma_rc - Gamma_ic}] u_i
        = beta_r (v_r - S^T (k_r * e^{Gamma_r})),
i.e.  (I + A) U = Diag(beta) (V - K_up S)  with  A strictly lower triangular,
A_ri = beta_r (K_up K_dn^T)_ri,  K_up = K * e^{Gamma},  K_dn = K * e^{-Gamma}.
Outputs and the carried state:
    O      = Q_up S + tril_incl(Q_up K_dn^T) U,       Q_up = Q * e^{Gamma}
    S_next = Diag(e^{Gamma_c}) S + K_right^T U,        K_right = K * e^{Gamma_c - Gamma}
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_step(S, q, k, v, g, beta):
    """One chunk. q, k, g: (c, dk); v: (c, dv); beta: (c,). Returns (O, S_next)."""
    c = q.shape[0]
    G = np.cumsum(g, axis=0)
    K_up, Q_up = k * np.exp(G), q * np.exp(G)
    K_dn = k * np.exp(-G)
    K_right = k * np.exp(G[-1] - G)
    A = np.tril(beta[:, None] * (K_up @ K_dn.T), -1)
    rhs = beta[:, None] * (v - K_up @ S)
    U = solve_triangular(np.eye(c) + A, rhs, lower=True, unit_diagonal=True)
    O = Q_up @ S + np.tril(Q_up @ K_dn.T) @ U
    S_next = np.exp(G[-1])[:, None] * S + K_right.T @ U
    return O, S_next


def chunked_forward(q, k, v, g, beta, S0, C):
    """Dense (B, T, H, .) inputs, chunk size C; returns (o, S_T)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for t0 in range(0, T, C):
                t1 = min(T, t0 + C)
                O, S = chunk_step(S, q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                                  g[b, t0:t1, h], beta[b, t0:t1, h])
                o[b, t0:t1, h] = O
            S_T[b, h] = S
    return o, S_T

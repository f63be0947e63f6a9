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


def chunk_step_bwd(S, q, k, v, g, beta, dO, D):
    """Gradients through one chunk (the reverse of ``chunk_step``).

    S: the state entering the chunk; D: the loss gradient with respect to the
    state leaving it.  Returns (dq, dk, dv, dg, dbeta, dS) with dS the gradient
    with respect to S.  The within-chunk decay factors are taken pairwise,
    F_ric = e^{Gamma_rc - Gamma_ic} for i <= r (never above 1), which is how
    the GPU backward forms them:
      M0 = [sum_c k_rc k_ic F_ric] (strictly lower), A = Diag(beta) M0,
      P  = [sum_c q_rc k_ic F_ric] (lower, diagonal included),
      T  = (I + A)^{-1},  T' = T Diag(beta),  X = V - K_up S,  U = T' X,
      O  = Q_up S + P U,  S_next = Diag(gamma) S + K_right^T U.
    Reverse, in the order the kernels take it:
      dU = P^T dO + K_right D;   dX = T'^T dU;   dV = dX
      dT' = dU X^T;  dP = tril_incl(dO U^T);  dbeta_i = sum_r T_ri dT'_ri
      dA = strict_lower(-T^T (dT' Diag(beta)) T^T);  dbeta_r += sum_i dA_ri M0_ri
      dM = Diag(beta) dA; then through the pairwise sums for M0 and P
      dS = Diag(gamma) D + Q_up^T dO - K_up^T dX
      dK_up = -dX S^T, dQ_up = dO S^T, dK_right = U D^T, dgamma = rowsum(D * S)
    and the chain rule from K_up, Q_up, K_right, gamma to k, q and Gamma, then
    dg_j = sum_{r >= j} dGamma_r + dGamma_c (Gamma_c enters gamma and K_right).
    """
    c, dk = q.shape
    G = np.cumsum(g, axis=0)
    Gc = G[-1]
    F = np.exp(G[:, None, :] - G[None, :, :])          # (r, i, c)
    F = F * np.tril(np.ones((c, c)))[:, :, None]       # i <= r only
    M0 = np.tril(np.einsum("rc,ic,ric->ri", k, k, F), -1)
    P = np.einsum("rc,ic,ric->ri", q, k, F)
    A = beta[:, None] * M0
    T = np.linalg.inv(np.eye(c) + A)
    Tp = T * beta[None, :]
    E = np.exp(G)
    K_up, Q_up = k * E, q * E
    K_right = k * np.exp(Gc - G)
    gam = np.exp(Gc)
    X = v - K_up @ S
    U = Tp @ X
    dU = P.T @ dO + K_right @ D
    dX = Tp.T @ dU
    dTp = dU @ X.T
    dP = np.tril(dO @ U.T)
    dbeta = np.sum(T * dTp, axis=0)
    dT = dTp * beta[None, :]
    dA = np.tril(-T.T @ dT @ T.T, -1)
    dbeta = dbeta + np.sum(dA * M0, axis=1)
    dM = beta[:, None] * dA
    dS = gam[:, None] * D + Q_up.T @ dO - K_up.T @ dX
    dK_up = -dX @ S.T
    dQ_up = dO @ S.T
    dK_right = U @ D.T
    dgam = np.sum(D * S, axis=1)
    # pairwise sums: M0 (weights dM) and P (weights dP)
    dq = np.einsum("ri,ic,ric->rc", dP, k, F) + dQ_up * E
    dk_ = (np.einsum("ri,ic,ric->rc", dM, k, F) + np.einsum("ri,rc,ric->ic", dM, k, F)
           + np.einsum("ri,rc,ric->ic", dP, q, F) + dK_up * E + dK_right * np.exp(Gc - G))
    W = (np.einsum("ri,rc,ic,ric->ric", dM, k, k, F) + np.einsum("ri,rc,ic,ric->ric", dP, q, k, F))
    dG = W.sum(axis=1) - W.sum(axis=0)
    dG = dG + dK_up * K_up + dQ_up * Q_up - dK_right * K_right
    dGc = np.sum(dK_right * K_right, axis=0) + dgam * gam
    dg = np.cumsum(dG[::-1], axis=0)[::-1] + dGc[None, :]
    return dq, dk_, dX, dg, dbeta, dS


def chunked_backward(q, k, v, g, beta, S0, dO, dS_T, C):
    """Dense (B, T, H, .) inputs, chunk size C: the states entering each chunk
    from a forward sweep, then the chunks in reverse.  Returns
    (dq, dk, dv, dg, dbeta, dS0)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = [np.zeros((B, T, H, dk)), np.zeros((B, T, H, dk)), np.zeros((B, T, H, dv)),
           np.zeros((B, T, H, dk)), np.zeros((B, T, H))]
    dS0 = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            starts = list(range(0, T, C))
            states = []
            for t0 in starts:
                t1 = min(T, t0 + C)
                states.append(S)
                _, S = chunk_step(S, q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                                  g[b, t0:t1, h], beta[b, t0:t1, h])
            D = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T[b, h], dtype=np.float64)
            for n in range(len(starts) - 1, -1, -1):
                t0 = starts[n]
                t1 = min(T, t0 + C)
                r = chunk_step_bwd(states[n], q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                                   g[b, t0:t1, h], beta[b, t0:t1, h], dO[b, t0:t1, h], D)
                for j in range(4):
                    out[j][b, t0:t1, h] = r[j]
                out[4][b, t0:t1, h] = r[4]
                D = r[5]
            dS0[b, h] = D
    return tuple(out) + (dS0,)

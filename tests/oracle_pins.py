"""Pins for the fp64 oracle: checks fixed by the pages and by mathematics.

Each ``pin_*`` function takes an oracle backend (an object with ``fwd`` and
``decode`` callables shaped like ``oracle.fwd`` / ``oracle.decode``) and raises
AssertionError when the backend disagrees with the pin.  test_oracle_pins.py
runs them against the real oracle; test_oracle_mutants.py runs them against
copies of the C loop with planted mistakes, each of which must fail at least
one pin.

None of these checks re-types the oracle's loop: each compares it with a value
printed on the pages, a closed form, a published recurrence in another
convention, an explicit matrix product, or a property that any correct
implementation must have.
"""
from __future__ import annotations

import os
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [float(x) for x in vals]
    return out


def rel_err(x, ref) -> float:
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (scale if scale > 0 else 1.0))


def _rng(seed):
    return np.random.default_rng(seed)


def _orthonormal(rng, n, m):
    """m orthonormal vectors of length n (rows)."""
    qm, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return qm[:, :m].T.copy()


def _rand_inputs(rng, B, T, H, dk, dv, s0=True, unit_k=False, beta_range=(0.0, 1.0)):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.exponential(0.3, size=(B, T, H, dk))
    beta = rng.uniform(*beta_range, size=(B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


# --------------------------------------------------------------------------
# Values the pages print
# --------------------------------------------------------------------------

def pin_decay_example(be):
    """Per-channel decay worked example: (0.9, 0.2) on a stored (10, 10) gives (9, 2).

    Teacher guide, chapter 12, section 12.1 "Per-channel decay" (fixture
    tests/golden/per_channel_decay.txt).  beta = 0 isolates the decay.
    """
    gd = read_golden("per_channel_decay.txt")
    a, stored, expected = gd["decay"], gd["stored"], gd["expected"]
    dk, dv = 2, 1
    S0 = np.array(stored, dtype=np.float64).reshape(1, 1, dk, dv)
    g = np.log(np.array(a)).reshape(1, 1, 1, dk)
    q = np.array([1.0, 1.0]).reshape(1, 1, 1, dk)
    k = np.array([0.3, -0.7]).reshape(1, 1, 1, dk)
    v = np.array([5.0]).reshape(1, 1, 1, dv)
    beta = np.zeros((1, 1, 1))
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    assert rel_err(S_T[0, 0, :, 0], expected) < 1e-14, S_T
    assert abs(o[0, 0, 0, 0] - sum(expected)) < 1e-12, o


def pin_half_life(be):
    """Channel half-lives ln(0.5)/ln(a): about 6.6 tokens vs 0.43 tokens, ratio about 15.

    Teacher guide, Misconceptions table, row 2 (fixture tests/golden/half_life.txt).
    The half-life is measured from the oracle's own outputs over 20 decay-only
    steps, one head reading each channel.
    """
    gd = read_golden("half_life.txt")
    a = np.array(gd["decay"])
    hl_ref, ratio_ref = gd["half_life"], gd["ratio"][0]
    tol_hl0, tol_hl1, tol_ratio = gd["tolerance"]
    T, H, dk, dv = 20, 2, 2, 1
    g = np.broadcast_to(np.log(a), (1, T, H, dk)).copy()
    q = np.zeros((1, T, H, dk))
    q[:, :, 0, 0] = 1.0   # head 0 reads channel 0
    q[:, :, 1, 1] = 1.0   # head 1 reads channel 1
    k = np.zeros((1, T, H, dk))
    v = np.zeros((1, T, H, dv))
    beta = np.zeros((1, T, H))
    S0 = np.ones((1, H, dk, dv))
    o, _ = be.fwd(q, k, v, g, beta, S0)
    hl = []
    for h in range(H):
        trace = o[0, :, h, 0]
        per_step = trace[5] / trace[4]
        hl.append(np.log(0.5) / np.log(per_step))
    assert abs(hl[0] - hl_ref[0]) < tol_hl0, hl
    assert abs(hl[1] - hl_ref[1]) < tol_hl1, hl
    assert abs(hl[0] / hl[1] - ratio_ref) < tol_ratio, hl
    # discrete reading: channel 0 is still above half after 6 tokens, below after 7
    tr0 = o[0, :, 0, 0]
    assert tr0[5] > 0.5 > tr0[6], tr0[:8]
    assert o[0, 0, 1, 0] < 0.5


def pin_overwrite_trace(be):
    """beta = 1 correction gives exactly (4, 4), then two 0.2-gate steps give 0.16.

    Teacher guide, Misconceptions table, row 3 (fixture tests/golden/overwrite_trace.txt).
    """
    gd = read_golden("overwrite_trace.txt")
    value, gate, steps = gd["value"], gd["gate"][0], int(gd["steps"][0])
    T, dk, dv = 1 + steps, 2, 2
    S0 = np.array([[1.5, -2.0], [3.0, 0.25]]).reshape(1, 1, dk, dv)
    k = np.zeros((1, T, 1, dk))
    k[0, 0, 0, 1] = 1.0
    v = np.zeros((1, T, 1, dv))
    v[0, 0, 0, :] = value
    beta = np.zeros((1, T, 1))
    beta[0, 0, 0] = gd["beta"][0]
    g = np.zeros((1, T, 1, dk))
    g[0, 1:, 0, 1] = np.log(gate)
    q = np.zeros((1, T, 1, dk))
    q[0, :, 0, 1] = 1.0
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    assert rel_err(o[0, 0, 0], gd["after_write"]) < 1e-15, o[0, 0, 0]
    assert rel_err(o[0, steps, 0], gd["after_decay"]) < 1e-14, o[0, steps, 0]
    assert rel_err(S_T[0, 0, 1], gd["after_decay"]) < 1e-14, S_T
    assert np.array_equal(S_T[0, 0, 0], S0[0, 0, 0]), S_T   # channel 1 untouched


# --------------------------------------------------------------------------
# Special cases that reduce to other published recurrences
# --------------------------------------------------------------------------

def pin_new_key_is_linear_attention(be):
    """A key orthogonal to every earlier key is written like plain linear attention.

    akshathtiwari.co.in "Kimi Delta Attention" explainer, delta-rule paragraph:
    with nothing stored for a new key the error is the value itself.  With
    alpha = 1, S0 = 0 and mutually orthogonal keys (any norms) the result must
    be the linear-attention sum  S_T = sum_t beta_t k_t v_t^T,
    o_t = sum_{i<=t} beta_i v_i (k_i . q_t).
    """
    rng = _rng(11)
    dk, dv, H = 8, 5, 2
    T = dk
    k = np.zeros((1, T, H, dk))
    for h in range(H):
        basis = _orthonormal(rng, dk, T)
        k[0, :, h, :] = basis * rng.uniform(0.5, 2.0, size=(T, 1))
    q = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    beta = rng.uniform(0.1, 1.5, size=(1, T, H))
    g = np.zeros((1, T, H, dk))
    o, S_T = be.fwd(q, k, v, g, beta, None)
    for h in range(H):
        S_ref = sum(beta[0, t, h] * np.outer(k[0, t, h], v[0, t, h]) for t in range(T))
        assert rel_err(S_T[0, h], S_ref) < 1e-12
        for t in range(T):
            o_ref = sum(beta[0, i, h] * v[0, i, h] * (k[0, i, h] @ q[0, t, h]) for i in range(t + 1))
            assert rel_err(o[0, t, h], o_ref) < 1e-12


def pin_one_hot_keys_gated_linear_attention(be):
    """Distinct one-hot keys turn KDA into gated linear attention with per-channel decay.

    A one-hot key on a never-written channel reads zero, so each write is
    beta_t k_t v_t^T, and that row then only decays:
    row c_t of S_T = (prod_{j>t} alpha_{j, c_t}) beta_t v_t.
    Pins the per-key-channel gate acting on rows and the write/decay order.
    """
    rng = _rng(12)
    dk, dv, H = 9, 4, 2
    T = 7
    ch = np.stack([rng.permutation(dk)[:T] for _ in range(H)], axis=1)  # (T, H)
    k = np.zeros((1, T, H, dk))
    for t in range(T):
        for h in range(H):
            k[0, t, h, ch[t, h]] = 1.0
    q = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    beta = rng.uniform(0.1, 1.0, size=(1, T, H))
    g = -rng.exponential(0.5, size=(1, T, H, dk))
    o, S_T = be.fwd(q, k, v, g, beta, None)
    for h in range(H):
        S_ref = np.zeros((dk, dv))
        for t in range(T):
            c = ch[t, h]
            S_ref[c] = np.exp(g[0, t + 1:, h, c].sum()) * beta[0, t, h] * v[0, t, h]
        assert rel_err(S_T[0, h], S_ref) < 1e-13
        # output at the last token reads the same closed form
        assert rel_err(o[0, T - 1, h], S_ref.T @ q[0, T - 1, h]) < 1e-13


def pin_widget_overwrite(be):
    """Three stored associations, then one key overwritten.

    akshathtiwari.co.in explainer, closing description of the first widget:
    additive memory returns the corrupted sum for the rewritten key while the
    delta rule returns the clean new value and leaves the other keys intact.
    Orthonormal keys, beta = 1, alpha = 1; head i reads key i at every token.
    """
    rng = _rng(13)
    dk, dv = 6, 3
    keys = _orthonormal(rng, dk, 3)
    vals = rng.standard_normal((3, dv))
    v2_new = rng.standard_normal(dv)
    seq_k = [keys[0], keys[1], keys[2], keys[1]]
    seq_v = [vals[0], vals[1], vals[2], v2_new]
    T, H = 4, 3
    k = np.zeros((1, T, H, dk))
    v = np.zeros((1, T, H, dv))
    q = np.zeros((1, T, H, dk))
    for t in range(T):
        k[0, t, :, :] = seq_k[t]
        v[0, t, :, :] = seq_v[t]
        for h in range(H):
            q[0, t, h] = keys[h]
    beta = np.ones((1, T, H))
    g = np.zeros((1, T, H, dk))
    o, _ = be.fwd(q, k, v, g, beta, None)
    recalled = o[0, T - 1]                      # (H, dv): head i recalls key i
    assert rel_err(recalled[0], vals[0]) < 1e-13
    assert rel_err(recalled[1], v2_new) < 1e-13
    assert rel_err(recalled[2], vals[2]) < 1e-13
    additive = sum(np.outer(seq_k[t], seq_v[t]) for t in range(T))
    add_recall = additive.T @ keys[1]
    assert rel_err(add_recall, vals[1] + v2_new) < 1e-13
    assert rel_err(recalled[1], add_recall) > 0.1


def _gated_deltanet_transposed(q, k, v, a, beta, S0):
    """Gated DeltaNet as published (Yang, Kautz & Hatamizadeh), value-by-key state.

    S_t = S_{t-1} (a_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T,  o_t = S_t q_t,
    with S of shape d_v x d_k and one scalar gate a_t per token.
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = S0.T.copy() if S0 is not None else np.zeros((dv, dk))
    o = np.zeros((T, dv))
    for t in range(T):
        P = a[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t]))
        S = S @ P + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S.T


def pin_scalar_gate_is_gated_deltanet(be):
    """alpha equal across channels reduces KDA to Gated DeltaNet.

    "The fourth layer remembers", section "What each kind of layer keeps": the
    earlier design uses one decay number per head per token; KDA generalises it
    to one per key channel.  Compared with Gated DeltaNet written in its own
    (value-by-key, right-multiplied) convention.
    """
    rng = _rng(14)
    B, T, H, dk, dv = 1, 12, 2, 6, 5
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0.0, 1.5))
    a_scalar = rng.uniform(0.3, 1.0, size=(B, T, H))
    g = np.repeat(np.log(a_scalar)[..., None], dk, axis=-1)
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    for h in range(H):
        o_ref, S_ref = _gated_deltanet_transposed(q[0, :, h], k[0, :, h], v[0, :, h],
                                                  a_scalar[0, :, h], beta[0, :, h], S0[0, h])
        assert rel_err(o[0, :, h], o_ref) < 1e-12
        assert rel_err(S_T[0, h], S_ref) < 1e-12


def pin_alpha_one_is_deltanet(be):
    """alpha = 1 reduces KDA to DeltaNet; with beta = 1 a rewritten key recalls its latest value.

    akshathtiwari.co.in explainer, delta-rule paragraph (DeltaNet read-error-write);
    weaving.news "Attention? More like notation warfare", Key Points, last bullet.
    DeltaNet written in its value-by-key convention: S_t = S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
    """
    rng = _rng(15)
    B, T, H, dk, dv = 1, 10, 2, 5, 7
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0.0, 2.0))
    g = np.zeros((B, T, H, dk))
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    for h in range(H):
        S = S0[0, h].T.copy()
        for t in range(T):
            kt = k[0, t, h]
            S = S @ (np.eye(dk) - beta[0, t, h] * np.outer(kt, kt)) + beta[0, t, h] * np.outer(v[0, t, h], kt)
            assert rel_err(o[0, t, h], S @ q[0, t, h]) < 1e-12
        assert rel_err(S_T[0, h], S.T) < 1e-12
    # exact recall of the latest value written under a repeated key
    dk, dv = 4, 3
    keys = _orthonormal(rng, dk, 2)
    vals = rng.standard_normal((4, dv))
    seq = [(0, vals[0]), (1, vals[1]), (0, vals[2]), (0, vals[3])]
    T = len(seq)
    k = np.zeros((1, T, 1, dk))
    v = np.zeros((1, T, 1, dv))
    for t, (ki, vi) in enumerate(seq):
        k[0, t, 0] = keys[ki]
        v[0, t, 0] = vi
    q = np.broadcast_to(keys[0], (1, T, 1, dk)).copy()
    o, _ = be.fwd(q, k, v, np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), None)
    assert rel_err(o[0, T - 1, 0], vals[3]) < 1e-13
    assert rel_err(o[0, 1, 0], vals[0]) < 1e-13


# --------------------------------------------------------------------------
# Brute force and properties
# --------------------------------------------------------------------------

def pin_brute_force(be):
    """Explicit product of d_k x d_k transition matrices, T <= 8, random shapes."""
    from oracle import brute_force
    rng = _rng(16)
    for trial in range(12):
        B = int(rng.integers(1, 3))
        T = int(rng.integers(1, 9))
        H = int(rng.integers(1, 4))
        dk = int(rng.integers(1, 8))
        dv = int(rng.integers(1, 8))
        q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, s0=bool(trial % 2),
                                            beta_range=(-0.5, 2.0))
        o, S_T = be.fwd(q, k, v, g, beta, S0)
        o_b, S_b = brute_force(q, k, v, g, beta, S0)
        assert rel_err(o, o_b) < 1e-13, (trial, rel_err(o, o_b))
        assert rel_err(S_T, S_b) < 1e-13, (trial, rel_err(S_T, S_b))


def pin_beta_zero_closed_form(be):
    """beta = 0: only the gate acts, S_t = Diag(exp(sum_{j<=t} log_alpha_j)) S0."""
    rng = _rng(17)
    B, T, H, dk, dv = 2, 9, 2, 5, 3
    q, k, v, g, _, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    beta = np.zeros((B, T, H))
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    for b in range(B):
        for h in range(H):
            G = np.cumsum(g[b, :, h], axis=0)
            assert rel_err(S_T[b, h], np.exp(G[-1])[:, None] * S0[b, h]) < 1e-13
            for t in range(T):
                assert rel_err(o[b, t, h], (np.exp(G[t])[:, None] * S0[b, h]).T @ q[b, t, h]) < 1e-13


def pin_affine_in_s0(be):
    """o and S_T are affine in S0 (the recurrence is linear in the state)."""
    rng = _rng(18)
    B, T, H, dk, dv = 1, 11, 2, 4, 6
    q, k, v, g, beta, Sa = _rand_inputs(rng, B, T, H, dk, dv)
    Sb = rng.standard_normal(Sa.shape)
    o0, S0_ = be.fwd(q, k, v, g, beta, None)
    oa, Sa_ = be.fwd(q, k, v, g, beta, Sa)
    ob, Sb_ = be.fwd(q, k, v, g, beta, Sb)
    oab, Sab_ = be.fwd(q, k, v, g, beta, 2.0 * Sa - 0.5 * Sb)
    assert rel_err(oab - o0, 2.0 * (oa - o0) - 0.5 * (ob - o0)) < 1e-12
    assert rel_err(Sab_ - S0_, 2.0 * (Sa_ - S0_) - 0.5 * (Sb_ - S0_)) < 1e-12


def pin_split_continuation(be):
    """Running [0, t1) then [t1, T) from the carried state equals one call."""
    rng = _rng(19)
    B, T, H, dk, dv = 2, 17, 2, 5, 4
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    for t1 in (0, 1, 8, 16, 17):
        sl1, sl2 = slice(0, t1), slice(t1, T)
        o1, S1 = be.fwd(q[:, sl1], k[:, sl1], v[:, sl1], g[:, sl1], beta[:, sl1], S0)
        o2, S2 = be.fwd(q[:, sl2], k[:, sl2], v[:, sl2], g[:, sl2], beta[:, sl2], S1)
        assert rel_err(np.concatenate([o1, o2], axis=1), o) < 1e-13
        assert rel_err(S2, S_T) < 1e-13


def pin_varlen_matches_separate(be):
    """Packed sequences (cu_seqlens) equal separate runs; states reset per sequence."""
    rng = _rng(20)
    lens = [5, 0, 9, 1, 13]
    H, dk, dv = 2, 4, 3
    T = sum(lens)
    q, k, v, g, beta, _ = _rand_inputs(rng, 1, T, H, dk, dv, s0=False)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S_T = be.fwd(q, k, v, g, beta, S0, cu_seqlens=cu)
    for s, L in enumerate(lens):
        sl = slice(cu[s], cu[s + 1])
        o_s, S_s = be.fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], S0[s:s + 1])
        assert rel_err(o[:, sl], o_s) < 1e-13 if L else True
        assert rel_err(S_T[s], S_s[0]) < 1e-13
    assert np.array_equal(S_T[1], S0[1])   # empty sequence: S_T = S0


def pin_decode_matches_forward(be):
    """Applying the one-token decode step T times equals the forward pass."""
    rng = _rng(21)
    N, T, H, dk, dv = 3, 6, 2, 5, 4
    q, k, v, g, beta, S0 = _rand_inputs(rng, N, T, H, dk, dv)
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    S = S0.copy()
    for t in range(T):
        o_t, S = be.decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        assert rel_err(o_t, o[:, t]) < 1e-13
    assert rel_err(S, S_T) < 1e-13


def pin_norm_bound(be):
    """Unit keys and beta in [0, 2] make I - beta k k^T a contraction, so
    ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||  at every token."""
    rng = _rng(22)
    B, T, H, dk, dv = 1, 40, 1, 6, 5
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, unit_k=True, beta_range=(0.0, 2.0))
    prev = np.linalg.norm(S0[0, 0])
    S = S0
    for t in range(T):
        _, S = be.fwd(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                      beta[:, t:t + 1], S)
        cur = np.linalg.norm(S[0, 0])
        assert cur <= prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12
        prev = cur


def pin_chunk_form(be):
    """The chunkwise (WY) form of the recurrence, derived independently, agrees.

    The chunked algebra (tests/chunk_form.py) regroups the same recurrence into
    per-chunk matrix products; at several chunk sizes, with ragged last chunks,
    it must match the token loop to rounding.
    """
    from chunk_form import chunked_forward
    rng = _rng(23)
    B, T, H, dk, dv = 2, 150, 2, 16, 12
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, unit_k=True)
    o, S_T = be.fwd(q, k, v, g, beta, S0)
    for C in (1, 7, 64):
        o_c, S_c = chunked_forward(q, k, v, g, beta, S0, C)
        assert rel_err(o_c, o) < 1e-11, (C, rel_err(o_c, o))
        assert rel_err(S_c, S_T) < 1e-11, (C, rel_err(S_c, S_T))


ALL_PINS = [
    pin_decay_example,
    pin_half_life,
    pin_overwrite_trace,
    pin_new_key_is_linear_attention,
    pin_one_hot_keys_gated_linear_attention,
    pin_widget_overwrite,
    pin_scalar_gate_is_gated_deltanet,
    pin_alpha_one_is_deltanet,
    pin_brute_force,
    pin_beta_zero_closed_form,
    pin_affine_in_s0,
    pin_split_continuation,
    pin_varlen_matches_separate,
    pin_decode_matches_forward,
    pin_norm_bound,
    pin_chunk_form,
]


def backend(lib=None):
    """The oracle (or a mutant library built from its source) as a pin backend."""
    import oracle

    def fwd(q, k, v, g, beta, S0=None, cu_seqlens=None):
        return oracle.fwd(q, k, v, g, beta, S0, cu_seqlens, nthreads=2, lib=lib)

    def decode(q, k, v, g, beta, S):
        return oracle.decode(q, k, v, g, beta, S, nthreads=2, lib=lib)

    return SimpleNamespace(fwd=fwd, decode=decode)

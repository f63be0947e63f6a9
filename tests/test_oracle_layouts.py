"""Pins for the oracle's gate layouts, state pools and input preparation (CPU only).

oracle.channel_gate, oracle.fwd_pooled and oracle.decode_pooled only
rearrange inputs and outputs around the token loop.  Each is compared here
with something written independently of that loop: the published scalar-gated
and ungated delta rules in their own (value-by-key) convention, and the
explicit transition-matrix products of oracle.brute_force, per sequence, with
the pool rows gathered and scattered by hand.
"""
import numpy as np
import pytest

import oracle
from oracle_pins import _gated_deltanet_transposed, _rand_inputs, _rng, rel_err


def _deltanet_transposed(q, k, v, beta, S0):
    """DeltaNet, value-by-key state: S_t = S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t."""
    T, dk = k.shape
    S = S0.T.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = S @ (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S.T


def test_head_gate_is_gated_deltanet():
    """One decay per (token, head) is Gated DeltaNet ("The fourth layer remembers", forget-gate paragraph)."""
    rng = _rng(31)
    B, T, H, dk, dv = 2, 11, 3, 6, 5
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0.0, 1.5))
    a = rng.uniform(0.2, 1.0, size=(B, T, H))
    o, S_T = oracle.fwd(q, k, v, np.log(a), beta, S0, gate="head", nthreads=2)
    for b in range(B):
        for h in range(H):
            o_ref, S_ref = _gated_deltanet_transposed(q[b, :, h], k[b, :, h], v[b, :, h],
                                                      a[b, :, h], beta[b, :, h], S0[b, h])
            assert rel_err(o[b, :, h], o_ref) < 1e-12
            assert rel_err(S_T[b, h], S_ref) < 1e-12


def test_no_gate_is_deltanet():
    """alpha = 1 is DeltaNet (akshathtiwari.co.in explainer, delta-rule paragraph)."""
    rng = _rng(32)
    B, T, H, dk, dv = 1, 9, 2, 5, 4
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0.0, 2.0))
    o, S_T = oracle.fwd(q, k, v, None, beta, S0, gate="none", nthreads=2)
    for h in range(H):
        o_ref, S_ref = _deltanet_transposed(q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], S0[0, h])
        assert rel_err(o[0, :, h], o_ref) < 1e-12
        assert rel_err(S_T[0, h], S_ref) < 1e-12


@pytest.mark.parametrize("gate", ["head", "none"])
def test_decode_gate_layouts(gate):
    """One decode step per layout equals the first step of the published loops."""
    rng = _rng(33)
    N, H, dk, dv = 3, 2, 4, 6
    q, k, v, _, beta, S0 = _rand_inputs(rng, N, 1, H, dk, dv, beta_range=(0.0, 1.0))
    a = rng.uniform(0.2, 1.0, size=(N, H))
    g = np.log(a) if gate == "head" else None
    o, S_new = oracle.decode(q[:, 0], k[:, 0], v[:, 0], g, beta[:, 0], S0, nthreads=2, gate=gate)
    for n in range(N):
        for h in range(H):
            if gate == "head":
                o_ref, S_ref = _gated_deltanet_transposed(q[n, :, h], k[n, :, h], v[n, :, h],
                                                          a[n:n + 1, h], beta[n, :, h], S0[n, h])
            else:
                o_ref, S_ref = _deltanet_transposed(q[n, :, h], k[n, :, h], v[n, :, h],
                                                    beta[n, :, h], S0[n, h])
            assert rel_err(o[n, h], o_ref[0]) < 1e-12
            assert rel_err(S_new[n, h], S_ref) < 1e-12


def test_gate_layout_shapes_are_checked():
    with pytest.raises(AssertionError):
        oracle.channel_gate(np.zeros((1, 2, 3, 4)), "head", (1, 2, 3, 4))
    with pytest.raises(ValueError):
        oracle.channel_gate(None, "per-token", (1, 2, 3, 4))


def _brute_rows(q, k, v, g, beta, cu, S0_rows):
    """brute_force per packed sequence (T <= 8 each), states given per sequence."""
    N = len(cu) - 1
    o = np.zeros(q.shape[:3] + (v.shape[-1],))
    S_T = []
    for s in range(N):
        ts = slice(cu[s], cu[s + 1])
        if cu[s + 1] == cu[s]:
            S_T.append(S0_rows[s].copy())
            continue
        os_, Ss = oracle.brute_force(q[:, ts], k[:, ts], v[:, ts], g[:, ts], beta[:, ts],
                                     S0_rows[s][None])
        o[:, ts] = os_
        S_T.append(Ss[0])
    return o, np.stack(S_T)


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
def test_fwd_pooled_against_brute_force(gate):
    """Slot map with a permutation, a padding slot (-1) and an index past the pool."""
    rng = _rng(34)
    H, dk, dv, P = 2, 4, 3, 6
    lens = [3, 0, 5, 2, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, g, beta, _ = _rand_inputs(rng, 1, T, H, dk, dv)
    if gate == "head":
        g_in = g[..., 0]
        g_full = np.repeat(g_in[..., None], dk, axis=-1)
    elif gate == "none":
        g_in, g_full = None, np.zeros_like(g)
    else:
        g_in = g_full = g
    pool = rng.standard_normal((P, H, dk, dv))
    idx = np.array([4, 1, -1, 0, 9])           # sequence 2: padding, 4: past the pool
    o, new_pool = oracle.fwd_pooled(q, k, v, g_in, beta, pool, idx, cu, gate=gate,
                                    S_T_pool=pool, nthreads=2)
    S0_rows = [pool[i] if 0 <= i < P else np.zeros((H, dk, dv)) for i in idx]
    o_ref, S_ref = _brute_rows(q, k, v, g_full, beta, cu, S0_rows)
    assert rel_err(o, o_ref) < 1e-12
    want = pool.copy()
    for s, i in enumerate(idx):
        if 0 <= i < P:
            want[i] = S_ref[s]
    assert rel_err(new_pool, want) < 1e-12
    # rows 2, 3, 5 are nobody's slot and stay bit-identical
    for r in (2, 3, 5):
        assert np.array_equal(new_pool[r], pool[r])
    # without an output pool only o is produced
    o2, none = oracle.fwd_pooled(q, k, v, g_in, beta, pool, idx, cu, gate=gate, nthreads=2)
    assert none is None and np.array_equal(o2, o)


def test_decode_pooled_against_brute_force():
    rng = _rng(35)
    N, H, dk, dv, P = 4, 2, 5, 3, 5
    q, k, v, g, beta, _ = _rand_inputs(rng, N, 1, H, dk, dv)
    pool = rng.standard_normal((P, H, dk, dv))
    idx = np.array([3, -2, 0, 5])
    o, new_pool = oracle.decode_pooled(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], pool, idx,
                                       nthreads=2)
    want = pool.copy()
    for n, i in enumerate(idx):
        S0 = pool[i] if 0 <= i < P else np.zeros((H, dk, dv))
        o_ref, S_ref = oracle.brute_force(q[n:n + 1], k[n:n + 1], v[n:n + 1], g[n:n + 1],
                                          beta[n:n + 1], S0[None])
        assert rel_err(o[n], o_ref[0, 0]) < 1e-12
        if 0 <= i < P:
            want[i] = S_ref[0]
    assert rel_err(new_pool, want) < 1e-12
    assert np.array_equal(new_pool[1], pool[1]) and np.array_equal(new_pool[2], pool[2])


# --------------------------------------------------------------------------
# Input preparation: L2-normalised q and k, softplus gate
# --------------------------------------------------------------------------

def test_prepare_l2norm_closed_forms():
    rng = _rng(40)
    q = rng.standard_normal((2, 5, 3, 7)) * rng.uniform(0.1, 50, size=(2, 5, 3, 1))
    k = rng.standard_normal((2, 5, 3, 7))
    k[0, 1, 2] = 0.0                                     # a zero key stays zero
    qn, kn, g = oracle.prepare(q, k, None, oracle.FLAG_L2NORM_QK)
    assert g is None
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1.0, atol=1e-14)
    nz = np.linalg.norm(k, axis=-1) > 0
    assert np.allclose(np.linalg.norm(kn, axis=-1)[nz], 1.0, atol=1e-14)
    assert np.array_equal(kn[0, 1, 2], np.zeros(7))
    # same direction: the normalised vector is a positive multiple of the input
    ratio = qn / q
    assert np.allclose(ratio, ratio[..., :1], rtol=1e-13) and (ratio > 0).all()
    # without the flag nothing changes
    q2, k2, _ = oracle.prepare(q, k, None, 0)
    assert np.array_equal(q2, q) and np.array_equal(k2, k)


def test_prepare_softplus_closed_forms():
    x = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 700.0, -700.0, 1e4])
    _, _, g = oracle.prepare(np.zeros((1, 1)), np.zeros((1, 1)), x, oracle.FLAG_GATE_SOFTPLUS)
    a = np.exp(g)
    assert np.isfinite(g).all()
    assert abs(a[0] - 0.5) < 1e-15                       # softplus(0) = ln 2
    # alpha = sigmoid(-x) = 1 / (1 + e^x), written out independently
    ref = np.array([1.0 / (1.0 + np.exp(v)) if v < 700 else 0.0 for v in x[:5]])
    assert np.allclose(a[:5], ref, rtol=1e-14, atol=1e-300)
    assert abs(g[3] + 30.0 + np.log1p(np.exp(-30.0))) < 1e-12
    assert abs(g[4] + np.log1p(np.exp(-30.0))) < 1e-24
    assert g[5] == -700.0 and g[7] == -1e4               # large x: log_alpha -> -x
    assert (g <= 0).all()


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_prepared_forward_against_brute_force(flags):
    """The forward with preparation flags equals the brute force on inputs
    prepared by hand (numpy's norm routine, the logistic function)."""
    rng = _rng(41 + flags)
    B, T, H, dk, dv = 2, 6, 2, 5, 4
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    q = q * 3.0
    x = rng.standard_normal((B, T, H, dk)) * 2.0
    gate_in = x if flags & 2 else g
    o, S_T = oracle.fwd(q, k, v, gate_in, beta, S0, nthreads=2, flags=flags)
    qq, kk = q, k
    if flags & 1:
        qq = q / np.linalg.norm(q, axis=-1, keepdims=True)
        kk = k / np.linalg.norm(k, axis=-1, keepdims=True)
    gg = np.log(1.0 / (1.0 + np.exp(x))) if flags & 2 else g
    o_ref, S_ref = oracle.brute_force(qq, kk, v, gg, beta, S0)
    assert rel_err(o, o_ref) < 1e-12 and rel_err(S_T, S_ref) < 1e-12
    # and the decode step agrees with the forward's first token
    od, Sd = oracle.decode(q[:, 0], k[:, 0], v[:, 0], gate_in[:, 0], beta[:, 0], S0, nthreads=2,
                           flags=flags)
    o1, S1 = oracle.brute_force(qq[:, :1], kk[:, :1], v[:, :1], gg[:, :1], beta[:, :1], S0)
    assert rel_err(od, o1[:, 0]) < 1e-12 and rel_err(Sd, S1) < 1e-12


def test_l2norm_makes_forward_scale_invariant_in_q_and_k():
    rng = _rng(44)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 7, 2, 4, 3)
    f = oracle.FLAG_L2NORM_QK
    o1, S1 = oracle.fwd(q, k, v, g, beta, S0, nthreads=2, flags=f)
    o2, S2 = oracle.fwd(5.0 * q, 0.25 * k, v, g, beta, S0, nthreads=2, flags=f)
    assert rel_err(o2, o1) < 1e-13 and rel_err(S2, S1) < 1e-13

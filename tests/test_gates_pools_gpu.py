"""Per-head and absent gates, and slot-indexed state pools, on the GPU.

kda_fwd_chunked_ex / kda_decode_step_ex through the C ABI against the fp64
oracle (oracle.fwd / decode with the same gate layout, oracle.fwd_pooled /
decode_pooled for pools).
"""
import sys

import numpy as np
import pytest
import torch

from gpu_util import TOL, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(B, T, H, dk, dv, dt, seed, gate, lengths=None, s0_std=0.5, gate_mu=-1.0):
    """The usual recipe; a per-head gate is the first key channel's gate values."""
    from gated_delta_rule_81_amd import synth
    x = synth.random_fwd(B, T, H, dk, dv, dtype=dt, seed=seed, gate_mu=gate_mu, s0_std=s0_std,
                         lengths=lengths)
    if gate == "head":
        x["log_alpha"] = x["log_alpha"][..., 0].contiguous()
    elif gate == "none":
        x["log_alpha"] = None
    return x


def _f64o(t):
    return None if t is None else f64(t)


def _run(x, gate, **kw):
    from gated_delta_rule_81_amd import kda
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o, S_T = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"],
                             g["cu_seqlens"], gate=gate, **kw)
    torch.cuda.synchronize()
    return g, o, S_T


def _check(x, gate, o, S_T, tol):
    import oracle
    cu = x["cu_seqlens"].tolist() if x["cu_seqlens"] is not None else None
    o_ref, S_ref = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), _f64o(x["log_alpha"]),
                              f64(x["beta"]), _f64o(x["S0"]), cu, gate=gate)
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S_T), S_ref)
    _say(f"  rel err o={eo:.3e} S_T={es:.3e} (tol {tol})")
    assert eo <= tol and es <= tol, (eo, es)


SMALL = [
    # B, T, H, dk, dv, dtype
    (2, 129, 3, 128, 128, torch.bfloat16),
    (1, 77, 4, 64, 128, torch.bfloat16),
    (2, 100, 2, 128, 64, torch.bfloat16),
    (1, 1, 2, 128, 128, torch.bfloat16),
    (2, 63, 3, 64, 64, torch.float32),
    (1, 200, 2, 64, 128, torch.float32),
]


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("B,T,H,dk,dv,dt", SMALL)
def test_gate_layouts_small(gate, B, T, H, dk, dv, dt):
    _say(f"case: gate={gate} B{B} T{T} H{H} dk{dk} dv{dv} {dt}")
    x = _inputs(B, T, H, dk, dv, dt, seed=T + 3 * H, gate=gate)
    _, o, S_T = _run(x, gate)
    _check(x, gate, o, S_T, TOL[dt])


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("dt,dk", [(torch.bfloat16, 128), (torch.float32, 64), (torch.float32, 128)])
def test_gate_layouts_varlen(gate, dt, dk):
    lens = [0, 1, 63, 64, 65, 130, 0, 7]
    H = 64 if dt == torch.bfloat16 else 3     # bf16: whole d_v per workgroup
    _say(f"case: gate={gate} varlen {lens} H{H} dk{dk} {dt}")
    x = _inputs(1, 0, H, dk, 128 if dk == 128 else 64, dt, seed=6, gate=gate, lengths=lens,
                s0_std=0.3)
    _, o, S_T = _run(x, gate)
    _check(x, gate, o, S_T, TOL[dt])


@pytest.mark.parametrize("kind", ["all_strong", "mixed_chunks"])
@pytest.mark.parametrize("dt,dk", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64),
                                   (torch.float32, 128)])
def test_head_gate_strong_decay(kind, dt, dk):
    """Decay beyond 2^100 within a chunk: the exact per-entry path with a per-head gate."""
    _say(f"case: head gate strong decay {kind} dk{dk} {dt}")
    T, H = 192, 2
    x = _inputs(1, T, H, dk, 64 if dt == torch.float32 else 128, dt, seed=12, gate="head")
    g = x["log_alpha"].float()
    if kind == "all_strong":
        g = torch.full_like(g, -30.0)
    else:
        g[:, 64:128] = -12.0
        g[:, 160:170] = -40.0
    x["log_alpha"] = g.to(dt)
    _, o, S_T = _run(x, "head")
    _check(x, "head", o, S_T, TOL[dt])


@pytest.mark.parametrize("gate", ["head", "none"])
def test_gate_layouts_h16_t4k(gate):
    from gated_delta_rule_81_amd import synth
    _say(f"case: gate={gate} B1 H16 T4096 d128 bf16 (full oracle)")
    x = synth.fwd_inputs(synth.FWD_H16_T4K)
    if gate == "head":
        x["log_alpha"] = x["log_alpha"][..., 0].contiguous()
    else:
        x["log_alpha"] = None
    _, o, S_T = _run(x, gate)
    _check(x, gate, o, S_T, TOL[torch.bfloat16])


def _pool_case(dt, dk, dv, gate, lengths, idx, P, seed):
    x = _inputs(1, 0, 2, dk, dv, dt, seed=seed, gate=gate, lengths=lengths, s0_std=0.0)
    gen = torch.Generator().manual_seed(seed + 100)
    pool = 0.3 * torch.randn(P, 2, dk, dv, generator=gen)
    return x, pool, torch.tensor(idx, dtype=torch.int32)


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dt,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64),
                                      (torch.float32, 64, 64)])
def test_pooled_chunked_in_place(gate, dt, dk, dv):
    """Sequences continued from and into pool rows: a permutation, a padding
    slot (-1) and an index past the pool; S0 and S_T are the same pool."""
    import oracle
    from gated_delta_rule_81_amd import kda
    lens = [40, 0, 70, 33, 5]
    idx = [3, 6, -1, 0, 11]
    P = 7
    _say(f"case: pooled chunked gate={gate} {dt} dk{dk} dv{dv} lens {lens} idx {idx}")
    x, pool, sidx = _pool_case(dt, dk, dv, gate, lens, idx, P, seed=21)
    pool_ref = f64(pool)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    pg = pool.to(DEV)
    o, S_T = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], pg,
                             g["cu_seqlens"], S_T=pg, gate=gate, state_idx=sidx.to(DEV))
    torch.cuda.synchronize()
    assert S_T is pg
    o_ref, pool_new = oracle.fwd_pooled(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                        _f64o(x["log_alpha"]), f64(x["beta"]), pool_ref, idx,
                                        x["cu_seqlens"].tolist(), gate=gate, S_T_pool=pool_ref)
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(pg), pool_new)
    _say(f"  rel err o={eo:.3e} pool={es:.3e}")
    assert eo <= TOL[dt] and es <= TOL[dt]
    # rows that are nobody's slot are untouched, bit for bit
    for r in (1, 2, 4, 5):
        assert torch.equal(pg[r].cpu(), pool[r])


def test_pooled_chunked_dense_batch_separate_pools():
    """Dense batch (no cu_seqlens), S0 and S_T different pools."""
    import oracle
    from gated_delta_rule_81_amd import kda
    dt, dk, dv, P = torch.bfloat16, 128, 128, 5
    idx = [2, 4, 0]
    _say(f"case: pooled dense B3 idx {idx} separate pools")
    x = _inputs(3, 90, 2, dk, dv, dt, seed=23, gate="channel", s0_std=0.0)
    gen = torch.Generator().manual_seed(7)
    pool0 = 0.3 * torch.randn(P, 2, dk, dv, generator=gen)
    pool1 = torch.full((P, 2, dk, dv), 7.0)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    p0, p1 = pool0.to(DEV), pool1.to(DEV)
    o, _ = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], p0, None, S_T=p1,
                           state_idx=torch.tensor(idx, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    o_ref, p1_ref = oracle.fwd_pooled(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]),
                                      f64(x["beta"]), f64(pool0), idx, None, S_T_pool=f64(pool1))
    assert rel_err(f64(o), o_ref) <= TOL[dt]
    assert rel_err(f64(p1), p1_ref) <= TOL[dt]
    assert torch.equal(p0.cpu(), pool0)                 # the input pool is only read
    assert torch.equal(p1[1].cpu(), pool1[1]) and torch.equal(p1[3].cpu(), pool1[3])


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_pooled_decode_chain(gate, dt):
    import oracle
    from gated_delta_rule_81_amd import kda
    N, H, dk, dv, P = 6, 3, 128, 64, 8
    idx = [7, 0, -1, 3, 9, 5]
    _say(f"case: pooled decode gate={gate} {dt} idx {idx}")
    gen = torch.Generator().manual_seed(41)
    pool = 0.2 * torch.randn(P, H, dk, dv, generator=gen)
    pool_ref = f64(pool)
    pg = pool.to(DEV)
    sidx = torch.tensor(idx, dtype=torch.int32, device=DEV)
    for step in range(4):
        x = _inputs(N, 1, H, dk, dv, dt, seed=50 + step, gate=gate, s0_std=0.0)
        xs = {k: (v[:, 0].contiguous() if isinstance(v, torch.Tensor) and v.dim() >= 3 else v)
              for k, v in x.items()}
        if gate == "head":
            xs["log_alpha"] = x["log_alpha"][:, 0].contiguous()
        xg = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in xs.items()}
        o = kda.decode_step(xg["q"], xg["k"], xg["v"], xg["log_alpha"], xg["beta"], pg,
                            gate=gate, state_idx=sidx)
        torch.cuda.synchronize()
        o_ref, pool_ref = oracle.decode_pooled(f64(xs["q"]), f64(xs["k"]), f64(xs["v"]),
                                               _f64o(xs["log_alpha"]), f64(xs["beta"]), pool_ref,
                                               idx, gate=gate)
        eo = rel_err(f64(o), o_ref)
        assert eo <= TOL[dt], (step, eo)
    es = rel_err(f64(pg), pool_ref)
    _say(f"  rel err pool={es:.3e}")
    assert es <= TOL[dt]
    for r in (1, 2, 4, 6):
        assert torch.equal(pg[r].cpu(), pool[r])


@pytest.mark.parametrize("gate", ["channel", "head"])
def test_multi_token_decode_matches_steps(gate):
    """Four tokens per sequence as one chunked call on the pool equal four decode steps."""
    from gated_delta_rule_81_amd import kda
    N, H, dk, dv, P, L = 5, 2, 128, 128, 6, 4
    idx = torch.tensor([5, 1, 0, 3, 2], dtype=torch.int32, device=DEV)
    _say(f"case: multi-token decode gate={gate} N{N} L{L}")
    x = _inputs(1, 0, H, dk, dv, torch.bfloat16, seed=61, gate=gate, lengths=[L] * N, s0_std=0.0)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    gen = torch.Generator().manual_seed(62)
    pool = (0.2 * torch.randn(P, H, dk, dv, generator=gen)).to(DEV)
    pool_a, pool_b = pool.clone(), pool.clone()
    o_chunk, _ = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], pool_a,
                                 g["cu_seqlens"], S_T=pool_a, gate=gate, state_idx=idx)
    outs = []
    for t in range(L):
        tok = torch.arange(N, device=DEV) * L + t
        sel = lambda z: z[0, tok].contiguous()
        outs.append(kda.decode_step(sel(g["q"]), sel(g["k"]), sel(g["v"]), sel(g["log_alpha"]),
                                    sel(g["beta"]), pool_b, gate=gate, state_idx=idx))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).reshape(1, N * L, H, dv)
    assert rel_err(f64(o_dec), f64(o_chunk)) <= TOL[torch.bfloat16]
    assert rel_err(f64(pool_b), f64(pool_a)) <= TOL[torch.bfloat16]
    assert torch.equal(pool_a[4].cpu(), pool[4].cpu()) and torch.equal(pool_b[4].cpu(), pool[4].cpu())


@pytest.mark.parametrize("L", [2, 5])
@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dt,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 128)])
def test_decode_several_tokens_per_sequence(L, gate, dt, dk, dv):
    """L tokens per sequence in one decode call (state kept in registers
    across them), on a pool with padding and out-of-pool slots."""
    import oracle
    from gated_delta_rule_81_amd import kda
    N, H, P = 6, 3, 8
    idx = [7, 0, -1, 3, 9, 5]
    _say(f"case: decode L={L} gate={gate} {dt} dk{dk} dv{dv} idx {idx}")
    x = _inputs(N, L, H, dk, dv, dt, seed=70 + L, gate=gate, s0_std=0.0)
    gen = torch.Generator().manual_seed(71)
    pool = 0.2 * torch.randn(P, H, dk, dv, generator=gen)
    xg = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    pg = pool.to(DEV)
    o = kda.decode_step(xg["q"], xg["k"], xg["v"], xg["log_alpha"], xg["beta"], pg, gate=gate,
                        state_idx=torch.tensor(idx, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert o.shape == (N, L, H, dv)
    # the (N, L, H, .) inputs are N dense sequences of L tokens
    o_ref, pool_ref = oracle.fwd_pooled(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                        _f64o(x["log_alpha"]), f64(x["beta"]), f64(pool), idx,
                                        None, gate=gate, S_T_pool=f64(pool))
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(pg), pool_ref)
    _say(f"  rel err o={eo:.3e} pool={es:.3e}")
    assert eo <= TOL[dt] and es <= TOL[dt]
    for r in (1, 2, 4, 6):
        assert torch.equal(pg[r].cpu(), pool[r])


def test_decode_tokens_match_chunked_and_single_steps():
    """Four tokens per sequence: one decode call with L = 4, the pooled chunked
    forward, and four single-token decode steps agree."""
    from gated_delta_rule_81_amd import kda
    N, H, dk, dv, P, L = 5, 2, 128, 128, 6, 4
    idx = torch.tensor([5, 1, 0, 3, 2], dtype=torch.int32, device=DEV)
    _say(f"case: decode L={L} vs chunked vs steps")
    x = _inputs(N, L, H, dk, dv, torch.bfloat16, seed=81, gate="channel", s0_std=0.0)
    g = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    pool = (0.2 * torch.randn(P, H, dk, dv, generator=torch.Generator().manual_seed(82))).to(DEV)
    pa, pb, pc = pool.clone(), pool.clone(), pool.clone()
    o_l = kda.decode_step(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], pa, state_idx=idx)
    flat = {k_: g[k_].reshape((1, N * L) + g[k_].shape[2:]).contiguous() for k_ in ("q", "k", "v", "log_alpha", "beta")}
    cu = torch.arange(0, N * L + 1, L, dtype=torch.int32, device=DEV)
    o_c, _ = kda.fwd_chunked(flat["q"], flat["k"], flat["v"], flat["log_alpha"], flat["beta"], pb,
                             cu, S_T=pb, state_idx=idx)
    steps = [kda.decode_step(*(g[k_][:, t].contiguous() for k_ in ("q", "k", "v", "log_alpha", "beta")),
                             pc, state_idx=idx) for t in range(L)]
    torch.cuda.synchronize()
    o_s = torch.stack(steps, dim=1)
    tol = TOL[torch.bfloat16]
    assert rel_err(f64(o_l), f64(o_s)) <= tol and rel_err(f64(pa), f64(pc)) <= tol
    assert rel_err(f64(o_l.reshape(1, N * L, H, dv)), f64(o_c)) <= tol
    assert rel_err(f64(pa), f64(pb)) <= tol


def _raw_inputs(B, T, H, dk, dv, dt, seed, gate, flags, lengths=None, strong=False):
    """Inputs for the preparation flags: q and k with row norms far from 1 (when
    normalisation is asked for), and the gate as the softplus input x."""
    x = _inputs(B, T, H, dk, dv, torch.float32, seed=seed, gate="channel", lengths=lengths,
                s0_std=0.3)
    gen = torch.Generator().manual_seed(seed + 1000)
    if flags & 1:
        x["q"] = x["q"] * (0.2 + 5.0 * torch.rand(x["q"].shape[:-1] + (1,), generator=gen))
        x["k"] = x["k"] * (0.2 + 5.0 * torch.rand(x["k"].shape[:-1] + (1,), generator=gen))
        if x["k"].shape[1] > 3:
            x["k"][:, 3] = 0.0                       # a zero key row stays zero
    g = x["log_alpha"]
    if flags & 2:
        g = torch.randn(g.shape, generator=gen) * 1.5 - 1.0
        if strong:
            g[:, 40:60] = 30.0                           # alpha ~ e^-30 per token
    if gate == "head":
        g = g[..., 0].contiguous()
    elif gate == "none":
        g = None
    for key in ("q", "k", "v", "beta", "S0"):
        if x[key] is not None and key != "S0":
            x[key] = x[key].to(dt)
    x["log_alpha"] = None if g is None else g.to(dt)
    return x


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("gate", ["channel", "head", "none"])
@pytest.mark.parametrize("dt,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 128),
                                      (torch.float32, 64, 64)])
def test_prepared_inputs_chunked(flags, gate, dt, dk, dv):
    if gate == "none" and flags == 2:
        pytest.skip("the softplus flag has no gate to act on")
    _say(f"case: chunked flags={flags} gate={gate} {dt} dk{dk} dv{dv}")
    x = _raw_inputs(2, 100, 3, dk, dv, dt, seed=90 + flags, gate=gate, flags=flags)
    _, o, S_T = _run(x, gate, flags=flags)
    import oracle
    o_ref, S_ref = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), _f64o(x["log_alpha"]),
                              f64(x["beta"]), _f64o(x["S0"]), None, gate=gate, flags=flags)
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S_T), S_ref)
    _say(f"  rel err o={eo:.3e} S_T={es:.3e}")
    assert eo <= TOL[dt] and es <= TOL[dt], (eo, es)


@pytest.mark.parametrize("gate", ["channel", "head"])
@pytest.mark.parametrize("dt,dk", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_prepared_inputs_varlen_strong_decay(gate, dt, dk):
    """Both flags, packed sequences, and softplus inputs of 30 (alpha ~ e^-30,
    the exact per-entry path) over some tokens."""
    lens = [0, 70, 33, 129, 5]
    H = 64 if dt == torch.bfloat16 else 3
    _say(f"case: chunked flags=3 gate={gate} varlen {lens} H{H} {dt} dk{dk}")
    x = _raw_inputs(1, 0, H, dk, 128 if dk == 128 else 64, dt, seed=95, gate=gate, flags=3,
                    lengths=lens, strong=True)
    _, o, S_T = _run(x, gate, flags=3)
    import oracle
    cu = x["cu_seqlens"].tolist()
    o_ref, S_ref = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), _f64o(x["log_alpha"]),
                              f64(x["beta"]), _f64o(x["S0"]), cu, gate=gate, flags=3)
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S_T), S_ref)
    _say(f"  rel err o={eo:.3e} S_T={es:.3e}")
    assert eo <= TOL[dt] and es <= TOL[dt], (eo, es)


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("L", [1, 3])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_prepared_inputs_decode(flags, L, dt):
    import oracle
    from gated_delta_rule_81_amd import kda
    N, H, dk, dv, P = 5, 2, 128, 64, 7
    idx = [6, 0, -1, 2, 4]
    _say(f"case: decode flags={flags} L={L} {dt}")
    x = _raw_inputs(N, L, H, dk, dv, dt, seed=96 + L, gate="channel", flags=flags)
    pool = 0.2 * torch.randn(P, H, dk, dv, generator=torch.Generator().manual_seed(97))
    xg = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    pg = pool.to(DEV)
    sel = (lambda z: z) if L > 1 else (lambda z: z[:, 0].contiguous())
    o = kda.decode_step(sel(xg["q"]), sel(xg["k"]), sel(xg["v"]), sel(xg["log_alpha"]),
                        sel(xg["beta"]), pg, state_idx=torch.tensor(idx, dtype=torch.int32, device=DEV),
                        flags=flags)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle.fwd_pooled(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]),
                                        f64(x["beta"]), f64(pool), idx, None, S_T_pool=f64(pool),
                                        flags=flags)
    if L == 1:
        o_ref = o_ref[:, 0]
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(pg), pool_ref)
    _say(f"  rel err o={eo:.3e} pool={es:.3e}")
    assert eo <= TOL[dt] and es <= TOL[dt], (eo, es)

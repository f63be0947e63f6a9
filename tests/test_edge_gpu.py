"""The operator at the edges of its domain, on the GPU against the fp64 oracle.

Cases (gated_delta_rule_81_amd.synth.EDGE_KINDS): beta drawn in [-0.5, 2),
beta exactly 0, exactly 1, or drawn from {0, 1}; keys that are not
normalised (norms 0.1 .. 4); a key element just above 2^16 in one 32-token
block (the bf16 forward's exact pairwise path); and the associative-recall
case of the delta rule: with orthonormal keys, no decay and beta = 1,
writing a key a second time replaces its value, so a query with that key
recalls exactly the latest value and every other key its own
(akshathtiwari.co.in "Kimi Delta Attention" explainer, the delta-rule
paragraph and the closing description of its first widget; "Teacher guide
-- Kimi Delta Attention", Misconceptions table, third row).

Each case runs through the chunked forward, a chain of decode steps and the
backward, with bf16 and fp32 inputs, and every output is compared element by
element with the oracle on the same inputs (max |x - ref| / max |ref| per
tensor within 1e-4 for fp32 inputs, 2e-2 for bf16).  Outputs are filled with
NaN before each call, so an element the kernels never write fails the check.
"""
import sys

import numpy as np
import pytest
import torch

from gpu_util import TOL, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KINDS = ("beta_wide", "beta_zero", "beta_one", "beta_01", "raw_keys", "big_key", "overwrite")
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(kind, dt, dk, dv, T=200, B=2, H=2, seed=0):
    from gated_delta_rule_81_amd import synth
    return synth.edge_fwd(kind, B, T, H, dk, dv, dtype=dt, seed=seed + 17 * dk + dv)


def _dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _oracle_fwd(x):
    import oracle
    S0 = f64(x["S0"]) if x["S0"] is not None else None
    return oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]),
                      f64(x["beta"]), S0)


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _check_recall(x, o, tol):
    """Query tokens of the overwrite case recall the latest value of their key."""
    exp = x["expected"]
    rows = ~torch.isnan(exp[..., 0])
    got = o.float().cpu()[rows]
    want = exp[rows]
    err = rel_err(got.numpy(), want.numpy())
    _say(f"  recall of latest values: rel err {err:.3e} over {int(rows.sum())} queries")
    assert err <= tol, err


FWD_CASES = [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64), (torch.float32, 64, 64),
             (torch.float32, 128, 128)]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt,dk,dv", FWD_CASES)
def test_edge_chunked_forward(kind, dt, dk, dv):
    from gated_delta_rule_81_amd import kda
    _say(f"case: edge forward {kind} {dt} dk{dk} dv{dv}")
    x = _inputs(kind, dt, dk, dv)
    g = _dev(x)
    B, T, H = x["B"], x["T"], x["H"]
    o = _nan((B, T, H, dv), dt)
    S_T = _nan((B, H, dk, dv), torch.float32)
    kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], o=o, S_T=S_T)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle_fwd(x)
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S_T), S_ref)
    _say(f"  rel err o={eo:.3e} S_T={es:.3e} (tol {TOL[dt]})")
    assert eo <= TOL[dt] and es <= TOL[dt], (eo, es)
    if kind == "overwrite":
        _check_recall(x, o, TOL[dt])
        # the oracle recalls the same values
        _check_recall(x, torch.from_numpy(o_ref), 1e-12)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64)])
def test_edge_decode_chain(kind, dt, dk, dv):
    """The same inputs one token at a time through kda_decode_step (one state
    per sequence, rewritten in place), against the oracle's token loop."""
    from gated_delta_rule_81_amd import kda
    T = 104 if kind == "overwrite" else 70
    _say(f"case: edge decode chain {kind} {dt} dk{dk} dv{dv} T{T}")
    x = _inputs(kind, dt, dk, dv, T=T)
    g = _dev(x)
    B, T, H = x["B"], x["T"], x["H"]
    S = g["S0"].clone() if g["S0"] is not None else torch.zeros(B, H, dk, dv, device=DEV)
    outs = []
    for t in range(T):
        o_t = _nan((B, H, dv), dt)
        kda.decode_step(*(z[:, t].contiguous() for z in
                          (g["q"], g["k"], g["v"], g["log_alpha"], g["beta"])), S, o=o_t)
        outs.append(o_t)
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1)
    o_ref, S_ref = _oracle_fwd(x)
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S), S_ref)
    _say(f"  rel err o={eo:.3e} S={es:.3e} (tol {TOL[dt]})")
    assert eo <= TOL[dt] and es <= TOL[dt], (eo, es)
    if kind == "overwrite":
        _check_recall(x, o, TOL[dt])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64),
                                      (torch.float32, 64, 64)])
def test_edge_backward(kind, dt, dk, dv):
    import oracle
    from gated_delta_rule_81_amd import kda
    T = 0 if kind == "overwrite" else 130
    _say(f"case: edge backward {kind} {dt} dk{dk} dv{dv}")
    x = _inputs(kind, dt, dk, dv, T=T)
    g = _dev(x)
    B, T, H = x["B"], x["T"], x["H"]
    gen = torch.Generator().manual_seed(23)
    dO = torch.randn((B, T, H, dv), generator=gen).to(dt)
    dST = torch.randn((B, H, dk, dv), generator=gen)
    out = (_nan((B, T, H, dk), dt), _nan((B, T, H, dk), dt), _nan((B, T, H, dv), dt),
           _nan((B, T, H, dk), dt), _nan((B, T, H), dt), _nan((B, H, dk, dv), torch.float32))
    got = kda.bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], dO.to(DEV), g["S0"],
                          dST.to(DEV), out=out)
    torch.cuda.synchronize()
    S0 = f64(x["S0"]) if x["S0"] is not None else None
    ref = oracle.bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]), f64(x["beta"]),
                     S0, f64(dO), f64(dST))
    errs = {n: rel_err(f64(a), b) for n, a, b in zip(NAMES, got, ref)}
    _say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {TOL[dt]})")
    bad = {n: e for n, e in errs.items() if not e <= TOL[dt]}
    assert not bad, bad

"""A bounded wait that runs out inside the chunked forward is reported, never
passed off as a result.

The wait limit is forced to 0 from the host (kda_set_wait_limit), so every
hand-off wait in the bf16 chunk kernel gives up at once and every workgroup
stops early; all kernels still exit normally.  The outputs must then be NaN
and the device error word must carry KDA_DEVERR_WAIT_TIMEOUT.  With the
default limit restored the same call gives the oracle's result and no error.
"""
import sys

import pytest
import torch

from gpu_util import TOL, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_wait_timeout_poisons_outputs_and_sets_error_bit():
    import oracle
    from gated_delta_rule_81_amd import kda, synth
    _say("case: forced wait timeout, bf16 B2 T150 H2 d128")
    x = synth.random_fwd(2, 150, 2, 128, 128, dtype=torch.bfloat16, seed=71, gate_mu=-1.0,
                         s0_std=0.5)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    assert kda.device_errors(clear=True) == 0
    kda.set_wait_limit(0)
    try:
        o = torch.zeros((2, 150, 2, 128), dtype=torch.bfloat16, device=DEV)
        S_T = torch.zeros((2, 2, 128, 128), dtype=torch.float32, device=DEV)
        kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], o=o, S_T=S_T)
        bits = kda.device_errors(clear=True)
    finally:
        kda.set_wait_limit(kda.WAIT_LIMIT_DEFAULT)
    _say(f"  error bits {bits}; o NaN {torch.isnan(o.float()).float().mean().item():.3f}, "
         f"S_T NaN {torch.isnan(S_T).float().mean().item():.3f}")
    assert bits & kda.KDA_DEVERR_WAIT_TIMEOUT
    # nothing was produced: every element is NaN, none is a plausible number
    assert torch.isnan(o.float()).all() and torch.isnan(S_T).all()
    assert kda.device_errors() == 0

    # the backward's first kernel is the same chain: the bit is set there too
    kda.set_wait_limit(0)
    try:
        gen = torch.Generator().manual_seed(72)
        dO = torch.randn(g["v"].shape, generator=gen).to(torch.bfloat16).to(DEV)
        kda.bwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], dO, g["S0"], None)
        bits = kda.device_errors(clear=True)
    finally:
        kda.set_wait_limit(kda.WAIT_LIMIT_DEFAULT)
    assert bits & kda.KDA_DEVERR_WAIT_TIMEOUT

    # default limit: the oracle's result, no error
    o, S_T = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"])
    assert kda.device_errors() == 0
    o_ref, S_ref = oracle.fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]),
                              f64(x["beta"]), f64(x["S0"]))
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S_T), S_ref)
    _say(f"  default limit: rel err o={eo:.3e} S_T={es:.3e}")
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]

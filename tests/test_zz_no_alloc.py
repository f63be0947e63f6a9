"""kda_fwd_chunked_noalloc (the forward with its scratch in a fixed device
array, for callers that cannot allocate) against kda_fwd_chunked_ex with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, each equal bit for bit to the workspace call on the same
inputs (the same kernels run on the same data), and within tolerance of the
oracle.  Also: more packed sequences than the scratch holds is rejected
before anything is enqueued."""
import sys

import pytest
import torch

from gpu_util import TOL, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(lengths, H, dk, dv, seed):
    from gated_delta_rule_81_amd import synth
    x = synth.random_fwd(1, 0, H, dk, dv, dtype=torch.bfloat16, seed=seed, gate_mu=-1.0,
                         s0_std=0.3, lengths=lengths)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _pair(g):
    from gated_delta_rule_81_amd import kda
    B, T, H, dv = 1, g["T"], g["H"], g["dv"]
    o_ws, S_ws = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"],
                                 g["cu_seqlens"])
    o = torch.full((B, T, H, dv), float("nan"), dtype=g["q"].dtype, device=DEV)
    S_T = torch.full_like(S_ws, float("nan"))
    kda.fwd_chunked_noalloc(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"],
                            g["cu_seqlens"], o, S_T)
    torch.cuda.synchronize()
    return o_ws, S_ws, o, S_T


def test_noalloc_matches_workspace_call_twice():
    import oracle
    big = [300, 0, 65, 1, 129, 700, 33, 64] * 12            # 96 sequences
    small = [70, 5, 0, 40]
    for label, lens, seed in (("first", big, 1), ("second, smaller", small, 2)):
        _say(f"case: noalloc {label}: {len(lens)} sequences, {sum(lens)} tokens, H3 d128 bf16")
        g = _case(lens, 3, 128, 128, seed)
        o_ws, S_ws, o, S_T = _pair(g)
        assert torch.equal(o, o_ws) and torch.equal(S_T, S_ws)
        cu = g["cu_seqlens"].tolist()
        o_ref, S_ref = oracle.fwd(f64(g["q"]), f64(g["k"]), f64(g["v"]), f64(g["log_alpha"]),
                                  f64(g["beta"]), f64(g["S0"]), cu)
        eo, es = rel_err(f64(o), o_ref), rel_err(f64(S_T), S_ref)
        _say(f"  bit-identical to the workspace call; oracle rel err o={eo:.3e} S_T={es:.3e}")
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_noalloc_dense_call():
    from gated_delta_rule_81_amd import kda, synth
    x = synth.random_fwd(2, 150, 2, 64, 64, dtype=torch.float32, seed=9, gate_mu=-1.0, s0_std=0.5)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    o_ws, S_ws = kda.fwd_chunked(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"])
    o = torch.empty_like(o_ws)
    S_T = torch.empty_like(S_ws)
    kda.fwd_chunked_noalloc(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], None, o, S_T)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(S_T, S_ws)


def test_noalloc_rejects_too_many_sequences():
    from gated_delta_rule_81_amd import kda
    n = kda.NOALLOC_MAX_SEQS + 1
    cu = torch.zeros(n + 1, dtype=torch.int32, device=DEV)
    z = torch.zeros((1, 0, 1, 64), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((1, 0, 1), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kda.KdaError) as e:
        kda.fwd_chunked_noalloc(z, z, z, z, b, None, cu, z)
    assert e.value.status == kda.KDA_ERR_SCRATCH_LIMIT

"""The entry points under HIP graph capture (torch.cuda.CUDAGraph).

Each call is captured once and the graph replayed several times, with eager
work and synchronisations between the replays and an input changed in place
before each one; every replay must equal an eager call on the same inputs,
bit for bit (the kernels are deterministic).  The calls allocate nothing
inside the library and record no memset, so they can sit inside a captured
serving or training step.
"""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _eager_noise():
    # unrelated eager work between replays
    a = torch.randn(256, 256, device=DEV)
    (a @ a).sum().item()
    torch.cuda.synchronize()


def _capture(fn):
    """Warm up on a side stream, then capture fn into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(warm=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(warm=False)
    torch.cuda.synchronize()
    return g


def test_decode_graph_replays():
    from gated_delta_rule_81_amd import kda
    _say("[graph decode] N=8 H=4 d=128 bf16, 3 replays")
    gen = torch.Generator(device=DEV).manual_seed(71)
    N, H, d = 8, 4, 128
    bf = torch.bfloat16
    q = torch.nn.functional.normalize(torch.randn(N, H, d, generator=gen, device=DEV), dim=-1).to(bf)
    k = torch.nn.functional.normalize(torch.randn(N, H, d, generator=gen, device=DEV), dim=-1).to(bf)
    v = torch.randn(N, H, d, generator=gen, device=DEV).to(bf)
    la = (-torch.nn.functional.softplus(torch.randn(N, H, d, generator=gen, device=DEV) - 2)).to(bf)
    b = torch.sigmoid(torch.randn(N, H, generator=gen, device=DEV)).to(bf)
    S0 = 0.02 * torch.randn(N, H, d, d, generator=gen, device=DEV)
    S_g = S0.clone()
    o_g = torch.empty(N, H, d, dtype=bf, device=DEV)
    S_w = S0.clone()

    def call(warm):
        kda.decode_step(q, k, v, la, b, S_w if warm else S_g, o=o_g)

    g = _capture(call)
    assert torch.equal(S_g, S0)                      # capture runs nothing
    S_e = S0.clone()
    for r in range(3):
        v.neg_()                                     # a new token's values, in place
        o_e = kda.decode_step(q, k, v, la, b, S_e)
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"o differs at replay {r}"
        assert torch.equal(S_g, S_e), f"state differs at replay {r}"


@pytest.mark.parametrize("varlen", [False, True])
def test_fwd_graph_replays(varlen):
    from gated_delta_rule_81_amd import kda, synth
    lengths = [45, 0, 70, 33] if varlen else None
    _say(f"[graph fwd] varlen={varlen} bf16, 3 replays")
    x = synth.random_fwd(2 if not varlen else 1, 100 if not varlen else 0, 2, 128, 128,
                         dtype=torch.bfloat16, seed=73, gate_mu=-1.0, s0_std=0.5,
                         lengths=lengths, device=DEV)
    N = len(lengths) if varlen else 2
    o_g = torch.empty_like(x["v"])
    S_g = torch.empty(N, 2, 128, 128, device=DEV)
    ws = torch.empty(max(kda.workspace_bytes(x["B"], x["T"], 2, 128, 128, N), 1),
                     dtype=torch.uint8, device=DEV)

    def call(warm):
        kda.fwd_chunked(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"], x["cu_seqlens"],
                        o=o_g, S_T=S_g, workspace=ws)

    g = _capture(call)
    for r in range(3):
        x["v"].neg_()
        o_e, S_e = kda.fwd_chunked(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"],
                                   x["cu_seqlens"])
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"o differs at replay {r}"
        assert torch.equal(S_g, S_e), f"S_T differs at replay {r}"


def test_bwd_graph_replays():
    from gated_delta_rule_81_amd import kda, synth
    _say("[graph bwd] B=1 T=100 H=2 d=128 bf16, 2 replays")
    x = synth.random_fwd(1, 100, 2, 128, 128, dtype=torch.bfloat16, seed=79, gate_mu=-1.0,
                         s0_std=0.5, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(80)
    dO = torch.randn(x["v"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    dST = torch.randn(1, 2, 128, 128, generator=gen, device=DEV)
    out = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]),
           torch.empty_like(x["log_alpha"]), torch.empty_like(x["beta"]),
           torch.empty(1, 2, 128, 128, device=DEV))
    ws = torch.empty(kda.bwd_workspace_bytes(1, 100, 2, 128, 128, 1), dtype=torch.uint8, device=DEV)

    def call(warm):
        kda.bwd_chunked(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], dO, x["S0"], dST,
                        workspace=ws, out=out)

    g = _capture(call)
    for r in range(2):
        dO.neg_()
        ref = kda.bwd_chunked(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], dO, x["S0"], dST)
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        for name, a, e in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), out, ref):
            assert torch.equal(a, e), f"{name} differs at replay {r}"

"""Seeded synthetic inputs: determinism, shapes, dtypes and the recipe's properties."""
import torch

from gated_delta_rule_81_amd import synth


def test_tiny_workload_shapes_and_recipe():
    x = synth.fwd_inputs(synth.TINY_FP32)
    B, T, H, d = 1, 256, 2, 64
    assert x["q"].shape == (B, T, H, d) and x["q"].dtype == torch.float32
    assert x["v"].shape == (B, T, H, d) and x["beta"].shape == (B, T, H)
    assert x["S0"] is None and x["cu_seqlens"] is None
    assert torch.allclose(x["q"].norm(dim=-1), torch.ones(B, T, H), atol=1e-5)
    assert torch.allclose(x["k"].norm(dim=-1), torch.ones(B, T, H), atol=1e-5)
    assert (x["log_alpha"] < 0).all()
    assert ((x["beta"] > 0) & (x["beta"] < 1)).all()


def test_seeded_and_deterministic():
    a = synth.fwd_inputs(synth.TINY_FP32)
    b = synth.fwd_inputs(synth.TINY_FP32)
    for key in ("q", "k", "v", "log_alpha", "beta"):
        assert torch.equal(a[key], b[key])
    c = synth.random_fwd(1, 256, 2, 64, 64, seed=1)
    assert not torch.equal(a["q"], c["q"])


def test_bf16_workload_rounding_and_state():
    x = synth.fwd_inputs(synth.FWD_H16_T4K, T=128)
    assert x["q"].dtype == torch.bfloat16 and x["S0"].dtype == torch.float32
    assert x["S0"].shape == (1, 16, 128, 128)
    assert abs(float(x["S0"].std()) - 0.02) < 0.002
    # slow decay with a wide channel spread: mean -softplus(N(-2, 1)) is about -0.17
    la = x["log_alpha"].float()
    assert -0.25 < float(la.mean()) < -0.1 and float(la.min()) < -1.0


def test_varlen_lengths_and_offsets():
    lens = synth.varlen_lengths(synth.VARLEN_64)
    assert len(lens) == 64 and min(lens) >= 512 and max(lens) <= 16384
    assert lens == synth.varlen_lengths(synth.VARLEN_64)
    x = synth.fwd_inputs(synth.VARLEN_64, lengths=[5, 0, 9])
    assert x["cu_seqlens"].tolist() == [0, 5, 5, 14]
    assert x["q"].shape[:2] == (1, 14) and x["S0"].shape[0] == 3


def test_decode_inputs_fresh_per_step():
    w = synth.DECODE_512
    a = synth.decode_step_inputs(w, 0, N=4)
    b = synth.decode_step_inputs(w, 1, N=4)
    assert a["q"].shape == (4, 32, 128) and a["beta"].shape == (4, 32)
    assert not torch.equal(a["q"], b["q"])
    assert torch.equal(a["v"], synth.decode_step_inputs(w, 0, N=4)["v"])

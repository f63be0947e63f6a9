"""Seeded synthetic inputs for the KDA operator.

This module only draws random numbers and shapes them into the operator's
inputs; it holds none of the operator's arithmetic.  Both the GPU path and the
fp64 oracle consume what it returns (the oracle after a copy to the host), so
neither side generates its own data.

Recipe (per workload):
  q, k  ~ N(0, 1), then L2-normalised per token over d_k
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1))                       one scalar per token and head
  log_alpha = -softplus(N(mu, 1))                one value per token, head, key channel
            mu = 0 for the tiny fp32 case, mu = -2 elsewhere (slow decay, wide spread)
  S0    = 0 (tiny case) or N(0, 0.02^2) (sigma = 0.02)
  varlen lengths ~ U{512 .. 16384} (inclusive), drawn first
Draw order from one generator seeded with the workload seed:
  lengths (varlen only), q, k, v, beta logits, gate logits, S0.
Values are drawn in fp32 and rounded once to the storage dtype (bf16 by
round-to-nearest-even).  The generator is torch's, on the device the tensors
are made on; the same seed on another device type gives other numbers, so a
parity test always generates on one device and copies to the other.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class FwdWorkload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    gate_mu: float
    s0_std: float          # 0.0 -> S0 = zeros (passed as None)
    seed: int
    varlen: Optional[List[int]] = None   # sequence lengths (B must be 1)
    varlen_n: int = 0                     # draw this many lengths when varlen is None
    varlen_lo: int = 512
    varlen_hi: int = 16384


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    steps: int
    gate_mu: float
    s0_std: float
    seed: int


# The five workloads of the operator: parity-only tiny fp32, two bf16 dense
# shapes, packed variable-length, and chained decode.
TINY_FP32 = FwdWorkload("kda_fwd_tiny_fp32_B1_H2_T256_d64", 1, 256, 2, 64, 64,
                        torch.float32, 0.0, 0.0, 0)
FWD_H16_T4K = FwdWorkload("kda_fwd_bf16_B1_H16_T4096_d128", 1, 4096, 16, 128, 128,
                          torch.bfloat16, -2.0, 0.02, 1)
FWD_H32_T8K = FwdWorkload("kda_fwd_bf16_B4_H32_T8192_d128", 4, 8192, 32, 128, 128,
                          torch.bfloat16, -2.0, 0.02, 2)
VARLEN_64 = FwdWorkload("kda_fwd_varlen_bf16_64seq_512to16384_H32_d128", 1, 0, 32, 128, 128,
                        torch.bfloat16, -2.0, 0.02, 3, varlen=None, varlen_n=64)
DECODE_512 = DecodeWorkload("kda_decode_bf16_N512_H32_d128_1000steps", 512, 32, 128, 128,
                            torch.bfloat16, 1000, -2.0, 0.02, 4)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def varlen_lengths(w: FwdWorkload, device="cpu") -> List[int]:
    """Sequence lengths of a packed workload (drawn first from its seed)."""
    if w.varlen is not None:
        return list(w.varlen)
    g = _gen(device, w.seed)
    lens = torch.randint(w.varlen_lo, w.varlen_hi + 1, (w.varlen_n,), generator=g, device=device)
    return [int(x) for x in lens.cpu()]


def fwd_inputs(w: FwdWorkload, device="cpu", T: Optional[int] = None,
               lengths: Optional[List[int]] = None) -> dict:
    """Inputs of one forward call.

    Returns a dict with q, k, v, log_alpha, beta (storage dtype), S0 (fp32 or
    None), cu_seqlens (int32 tensor or None), and the shape fields.
    ``T`` overrides the workload's sequence length (dense case only);
    ``lengths`` overrides the packed lengths.
    """
    g = _gen(device, w.seed)
    f32 = dict(device=device, dtype=torch.float32)
    is_varlen = lengths is not None or w.varlen is not None or w.varlen_n > 0
    if is_varlen:
        if lengths is None:
            if w.varlen is not None:
                lengths = list(w.varlen)
            else:
                lens = torch.randint(w.varlen_lo, w.varlen_hi + 1, (w.varlen_n,),
                                     generator=g, device=device)
                lengths = [int(x) for x in lens.cpu()]
        B, Ttot, N = 1, int(sum(lengths)), len(lengths)
        cu = torch.zeros(N + 1, dtype=torch.int64)
        if N:
            cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
        cu_seqlens = cu.to(torch.int32).to(device)
    else:
        B, Ttot, N = w.B, (w.T if T is None else T), w.B
        cu_seqlens = None
    H, dk, dv = w.H, w.dk, w.dv
    q = _unit_rows(torch.randn(B, Ttot, H, dk, generator=g, **f32))
    k = _unit_rows(torch.randn(B, Ttot, H, dk, generator=g, **f32))
    v = torch.randn(B, Ttot, H, dv, generator=g, **f32)
    beta = torch.sigmoid(torch.randn(B, Ttot, H, generator=g, **f32))
    log_alpha = -F.softplus(torch.randn(B, Ttot, H, dk, generator=g, **f32) + w.gate_mu)
    S0 = None
    if w.s0_std > 0:
        S0 = w.s0_std * torch.randn(N, H, dk, dv, generator=g, **f32)
    dt = w.dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=log_alpha.to(dt),
                beta=beta.to(dt), S0=S0, cu_seqlens=cu_seqlens,
                B=B, T=Ttot, H=H, dk=dk, dv=dv, N=N, lengths=lengths)


def decode_state(w: DecodeWorkload, device="cpu") -> torch.Tensor:
    """Initial fp32 state cache (N, H, dk, dv) ~ N(0, s0_std^2)."""
    g = _gen(device, w.seed)
    return w.s0_std * torch.randn(w.N, w.H, w.dk, w.dv, generator=g, device=device,
                                  dtype=torch.float32)


def decode_step_inputs(w: DecodeWorkload, step: int, device="cpu", N: Optional[int] = None) -> dict:
    """Fresh q, k, v, beta, log_alpha for decode step ``step`` (own seed per step)."""
    g = _gen(device, w.seed * 1_000_003 + 7919 * (step + 1))
    n = w.N if N is None else N
    f32 = dict(device=device, dtype=torch.float32)
    H, dk, dv = w.H, w.dk, w.dv
    q = _unit_rows(torch.randn(n, H, dk, generator=g, **f32))
    k = _unit_rows(torch.randn(n, H, dk, generator=g, **f32))
    v = torch.randn(n, H, dv, generator=g, **f32)
    beta = torch.sigmoid(torch.randn(n, H, generator=g, **f32))
    log_alpha = -F.softplus(torch.randn(n, H, dk, generator=g, **f32) + w.gate_mu)
    dt = w.dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=log_alpha.to(dt), beta=beta.to(dt))


def random_fwd(B, T, H, dk, dv, dtype=torch.float32, seed=0, gate_mu=0.0, s0_std=0.0,
               lengths=None, device="cpu") -> dict:
    """Small ad-hoc shapes for tests (same recipe as the named workloads)."""
    w = FwdWorkload(f"adhoc_{B}x{T}x{H}x{dk}x{dv}", B, T, H, dk, dv, dtype, gate_mu,
                    s0_std, seed, varlen=list(lengths) if lengths is not None else None)
    return fwd_inputs(w, device=device)


# ---- inputs at the edges of the operator's domain ---------------------------
#
# Each case changes one thing about the recipe above (seeded like it); the
# tests run the GPU path and the oracle on the same tensors.
#   beta_wide    beta ~ U[-0.5, 2): negative and greater-than-one write strengths
#   beta_zero    beta = 0 exactly: nothing is written, only decay
#   beta_one     beta = 1 exactly
#   beta_01      beta drawn from {0, 1}
#   raw_keys     keys not normalised: unit directions times norms ~ U[0.1, 4],
#                beta = u * 1.9 / |k|^2 with u ~ U(0, 1) (so beta |k|^2 < 2 and
#                the state stays bounded; beta itself spans about 0 .. 190)
#   big_key      as the recipe, but one 32-token block (tokens 32..63) holds a
#                key with one element just above 2^16 in magnitude (66048) and
#                beta = 1 / |k|^2 on that token
#   overwrite    associative recall: orthonormal keys (rows of a Hadamard
#                matrix / 8 at d_k = 64, signed unit vectors otherwise; exact in
#                bf16), no decay (log_alpha = 0), S0 = 0; tokens 0..47 write
#                keys 0..47 with beta = 1, tokens 48..55 write new values for
#                keys 1, 7, 13, .., 43 with beta = 1, tokens 56..103 query every
#                key (q = k = key j, beta = 0)
EDGE_KINDS = ("beta_wide", "beta_zero", "beta_one", "beta_01", "raw_keys", "big_key", "overwrite")

OVERWRITE_WRITES = 48
OVERWRITE_REWRITES = tuple(range(1, 48, 6))          # keys written a second time
OVERWRITE_T = 48 + len(OVERWRITE_REWRITES) + 48      # writes, rewrites, queries


def _hadamard(n: int) -> torch.Tensor:
    h = torch.ones(1, 1)
    while h.shape[0] < n:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return h


def orthonormal_keys(dk: int, g: torch.Generator) -> torch.Tensor:
    """dk orthonormal rows whose entries are exact in bf16: a row-permuted
    Hadamard matrix scaled by 1/8 at dk = 64, signed permuted unit vectors
    otherwise."""
    perm = torch.randperm(dk, generator=g)
    if dk == 64:
        return _hadamard(64)[perm] / 8.0
    sign = torch.where(torch.rand(dk, generator=g) < 0.5, -1.0, 1.0)
    return torch.eye(dk)[perm] * sign[:, None]


def edge_fwd(kind: str, B: int, T: int, H: int, dk: int, dv: int, dtype=torch.bfloat16,
             seed: int = 0, gate_mu: float = -1.0, s0_std: float = 0.5) -> dict:
    """Forward inputs for one of EDGE_KINDS (generated on the CPU).  For
    "overwrite" T is fixed (OVERWRITE_T) and the result also holds
    "expected": (B, OVERWRITE_T, H, dv) fp32 values the query tokens must
    recall (the latest value written for their key; rows of write tokens are
    NaN), as bookkeeping of which value was written last -- no arithmetic of
    the operator."""
    if kind not in EDGE_KINDS:
        raise ValueError(f"unknown edge case {kind!r}")
    if kind == "overwrite":
        return _overwrite_inputs(B, H, dk, dv, dtype, seed)
    x = random_fwd(B, T, H, dk, dv, dtype=torch.float32, seed=seed, gate_mu=gate_mu,
                   s0_std=s0_std)
    g = _gen("cpu", seed * 7 + 13)
    beta = x["beta"]
    if kind == "beta_wide":
        beta = torch.rand(beta.shape, generator=g) * 2.5 - 0.5
    elif kind == "beta_zero":
        beta = torch.zeros_like(beta)
    elif kind == "beta_one":
        beta = torch.ones_like(beta)
    elif kind == "beta_01":
        beta = (torch.rand(beta.shape, generator=g) < 0.5).float()
    elif kind == "raw_keys":
        norms = 0.1 + 3.9 * torch.rand(x["k"].shape[:-1] + (1,), generator=g)
        k = (x["k"] * norms).to(dtype).float()     # the stored keys decide beta below
        sq = (k * k).sum(-1)
        beta = torch.rand(beta.shape, generator=g).clamp_min(1e-3) * 1.9 / sq
        x["k"] = k
    elif kind == "big_key":
        t = min(40, T - 1)
        k = x["k"].clone()
        k[:, t, :, 3] = 66048.0                     # bf16 0x4781: just above 2^16
        sq = (k[:, t].to(dtype).float() ** 2).sum(-1)
        beta = beta.clone()
        beta[:, t] = 1.0 / sq
        x["k"] = k
    x["beta"] = beta
    for key in ("q", "k", "v", "log_alpha", "beta"):
        x[key] = x[key].to(dtype)
    return x


def _overwrite_inputs(B, H, dk, dv, dtype, seed):
    g = _gen("cpu", seed)
    T = OVERWRITE_T
    q = torch.zeros(B, T, H, dk)
    k = torch.zeros(B, T, H, dk)
    v = torch.zeros(B, T, H, dv)
    beta = torch.zeros(B, T, H)
    expected = torch.full((B, T, H, dv), float("nan"))
    nw, nr = OVERWRITE_WRITES, len(OVERWRITE_REWRITES)
    for b in range(B):
        for h in range(H):
            keys = orthonormal_keys(dk, g)[:nw]
            vals = torch.randn(nw, dv, generator=g).to(dtype).float()
            latest = vals.clone()
            k[b, :nw, h] = keys
            v[b, :nw, h] = vals
            beta[b, :nw, h] = 1.0
            for i, j in enumerate(OVERWRITE_REWRITES):
                new = torch.randn(dv, generator=g).to(dtype).float()
                k[b, nw + i, h] = keys[j]
                v[b, nw + i, h] = new
                beta[b, nw + i, h] = 1.0
                latest[j] = new
            q[b, : nw + nr, h] = torch.randn(nw + nr, dk, generator=g) / dk ** 0.5
            order = torch.randperm(nw, generator=g)
            for i, j in enumerate(order.tolist()):
                t = nw + nr + i
                q[b, t, h] = keys[j]
                k[b, t, h] = keys[j]
                v[b, t, h] = torch.randn(dv, generator=g)
                expected[b, t, h] = latest[j]
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype),
                log_alpha=torch.zeros(B, T, H, dk).to(dtype), beta=beta.to(dtype), S0=None,
                cu_seqlens=None, B=B, T=T, H=H, dk=dk, dv=dv, N=B, lengths=None,
                expected=expected)

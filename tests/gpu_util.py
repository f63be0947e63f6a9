"""Helpers shared by the GPU parity tests: tolerances and sampled oracle runs."""
from __future__ import annotations

import numpy as np
import torch

# max |x - ref| / max |ref| per tensor (o and final state separately)
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/fp32 tensor to a float64 numpy array on the host."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / (scale if scale > 0 else 1.0))


def unit_slices(x: dict, seq: int, head: int):
    """Token slice and batch row of one (sequence, head) unit of forward inputs."""
    cu = x["cu_seqlens"]
    if cu is None:
        return seq, slice(0, x["T"])
    cuh = cu.tolist() if isinstance(cu, torch.Tensor) else list(cu)
    return 0, slice(cuh[seq], cuh[seq + 1])


def oracle_on_units(x: dict, units, o_gpu: torch.Tensor, S_gpu, nthreads=None):
    """Run the fp64 oracle on selected (sequence, head) units of a forward call.

    The selected units are packed as separate sequences of one varlen oracle
    call (units are independent), so the oracle's threads work on them in
    parallel.  Returns (rel error of o, rel error of S_T) over all selected
    units together.
    """
    import oracle
    parts = {k: [] for k in ("q", "k", "v", "log_alpha", "beta")}
    S0s, o_got, S_got, lens = [], [], [], []
    for seq, head in units:
        b, ts = unit_slices(x, seq, head)
        hs = slice(head, head + 1)
        for key in parts:
            parts[key].append(f64(x[key][b:b + 1, ts, hs]))
        lens.append(parts["q"][-1].shape[1])
        if x["S0"] is not None:
            S0s.append(f64(x["S0"][seq:seq + 1, hs]))
        else:
            dk, dv = x["q"].shape[-1], x["v"].shape[-1]
            S0s.append(np.zeros((1, 1, dk, dv)))
        o_got.append(f64(o_gpu[b:b + 1, ts, hs]).reshape(-1))
        if S_gpu is not None:
            S_got.append(f64(S_gpu[seq:seq + 1, hs]).reshape(-1))
    cat = {k: np.concatenate(v, axis=1) for k, v in parts.items()}
    cu = np.concatenate([[0], np.cumsum(lens)])
    o_ref, S_ref = oracle.fwd(cat["q"], cat["k"], cat["v"], cat["log_alpha"], cat["beta"],
                              np.concatenate(S0s, axis=0), cu, nthreads=nthreads)
    eo = rel_err(np.concatenate(o_got), o_ref.reshape(-1))
    es = rel_err(np.concatenate(S_got), S_ref.reshape(-1)) if S_gpu is not None else 0.0
    return eo, es


def sample_units(n_seqs: int, H: int, count: int, seed: int):
    g = torch.Generator().manual_seed(seed)
    idx = torch.randperm(n_seqs * H, generator=g)[:count].tolist()
    return [(i // H, i % H) for i in idx]

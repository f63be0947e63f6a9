"""A seeded sweep of shape combinations on the GPU against the fp64 oracle.

The fixed-shape parity tests pick their shapes by hand; this sweep draws the
forward's and the backward's arguments together from one seeded generator, so
that unusual combinations meet: batch or packed sequences (empty and short
ones included), a ragged last chunk, 1 to 5 heads, every (d_k, d_v) pair, both
input precisions, the three gate layouts, with and without an initial state.
Each case is compared element by element at the same tolerances as the rest
of the suite; the case list is the same on every run.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL
from test_bwd_gpu import _case as _bwd_case, _compare as _bwd_compare, _gpu as _bwd_gpu, _ref as _bwd_ref
from test_gates_pools_gpu import _check as _fwd_check, _inputs as _fwd_inputs, _run as _fwd_run

pytestmark = pytest.mark.gpu

_DIMS = [(64, 64), (64, 128), (128, 64), (128, 128)]
_GATES = ["channel", "head", "none"]


def _draw(n, seed, max_t, max_len):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dk, dv = _DIMS[int(rng.integers(len(_DIMS)))]
        dt = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        gate = _GATES[int(rng.integers(len(_GATES)))]
        H = int(rng.integers(1, 6))
        if rng.random() < 0.4:
            lengths = [int(v) for v in rng.integers(0, max_len, size=int(rng.integers(1, 6)))]
            B, T = 1, 0
        else:
            lengths = None
            B, T = int(rng.integers(1, 4)), int(rng.integers(1, max_t))
        s0 = bool(rng.random() < 0.7)
        cases.append(pytest.param(B, T, H, dk, dv, dt, gate, lengths, s0, int(rng.integers(1, 1 << 20)),
                                  id=f"c{i}"))
    return cases


@pytest.mark.parametrize("B,T,H,dk,dv,dt,gate,lengths,s0,seed", _draw(16, 20251203, 260, 180))
def test_forward_sweep(B, T, H, dk, dv, dt, gate, lengths, s0, seed):
    print(f"case: fwd sweep B{B} T{T} H{H} dk{dk} dv{dv} {dt} gate={gate} lengths={lengths} "
          f"s0={s0} seed={seed}", flush=True)
    x = _fwd_inputs(B, T, H, dk, dv, dt, seed, gate, lengths=lengths, s0_std=0.5 if s0 else 0.0)
    _, o, S_T = _fwd_run(x, gate)
    _fwd_check(x, gate, o, S_T, TOL[dt])


@pytest.mark.parametrize("B,T,H,dk,dv,dt,gate,lengths,s0,seed", _draw(10, 20251204, 200, 140))
def test_backward_sweep(B, T, H, dk, dv, dt, gate, lengths, s0, seed):
    print(f"case: bwd sweep B{B} T{T} H{H} dk{dk} dv{dv} {dt} gate={gate} lengths={lengths} "
          f"s0={s0} seed={seed}", flush=True)
    x = _bwd_case(B, T, H, dk, dv, dt, seed, gate=gate, lengths=lengths, s0=s0)
    _bwd_compare(_bwd_gpu(x, gate), _bwd_ref(x, gate), TOL[dt], "sweep")

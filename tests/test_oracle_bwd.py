"""The oracle's backward against its pins, and planted mistakes against them.

Each mutant is a copy of oracle/kda_oracle.c with one plausible slip in the
backward token step (a dropped term, a wrong sign, the wrong operand or
state), compiled on the CPU; at least one pin of oracle_bwd_pins.py must fail
for each.
"""
import os
import subprocess

import pytest

import oracle
from oracle_bwd_pins import BWD_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_bwd_pin(pin):
    pin(oracle.load())


# (name, exact text in kda_oracle.c, replacement)
MUTANTS = [
    ("dq_without_write", "acc += (Sp[(size_t)i * dv + j] + k[i] * u[j]) * dO[j];",
     "acc += Sp[(size_t)i * dv + j] * dO[j];"),
    ("no_output_term", "dS[(size_t)i * dv + j] += q[i] * dO[j];", "(void)0;"),
    ("output_term_with_key", "dS[(size_t)i * dv + j] += q[i] * dO[j];",
     "dS[(size_t)i * dv + j] += k[i] * dO[j];"),
    ("dk_from_v", "acc += dS[(size_t)i * dv + j] * u[j];", "acc += dS[(size_t)i * dv + j] * v[j];"),
    ("dbeta_without_read", "db += du[j] * (v[j] - e[j]);", "db += du[j] * v[j];"),
    ("de_sign", "du[j] = -beta * du[j];", "du[j] = beta * du[j];"),
    ("dv_without_beta", "dvt[j] = beta * du[j];", "dvt[j] = du[j];"),
    ("no_read_term_in_dk", "        dkt[i] += acc;\n", "        (void)acc;\n"),
    ("no_read_term_in_dS", "dS[(size_t)i * dv + j] += k[i] * du[j];", "(void)0;"),
    ("dgate_from_previous_state", "acc += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];",
     "acc += dS[(size_t)i * dv + j] * S_prev[(size_t)i * dv + j];"),
    ("no_decay_in_state_gradient", "dS[(size_t)i * dv + j] *= a;", "(void)a;"),
    ("checkpoint_off_by_one", "memcpy(seg, ck + (size_t)m * SS, sizeof(double) * SS);",
     "memcpy(seg, ck + (size_t)(m > 0 ? m - 1 : 0) * SS, sizeof(double) * SS);"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    c_path = tmp_path / f"mut_{name}.c"
    so_path = tmp_path / f"mut_{name}.so"
    c_path.write_text(src.replace(old, new, 1))
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                    str(so_path), str(c_path), "-lm"], check=True)
    return str(so_path)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_bwd_mutant_is_caught(tmp_path, name, old, new):
    lib = oracle.load_path(_build_mutant(tmp_path, name, old, new))
    failed = []
    for pin in BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("C", [1, 7, 32])
def test_chunk_form_backward_matches_oracle(C):
    """The chunked backward algebra (chunk_form.chunk_step_bwd, the form the GPU
    kernels take) reaches the oracle's token-loop gradients in fp64, with a
    ragged last chunk."""
    import numpy as np
    from chunk_form import chunked_backward
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 2, 77, 2, 6, 5
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk)) / np.sqrt(dk)
    v = rng.normal(size=(B, T, H, dv))
    g = -np.log1p(np.exp(rng.normal(-1, 1, size=(B, T, H, dk))))
    b = rng.random((B, T, H))
    S0 = rng.normal(size=(B, H, dk, dv))
    dO = rng.normal(size=(B, T, H, dv))
    dST = rng.normal(size=(B, H, dk, dv))
    ref = oracle.bwd(q, k, v, g, b, S0, dO, dST)
    got = chunked_backward(q, k, v, g, b, S0, dO, dST, C)
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
        err = float(np.max(np.abs(x - y)) / np.max(np.abs(y)))
        assert err < 1e-12, (name, err)

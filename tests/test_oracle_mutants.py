"""Planted mistakes in the oracle's C loop must each fail at least one pin.

Each mutant is a copy of oracle/kda_oracle.c with one plausible slip (a
dropped term, a wrong sign, a wrong index, a transposed operand, an
off-by-one), compiled into a temporary library on the CPU.  The pins of
oracle_pins.py are then run against it; a mutant that passes every pin would
mean the pins cannot tell that slip from the real recurrence.
"""
import os
import subprocess

import pytest

from oracle_pins import ALL_PINS, backend

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

# (name, exact text in kda_oracle.c, replacement)
MUTANTS = [
    ("no_decay", "S[(size_t)i * dv + j] *= a;", "(void)a;"),
    ("decay_sign", "exp(log_alpha[i])", "exp(-log_alpha[i])"),
    ("scalar_gate_channel0", "exp(log_alpha[i])", "exp(log_alpha[0])"),
    ("decay_by_value_column", "S[(size_t)i * dv + j] *= a;",
     "S[(size_t)i * dv + j] *= exp(log_alpha[j % dk]); (void)a;"),
    ("error_sign", "u[j] = beta * (v[j] - e);", "u[j] = beta * (v[j] + e);"),
    ("no_beta", "u[j] = beta * (v[j] - e);", "u[j] = (v[j] - e);"),
    ("no_subtract", "u[j] = beta * (v[j] - e);", "u[j] = beta * v[j];"),
    ("read_with_query", "e += S[(size_t)i * dv + j] * k[i];", "e += S[(size_t)i * dv + j] * q[i];"),
    ("write_with_query", "S[(size_t)i * dv + j] += k[i] * u[j];", "S[(size_t)i * dv + j] += q[i] * u[j];"),
    ("output_with_key", "acc += S[(size_t)i * dv + j] * q[i];", "acc += S[(size_t)i * dv + j] * k[i];"),
    ("transposed_read", "e += S[(size_t)i * dv + j] * k[i];",
     "e += S[(size_t)(j % dk) * dv + (i % dv)] * k[i];"),
    ("drop_last_token", "for (long t = t0; t < t1; ++t)", "for (long t = t0; t + 1 < t1; ++t)"),
    ("s0_of_first_sequence", "if (S0) memcpy(S, S0 + sidx,", "if (S0) memcpy(S, S0 + (size_t)h * dk * dv,"),
    ("beta_of_head0", "beta[th]", "beta[th - h]"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / f"mut_{name}.c"
    so_path = tmp_path / f"mut_{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                    str(so_path), str(c_path), "-lm"], check=True)
    return str(so_path)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    import oracle
    lib = oracle.load_path(_build_mutant(tmp_path, name, old, new))
    be = backend(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(be)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

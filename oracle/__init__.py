"""fp64 CPU oracle for the Kimi Delta Attention recurrence (test infrastructure).

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of bench.py
may import this package.  The GPU library never imports or calls it.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    load_path,
    fwd,
    decode,
    bwd,
    prepare_vjp,
    brute_force,
    channel_gate,
    pool_rows,
    fwd_pooled,
    decode_pooled,
    GATES,
    prepare,
    FLAG_L2NORM_QK,
    FLAG_GATE_SOFTPLUS,
    max_threads,
    default_threads,
)

"""C ABI checks that need no GPU: symbols, status strings, argument validation.

Every call here returns before any HIP launch (invalid or empty arguments), so
it runs on a host without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kda_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from gated_delta_rule_81_amd import kda
    return kda.lib()


def test_header_declares_expected_entry_points():
    assert declared_functions() == ["kda_bwd_chunked", "kda_bwd_workspace_bytes",
                                    "kda_decode_step", "kda_decode_step_ex", "kda_device_errors",
                                    "kda_fwd_chunked", "kda_fwd_chunked_ex",
                                    "kda_fwd_chunked_noalloc",
                                    "kda_fwd_workspace_bytes", "kda_set_wait_limit",
                                    "kda_status_string"]


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings(L):
    from gated_delta_rule_81_amd import kda
    assert kda.status_string(0) == "KDA_OK"
    assert kda.status_string(1) == "KDA_ERR_INVALID_ARG"
    assert kda.status_string(2) == "KDA_ERR_UNSUPPORTED"
    assert kda.status_string(3) == "KDA_ERR_HIP"
    assert kda.status_string(4) == "KDA_ERR_SCRATCH_LIMIT"
    assert kda.status_string(99) == "KDA_ERR_UNKNOWN"


def test_workspace_bytes(L):
    from gated_delta_rule_81_amd import kda
    assert kda.workspace_bytes(1, 100, 32, 128, 128, 1) == 0
    assert kda.workspace_bytes(1, 100, 32, 128, 128, 64) >= 64 * 4
    assert kda.workspace_bytes(1, 100, 32, 128, 128, 64) % 256 == 0


FAKE = 1 << 20   # a 16-byte aligned non-NULL address; never dereferenced


def fwd(L, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, S0=None, cu=None, N=0, B=1, T=64, H=2,
        dk=128, dv=128, dt=1, o=FAKE, S_T=None, ws=None, wsb=0):
    return L.kda_fwd_chunked(q, k, v, g, b, S0, cu, N, B, T, H, dk, dv, dt, o, S_T, ws, wsb, None)


def dec(L, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, S=FAKE, N=4, H=2, dk=128, dv=128, dt=1, o=FAKE):
    return L.kda_decode_step(q, k, v, g, b, S, N, H, dk, dv, dt, o, None)


@pytest.mark.parametrize("dk,dv", [(32, 128), (128, 96), (256, 128), (128, 256)])
def test_fwd_unsupported_sizes(L, dk, dv):
    assert fwd(L, dk=dk, dv=dv) == 2


@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("dk,dv", [(96, 64), (64, 32), (256, 128)])
def test_fwd_unsupported_dims(L, dt, dk, dv):
    assert fwd(L, dk=dk, dv=dv, dt=dt) == 2


@pytest.mark.parametrize("kw", [dict(q=None), dict(k=None), dict(v=None), dict(g=None),
                                dict(b=None), dict(o=None)])
def test_fwd_null_pointers(L, kw):
    assert fwd(L, **kw) == 1


@pytest.mark.parametrize("kw", [dict(B=-1), dict(T=-1), dict(H=0), dict(dt=7)])
def test_fwd_bad_sizes(L, kw):
    assert fwd(L, **kw) == 1


@pytest.mark.parametrize("kw", [dict(q=FAKE + 4), dict(o=FAKE + 2), dict(S0=FAKE + 8),
                                dict(S_T=FAKE + 12)])
def test_fwd_misaligned(L, kw):
    assert fwd(L, **kw) == 1


def test_fwd_varlen_rules(L):
    # cu_seqlens needs B == 1
    assert fwd(L, cu=FAKE, N=4, B=2) == 1
    # negative number of sequences
    assert fwd(L, cu=FAKE, N=-1) == 1
    # more than one packed sequence needs a workspace of the reported size
    assert fwd(L, cu=FAKE, N=8) == 1
    assert fwd(L, cu=FAKE, N=8, ws=FAKE, wsb=16) == 1
    # zero sequences: nothing to do
    assert fwd(L, cu=FAKE, N=0, T=0) == 0


def test_fwd_empty_batch_is_ok(L):
    assert fwd(L, B=0, T=0) == 0
    assert fwd(L, q=None, k=None, v=None, g=None, b=None, o=None, B=0, T=0) == 0


@pytest.mark.parametrize("kw", [dict(q=None), dict(S=None), dict(o=None)])
def test_decode_null_pointers(L, kw):
    assert dec(L, **kw) == 1


@pytest.mark.parametrize("kw", [dict(dk=96), dict(dv=32)])
def test_decode_unsupported(L, kw):
    assert dec(L, **kw) == 2


@pytest.mark.parametrize("kw", [dict(N=-1), dict(H=0), dict(dt=5), dict(S=FAKE + 4)])
def test_decode_invalid(L, kw):
    assert dec(L, **kw) == 1


def test_decode_empty_is_ok(L):
    assert dec(L, N=0) == 0


def fwd_ex(L, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, gate=0, flags=0, S0=None, S_T=None, idx=None,
           P=0, cu=None, N=0, B=1, T=64, H=2, dk=128, dv=128, dt=1, o=FAKE, ws=None, wsb=0):
    return L.kda_fwd_chunked_ex(q, k, v, g, b, gate, flags, S0, S_T, idx, P, cu, N, B, T, H, dk, dv,
                                dt, o, ws, wsb, None)


def dec_ex(L, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, gate=0, flags=0, S=FAKE, idx=None, P=0, N=4,
           T=1, H=2, dk=128, dv=128, dt=1, o=FAKE):
    return L.kda_decode_step_ex(q, k, v, g, b, gate, flags, S, idx, P, N, T, H, dk, dv, dt, o, None)


@pytest.mark.parametrize("gate", [-1, 3, 100])
def test_ex_rejects_unknown_gate(L, gate):
    assert fwd_ex(L, gate=gate) == 1
    assert dec_ex(L, gate=gate) == 1


def test_ex_gate_needs_log_alpha_unless_none(L):
    assert fwd_ex(L, g=None, gate=0) == 1
    assert fwd_ex(L, g=None, gate=1) == 1
    assert dec_ex(L, g=None, gate=0) == 1
    assert dec_ex(L, g=None, gate=1) == 1
    # without a gate log_alpha is not read: NULL and even misaligned pass the checks
    assert fwd_ex(L, g=None, gate=2, B=0, T=0) == 0
    assert fwd_ex(L, g=FAKE + 2, gate=2, B=0, T=0) == 0
    assert dec_ex(L, g=None, gate=2, N=0) == 0


def test_ex_slot_map_rules(L):
    assert fwd_ex(L, idx=FAKE, P=-1) == 1
    assert fwd_ex(L, idx=FAKE + 2, P=4) == 1            # int32 array misaligned
    assert dec_ex(L, idx=FAKE, P=-1) == 1
    assert dec_ex(L, idx=FAKE + 1, P=4) == 1
    # the ordinary checks still apply
    assert fwd_ex(L, dk=96) == 2
    assert dec_ex(L, dv=32) == 2
    assert fwd_ex(L, cu=FAKE, N=8, idx=FAKE, P=8) == 1  # varlen workspace missing
    assert fwd_ex(L, B=0, T=0, idx=FAKE, P=0) == 0


@pytest.mark.parametrize("flags", [4, 8, 0x80000000])
def test_ex_rejects_unknown_flags(L, flags):
    assert fwd_ex(L, flags=flags) == 1
    assert dec_ex(L, flags=flags) == 1
    # known flags pass the checks (empty work)
    assert fwd_ex(L, flags=3, B=0, T=0) == 0
    assert dec_ex(L, flags=3, N=0) == 0


def test_decode_ex_tokens_per_sequence(L):
    assert dec_ex(L, T=-1) == 1
    assert dec_ex(L, T=0) == 0                          # nothing to do
    assert dec_ex(L, T=0, q=None, S=None) == 0
    assert dec_ex(L, T=3, q=None) == 1


def test_binding_rejects_bad_gate_shapes():
    import torch
    from gated_delta_rule_81_amd import kda
    q = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError, match="gate must be one of"):
        kda.fwd_chunked(q, q, q, q, torch.zeros(1, 4, 2), gate="token")
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.fwd_chunked(q, q, q, None, torch.zeros(1, 4, 2), gate="none")


def test_binding_rejects_cpu_and_mismatched_tensors():
    import torch
    from gated_delta_rule_81_amd import kda
    q = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.fwd_chunked(q, q.clone(), q.clone(), q.clone(), torch.zeros(1, 4, 2), None)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.decode_step(q[0], q[0].clone(), q[0].clone(), q[0].clone(), torch.zeros(4, 2),
                        torch.zeros(4, 2, 64, 64))


def bwd(L, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, gate=0, S0=None, dO=FAKE, dST=None, cu=None,
        N=0, B=1, T=64, H=2, dk=128, dv=128, dt=1, dq=FAKE, dk_=FAKE, dv_=FAKE, dg=FAKE,
        db=FAKE, dS0=None, ws=None, wsb=0):
    return L.kda_bwd_chunked(q, k, v, g, b, gate, S0, dO, dST, cu, N, B, T, H, dk, dv, dt, dq,
                             dk_, dv_, dg, db, dS0, ws, wsb, None)


def test_bwd_workspace_bytes(L):
    from gated_delta_rule_81_amd import kda
    # per (32-token chunk slot, head): two fp32 dk x dv matrices and three 32 x 32
    n = kda.bwd_workspace_bytes(4, 8192, 32, 128, 128, 4)
    slots = 32 * (4 * 256 + 4 + 1)
    assert n >= slots * (2 * 128 * 128 + 3 * 32 * 32) * 4
    assert n % 256 == 0
    assert kda.bwd_workspace_bytes(1, 100, 2, 64, 64, 3) >= 2 * (4 + 3 + 1) * (2 * 64 * 64 + 3 * 1024) * 4
    assert kda.bwd_workspace_bytes(-1, 100, 2, 64, 64, 1) == 0


@pytest.mark.parametrize("kw", [dict(q=None), dict(k=None), dict(v=None), dict(g=None),
                                dict(b=None), dict(dO=None), dict(dq=None), dict(dk_=None),
                                dict(dv_=None), dict(dg=None), dict(db=None)])
def test_bwd_null_pointers(L, kw):
    assert bwd(L, ws=FAKE, wsb=1 << 40, **kw) == 1


@pytest.mark.parametrize("kw", [dict(dk=32), dict(dv=256), dict(dk=96)])
def test_bwd_unsupported_sizes(L, kw):
    assert bwd(L, **kw) == 2


@pytest.mark.parametrize("kw", [dict(dt=2), dict(gate=3), dict(B=-1), dict(H=0),
                                dict(q=FAKE + 4), dict(dS0=FAKE + 8), dict(dg=FAKE + 2)])
def test_bwd_invalid(L, kw):
    assert bwd(L, ws=FAKE, wsb=1 << 40, **kw) == 1


def test_bwd_workspace_rules(L):
    from gated_delta_rule_81_amd import kda
    need = kda.bwd_workspace_bytes(1, 64, 2, 128, 128, 1)
    assert bwd(L) == 1                                   # no workspace
    assert bwd(L, ws=FAKE, wsb=need - 1) == 1            # too small
    assert bwd(L, ws=FAKE + 16, wsb=need) == 1           # not 256-byte aligned
    # no gate: log_alpha and dlog_alpha unused
    assert bwd(L, g=None, dg=None, gate=2, B=0) == 0
    # varlen needs B == 1
    assert bwd(L, cu=FAKE, N=2, B=2) == 1
    assert bwd(L, B=0) == 0                              # nothing to do


def test_diagnostics_argument_checks(L):
    # no GPU work: both return before touching the device
    assert L.kda_set_wait_limit(-1) == 1
    assert L.kda_device_errors(None, 0, None) == 1
    assert L.kda_set_wait_limit(1 << 20) == 0

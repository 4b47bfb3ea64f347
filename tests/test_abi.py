"""The C ABI without a GPU: the library loads, exports every function that
include/mita.h declares, and rejects bad arguments on the host before any
HIP call (so these run on a machine with no GPU).  No compute call is made
with valid arguments here."""
import ctypes
import math
import os
import re

import pytest

import mixture_top_sparse_amd as mts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mita.h")

A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mita_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mts.LIB_PATH):
        pytest.fail("libmita.so is not built (run __graft_entry__.build())")
    return mts.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert "mita_forward" in names and "mita_forward_ex" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in mita.h but not exported"


def test_version_and_status_strings(L):
    assert mts.mita_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert mts.mita_status_string(code)
    assert mts.mita_status_string(12345) == "unknown status"


def call(L, **over):
    a = dict(Q=A, K=A, V=A, dtype=1, B=2, H=3, N=4096, d=64, grid=None, m=64, k=64, scale=0.125,
             out=A, idx=A, route=A, stream=None, dbg=None)
    a.update(over)
    g = None
    if a["grid"] is not None:
        g = ctypes.byref(mts.MitaGrid(*a["grid"]))
    args = [a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"], a["d"], g, a["m"], a["k"],
            a["scale"], a["out"], a["idx"], a["route"], a["stream"]]
    if a["dbg"] is not None:
        return L.mita_forward_ex(*args, ctypes.byref(mts.MitaIntermediates(*a["dbg"])))
    return L.mita_forward(*args)


INVALID = {
    "null_q": dict(Q=None),
    "null_v": dict(V=None),
    "null_out": dict(out=None),
    "null_idx": dict(idx=None),
    "null_route": dict(route=None),
    "bad_dtype": dict(dtype=7),
    "zero_batch": dict(B=0),
    "zero_heads": dict(H=0),
    "zero_tokens": dict(N=0),
    "huge_n": dict(N=1 << 31),
    "m_zero": dict(m=0),
    "m_above_n": dict(N=32, m=33, k=8),
    "k_zero": dict(k=0),
    "k_above_n": dict(N=32, m=8, k=33),
    "scale_zero": dict(scale=0.0),
    "scale_negative": dict(scale=-1.0),
    "scale_nan": dict(scale=math.nan),
    "scale_inf": dict(scale=math.inf),
    "grid_tokens": dict(grid=(14, 14, 5, 5), N=200, m=25),
    "grid_landmarks": dict(grid=(14, 14, 5, 5), N=196, m=24),
    "grid_landmarks_exceed": dict(grid=(2, 98, 4, 1), N=196, m=4),
    "grid_nonpositive": dict(grid=(0, 196, 1, 4), N=196, m=4),
    "misaligned_q": dict(Q=A + 8),
    "misaligned_out": dict(out=A + 4),
    "misaligned_dbg": dict(dbg=(A + 2, None, None, None)),
}

UNSUPPORTED = {
    "d_128": dict(d=128),
    "m_65": dict(m=65),
    "k_65": dict(k=65),
    "too_many_heads": dict(B=300, H=300),
}


@pytest.mark.parametrize("case", sorted(INVALID))
def test_invalid_arguments(L, case):
    assert call(L, **INVALID[case]) == mts.MITA_ERR_INVALID_ARG
    assert mts.mita_last_error() != ""


@pytest.mark.parametrize("case", sorted(UNSUPPORTED))
def test_unsupported(L, case):
    assert call(L, **UNSUPPORTED[case]) == mts.MITA_ERR_UNSUPPORTED
    assert mts.mita_last_error() != ""


def call_noalloc(L, **over):
    a = dict(Q=A, K=A, V=A, dtype=1, B=2, H=3, N=4096, d=64, grid=None, m=64, k=64, scale=0.125,
             out=A, idx=A, route=A, stream=None)
    a.update(over)
    g = None if a["grid"] is None else ctypes.byref(mts.MitaGrid(*a["grid"]))
    return L.mita_forward_noalloc(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"],
                                  a["d"], g, a["m"], a["k"], a["scale"], a["out"], a["idx"],
                                  a["route"], a["stream"])


@pytest.mark.parametrize("case", sorted(set(INVALID) - {"misaligned_dbg"}))
def test_noalloc_invalid_arguments(L, case):
    """The no-allocation entry point validates exactly like mita_forward."""
    assert call_noalloc(L, **INVALID[case]) == mts.MITA_ERR_INVALID_ARG
    assert mts.mita_last_error() != ""


def test_noalloc_rejects_work_space_beyond_scratch(L):
    """2^23 tokens x 2 heads needs more than the 64 MiB static array (the
    query permutation alone is 64 MiB): rejected on the host, with the byte
    counts, before any launch."""
    assert call_noalloc(L, B=1, H=2, N=1 << 23) == mts.MITA_ERR_UNSUPPORTED
    msg = mts.mita_last_error()
    assert "scratch" in msg and str(64 << 20) in msg


def call_s(L, s, **over):
    a = dict(Q=A, K=A, V=A, dtype=1, B=2, H=3, N=4096, d=64, grid=None, m=64, k=64, scale=0.125,
             out=A, idx=A, route=A, stream=None)
    a.update(over)
    return L.mita_forward_s(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"], a["d"],
                            None, a["m"], a["k"], s, a["scale"], a["out"], a["idx"], a["route"],
                            a["stream"])


@pytest.mark.parametrize("s, over, want", [
    (0, {}, "invalid"), (65, {}, "invalid"), (3, dict(m=2), "invalid"),
    (9, {}, "unsupported"), (2, dict(dtype=0), "unsupported"),
    (2, dict(Q=None), "invalid"), (2, dict(scale=-1.0), "invalid")])
def test_forward_s_argument_checks(L, s, over, want):
    """mita_forward_s validates s (1 <= s <= m, s <= 8, bf16 for s > 1) and
    every other argument as mita_forward does, before any HIP call."""
    code = mts.MITA_ERR_INVALID_ARG if want == "invalid" else mts.MITA_ERR_UNSUPPORTED
    assert call_s(L, s, **over) == code
    assert mts.mita_last_error() != ""


def test_injected_allocation_failure(L, monkeypatch):
    monkeypatch.setenv("MITA_FAULT_INJECT", "alloc")
    assert call(L) == mts.MITA_ERR_OOM
    assert "injected" in mts.mita_last_error()


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mts.mita_forward(q, q, q, m=4, k=4)


def test_profiler_without_calls(L):
    mts.mita_profile_enable(True)
    ms, calls = mts.mita_profile_read()
    assert calls == 0 and list(ms) == ["pool", "landmark_threshold", "route", "landmark_scan",
                                       "landmark_merge", "expert_attend", "single_launch",
                                       "bw_zero", "bw_pool", "bw_landmark_fwd", "bw_bucket",
                                       "bw_attend", "bw_cross", "bw_pool_grad"]
    mts.mita_profile_enable(False)


# ---- mita_backward ---------------------------------------------------------


def bw_call(L, **over):
    a = dict(Q=A, K=A, V=A, dtype=1, B=2, H=3, N=4096, d=64, grid=None, m=64, k=64, scale=0.125,
             idx=A, route=A, dout=A, dQ=A, dK=A + 0x100, dV=A + 0x200, stream=None)
    a.update(over)
    g = None if a["grid"] is None else ctypes.byref(mts.MitaGrid(*a["grid"]))
    return L.mita_backward(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"], a["d"], g,
                           a["m"], a["k"], a["scale"], a["idx"], a["route"], a["dout"], a["dQ"],
                           a["dK"], a["dV"], a["stream"])


BW_INVALID = dict(
    {k_: v for k_, v in INVALID.items()
     if k_ not in ("null_out", "misaligned_out", "misaligned_dbg")},
    null_dout=dict(dout=None), null_dq=dict(dQ=None), null_dk=dict(dK=None),
    null_dv=dict(dV=None), misaligned_dout=dict(dout=A + 4), misaligned_dk=dict(dK=A + 8),
    same_dk_dv=dict(dV=A + 0x100), same_dq_dk=dict(dK=A),
)


@pytest.mark.parametrize("case", sorted(BW_INVALID))
def test_backward_invalid_arguments(L, case):
    """mita_backward validates on the host like mita_forward, plus its own
    gradient buffers, before any HIP call."""
    assert bw_call(L, **BW_INVALID[case]) == mts.MITA_ERR_INVALID_ARG
    assert mts.mita_last_error() != ""


@pytest.mark.parametrize("case", sorted(UNSUPPORTED))
def test_backward_unsupported(L, case):
    assert bw_call(L, **UNSUPPORTED[case]) == mts.MITA_ERR_UNSUPPORTED


def test_backward_injected_allocation_failure(L, monkeypatch):
    monkeypatch.setenv("MITA_FAULT_INJECT", "alloc")
    assert bw_call(L) == mts.MITA_ERR_OOM
    assert "injected" in mts.mita_last_error()


# ---- mita_dense_attention (the full-attention baseline) ------------------


def dense_call(L, **over):
    a = dict(Q=A, K=A, V=A, dtype=1, B=2, H=3, N=4096, d=64, scale=0.125, out=A, stream=None)
    a.update(over)
    return L.mita_dense_attention(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"],
                                  a["d"], a["scale"], a["out"], a["stream"])


DENSE_INVALID = {
    "null_q": dict(Q=None),
    "null_out": dict(out=None),
    "bad_dtype": dict(dtype=7),
    "zero_tokens": dict(N=0),
    "huge_n": dict(N=1 << 31),
    "scale_zero": dict(scale=0.0),
    "scale_nan": dict(scale=math.nan),
    "misaligned_k": dict(K=A + 8),
}

DENSE_UNSUPPORTED = {
    "f32": dict(dtype=0),
    "d_96": dict(d=96),
    "too_many_heads": dict(B=300, H=300),
}


@pytest.mark.parametrize("case", sorted(DENSE_INVALID))
def test_dense_invalid_arguments(L, case):
    assert dense_call(L, **DENSE_INVALID[case]) == mts.MITA_ERR_INVALID_ARG
    assert mts.mita_last_error() != ""


@pytest.mark.parametrize("case", sorted(DENSE_UNSUPPORTED))
def test_dense_unsupported(L, case):
    assert dense_call(L, **DENSE_UNSUPPORTED[case]) == mts.MITA_ERR_UNSUPPORTED
    assert mts.mita_last_error() != ""

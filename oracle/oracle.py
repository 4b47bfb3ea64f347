"""ctypes wrapper around ``libmita_oracle.so`` (the fp64 C oracle).

Test infrastructure only.  Every function takes and returns numpy arrays; the
inputs are converted to fp64 (exactly, for bf16 and fp32 values) and made
contiguous before the call.  All arithmetic happens in the C library; this
file only marshals arguments.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

ROUND_NONE = 0
ROUND_F32 = 1
ROUND_BF16 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mita_oracle.c")
_SO = os.path.join(_HERE, "libmita_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build() -> str:
    """Compile the oracle with gcc (plain IEEE fp64: no fast-math, no FMA
    contraction) into ``oracle/libmita_oracle.so``."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _SO + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    L.mita_oracle_round_bf16.restype = ctypes.c_double
    L.mita_oracle_round_bf16.argtypes = [ctypes.c_double]
    L.mita_oracle_window.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64p, _i64p, _i64p, _i64p]
    L.mita_oracle_pool.argtypes = [_f64p, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                   _f64p]
    L.mita_oracle_topk.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _i64, _i32p, _f64p]
    L.mita_oracle_landmark_values.argtypes = [_f64p, _f64p, _f64p, _i64, _i64, _i64,
                                              ctypes.c_double, _f64p]
    L.mita_oracle_route.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _i64p, _i64, _i32p, _f64p]
    L.mita_oracle_bucket.argtypes = [_i32p, _i64, _i64, _i32p, _i32p]
    L.mita_oracle_output.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p, _i32p, _i32p, _i64,
                                     _i64, _i64, _i64, ctypes.c_double, _i64p, _i64, _f64p]
    L.mita_oracle_forward.argtypes = [_f64p, _f64p, _f64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _f64p,
                                      _i32p, _i32p, _f64p, _f64p, _i32p, _i32p]
    L.mita_oracle_dense.argtypes = [_f64p, _f64p, _f64p, _i64, _i64, ctypes.c_double, _i64p,
                                    _i64, _f64p]
    L.mita_oracle_route_s.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _i64, _i64p, _i64, _i32p]
    L.mita_oracle_bucket_s.argtypes = [_i32p, _i64, _i64, _i64, _i32p, _i32p]
    L.mita_oracle_output_s.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p, _i32p, _i32p, _i64,
                                       _i64, _i64, _i64, _i64, ctypes.c_double, _i64p, _i64,
                                       _f64p]
    L.mita_oracle_backward.argtypes = [_f64p, _f64p, _f64p, _i64, _i64, _i64, _i64, _i64, _i64,
                                       _i64, ctypes.c_double, ctypes.c_int, _i32p, _i32p, _f64p,
                                       _f64p, _f64p, _f64p]
    L.mita_oracle_threads.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        _lib = _load(_SO)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Temporarily route every call to another build of the oracle source
    (the mutation tests use this to check that the pins catch planted
    mistakes)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def threads() -> int:
    return int(lib().mita_oracle_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: np.ndarray, t):
    if a is None:
        return None
    return a.ctypes.data_as(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def round_bf16(x: float) -> float:
    return float(lib().mita_oracle_round_bf16(float(x)))


def window(gh: int, gw: int, mh: int, mw: int, i: int) -> tuple[int, int, int, int]:
    r0, r1, c0, c1 = (ctypes.c_int64() for _ in range(4))
    _check(lib().mita_oracle_window(gh, gw, mh, mw, i, ctypes.byref(r0), ctypes.byref(r1),
                                    ctypes.byref(c0), ctypes.byref(c1)), "window")
    return r0.value, r1.value, c0.value, c1.value


def pool(Q, gh: int, gw: int, mh: int, mw: int, round_mode: int = ROUND_NONE) -> np.ndarray:
    Q = _f64(Q)
    N, d = Q.shape
    Ql = np.empty((mh * mw, d), np.float64)
    _check(lib().mita_oracle_pool(_p(Q, _f64p), N, d, gh, gw, mh, mw, round_mode,
                                  _p(Ql, _f64p)), "pool")
    return Ql


def topk(Ql, K, k: int, with_gap: bool = False):
    Ql, K = _f64(Ql), _f64(K)
    m, d = Ql.shape
    N = K.shape[0]
    idx = np.empty((m, k), np.int32)
    gap = np.empty((m, 4), np.float64) if with_gap else None
    _check(lib().mita_oracle_topk(_p(Ql, _f64p), _p(K, _f64p), N, d, m, k, _p(idx, _i32p),
                                  _p(gap, _f64p)), "topk")
    return (idx, gap) if with_gap else idx


def landmark_values(Ql, K, V, scale: float) -> np.ndarray:
    Ql, K, V = _f64(Ql), _f64(K), _f64(V)
    m, d = Ql.shape
    N = K.shape[0]
    Vl = np.empty((m, d), np.float64)
    _check(lib().mita_oracle_landmark_values(_p(Ql, _f64p), _p(K, _f64p), _p(V, _f64p), N, d, m,
                                             float(scale), _p(Vl, _f64p)), "landmark_values")
    return Vl


def route(Q, Ql, qsel=None, with_top2: bool = False):
    Q, Ql = _f64(Q), _f64(Ql)
    N, d = Q.shape
    m = Ql.shape[0]
    sel = None if qsel is None else np.ascontiguousarray(np.asarray(qsel, dtype=np.int64))
    nq = N if sel is None else sel.shape[0]
    r = np.empty(nq, np.int32)
    top2 = np.empty((nq, 4), np.float64) if with_top2 else None
    _check(lib().mita_oracle_route(_p(Q, _f64p), _p(Ql, _f64p), N, d, m, _p(sel, _i64p), nq,
                                   _p(r, _i32p), _p(top2, _f64p)), "route")
    return (r, top2) if with_top2 else r


def bucket(route_, m: int):
    r = _i32(route_)
    N = r.shape[0]
    offsets = np.empty(m + 1, np.int32)
    perm = np.empty(N, np.int32)
    _check(lib().mita_oracle_bucket(_p(r, _i32p), N, m, _p(offsets, _i32p), _p(perm, _i32p)),
           "bucket")
    return offsets, perm


def output(Q, K, V, Ql, Vl, idx, route_, scale: float, qsel=None) -> np.ndarray:
    Q, K, V, Ql, Vl = _f64(Q), _f64(K), _f64(V), _f64(Ql), _f64(Vl)
    idx, r = _i32(idx), _i32(route_)
    N, d = Q.shape
    m, k = idx.shape
    sel = None if qsel is None else np.ascontiguousarray(np.asarray(qsel, dtype=np.int64))
    nq = N if sel is None else sel.shape[0]
    out = np.empty((nq, d), np.float64)
    _check(lib().mita_oracle_output(_p(Q, _f64p), _p(K, _f64p), _p(V, _f64p), _p(Ql, _f64p),
                                    _p(Vl, _f64p), _p(idx, _i32p), _p(r, _i32p), N, d, m, k,
                                    float(scale), _p(sel, _i64p), nq, _p(out, _f64p)), "output")
    return out


def route_s(Q, Ql, s: int, qsel=None) -> np.ndarray:
    """[nq, s] int32: each query's s experts, best first."""
    Q, Ql = _f64(Q), _f64(Ql)
    N, d = Q.shape
    m = Ql.shape[0]
    sel = None if qsel is None else np.ascontiguousarray(np.asarray(qsel, dtype=np.int64))
    nq = N if sel is None else sel.shape[0]
    r = np.empty((nq, s), np.int32)
    _check(lib().mita_oracle_route_s(_p(Q, _f64p), _p(Ql, _f64p), N, d, m, s, _p(sel, _i64p), nq,
                                     _p(r, _i32p)), "route_s")
    return r


def bucket_s(routes, m: int):
    """offsets [m+1] and perm [N*s] over every (query, expert) assignment."""
    r = _i32(routes)
    N, s = r.shape
    offsets = np.empty(m + 1, np.int32)
    perm = np.empty(N * s, np.int32)
    _check(lib().mita_oracle_bucket_s(_p(r, _i32p), N, m, s, _p(offsets, _i32p),
                                      _p(perm, _i32p)), "bucket_s")
    return offsets, perm


def output_s(Q, K, V, Ql, Vl, idx, routes, scale: float, qsel=None) -> np.ndarray:
    Q, K, V, Ql, Vl = _f64(Q), _f64(K), _f64(V), _f64(Ql), _f64(Vl)
    idx, r = _i32(idx), _i32(routes)
    N, d = Q.shape
    m, k = idx.shape
    s = r.shape[1]
    sel = None if qsel is None else np.ascontiguousarray(np.asarray(qsel, dtype=np.int64))
    nq = N if sel is None else sel.shape[0]
    out = np.empty((nq, d), np.float64)
    _check(lib().mita_oracle_output_s(_p(Q, _f64p), _p(K, _f64p), _p(V, _f64p), _p(Ql, _f64p),
                                      _p(Vl, _f64p), _p(idx, _i32p), _p(r, _i32p), N, d, m, k,
                                      s, float(scale), _p(sel, _i64p), nq, _p(out, _f64p)),
           "output_s")
    return out


def dense(Q, K, V, scale: float, qsel=None) -> np.ndarray:
    """Dense attention over all N pairs (the pages' full-attention baseline)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    N, d = Q.shape
    sel = None if qsel is None else np.ascontiguousarray(np.asarray(qsel, dtype=np.int64))
    nq = N if sel is None else sel.shape[0]
    out = np.empty((nq, d), np.float64)
    _check(lib().mita_oracle_dense(_p(Q, _f64p), _p(K, _f64p), _p(V, _f64p), N, d, float(scale),
                                   _p(sel, _i64p), nq, _p(out, _f64p)), "dense")
    return out


def forward(Q, K, V, grid: tuple[int, int, int, int], k: int, scale: float,
            round_mode: int) -> dict:
    """All steps for [B, H, N, d] inputs; grid = (gh, gw, mh, mw)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    gh, gw, mh, mw = grid
    m = mh * mw
    res = {
        "out": np.empty((B, H, N, d), np.float64),
        "idx": np.empty((B, H, m, k), np.int32),
        "route": np.empty((B, H, N), np.int32),
        "ql": np.empty((B, H, m, d), np.float64),
        "vl": np.empty((B, H, m, d), np.float64),
        "offsets": np.empty((B, H, m + 1), np.int32),
        "perm": np.empty((B, H, N), np.int32),
    }
    _check(lib().mita_oracle_forward(
        _p(Q, _f64p), _p(K, _f64p), _p(V, _f64p), B, H, N, d, gh, gw, mh, mw, k, float(scale),
        round_mode, _p(res["out"], _f64p), _p(res["idx"], _i32p), _p(res["route"], _i32p),
        _p(res["ql"], _f64p), _p(res["vl"], _f64p), _p(res["offsets"], _i32p),
        _p(res["perm"], _i32p)), "forward")
    return res


def backward(Q, K, V, grid, k: int, scale: float, round_mode, idx, route_, dout):
    """Gradients (dQ, dK, dV) of sum(dout * out) for one head, the experts
    and routes held fixed (mita_oracle_backward)."""
    Q, K, V, dout = _f64(Q), _f64(K), _f64(V), _f64(dout)
    idx, r = _i32(idx), _i32(route_)
    N, d = Q.shape
    gh, gw, mh, mw = grid
    dQ = np.empty((N, d), np.float64)
    dK = np.empty((N, d), np.float64)
    dV = np.empty((N, d), np.float64)
    _check(lib().mita_oracle_backward(_p(Q, _f64p), _p(K, _f64p), _p(V, _f64p), N, d, gh, gw, mh,
                                      mw, k, float(scale), int(round_mode), _p(idx, _i32p),
                                      _p(r, _i32p), _p(dout, _f64p), _p(dQ, _f64p),
                                      _p(dK, _f64p), _p(dV, _f64p)), "backward")
    return dQ, dK, dV

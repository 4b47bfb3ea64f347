"""MiTA (Mixture-of-Top-k Attention) on AMD MI355X (gfx950): the forward
pass and its backward with the selections held fixed.

Thin ctypes binding over ``libmita.so`` (declared in ``include/mita.h``).
This module only marshals arguments: it checks tensor shapes, types and
devices, allocates the output tensors with torch and passes raw device
pointers and torch's current HIP stream to the C ABI.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path —
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "mita_forward",
    "mita_forward_ex",
    "mita_forward_noalloc",
    "mita_forward_s",
    "mita_dense_attention",
    "mita_backward",
    "mita_release_workspace",
    "mita_status_string",
    "mita_last_error",
    "mita_version",
    "mita_profile_enable",
    "mita_profile_read",
    "lib",
    "LIB_PATH",
    "MITA_F32",
    "MITA_BF16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmita.so")

MITA_OK = 0
MITA_ERR_INVALID_ARG = -1
MITA_ERR_UNSUPPORTED = -2
MITA_ERR_OOM = -3
MITA_ERR_HIP = -4
MITA_ERR_INTERNAL = -5
MITA_F32 = 0
MITA_BF16 = 1


class MitaGrid(ctypes.Structure):
    _fields_ = [("gh", ctypes.c_int32), ("gw", ctypes.c_int32), ("mh", ctypes.c_int32),
                ("mw", ctypes.c_int32)]


class MitaIntermediates(ctypes.Structure):
    _fields_ = [("ql", ctypes.c_void_p), ("vl", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p)]


_FWD_ARGS = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(MitaGrid),
             ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
             ctypes.c_void_p, ctypes.c_void_p]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmita.so (built by ``mixture_top_sparse_amd.build``); raises if
    it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mixture_top_sparse_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        L.mita_forward.argtypes = _FWD_ARGS
        L.mita_forward.restype = ctypes.c_int
        L.mita_forward_ex.argtypes = _FWD_ARGS + [ctypes.POINTER(MitaIntermediates)]
        L.mita_forward_ex.restype = ctypes.c_int
        L.mita_forward_noalloc.argtypes = _FWD_ARGS
        L.mita_forward_noalloc.restype = ctypes.c_int
        L.mita_forward_s.argtypes = _FWD_ARGS[:11] + [ctypes.c_int64] + _FWD_ARGS[11:]
        L.mita_forward_s.restype = ctypes.c_int
        L.mita_dense_attention.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_void_p]
        L.mita_dense_attention.restype = ctypes.c_int
        L.mita_backward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.POINTER(MitaGrid), ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.mita_backward.restype = ctypes.c_int
        L.mita_status_string.argtypes = [ctypes.c_int]
        L.mita_status_string.restype = ctypes.c_char_p
        L.mita_last_error.argtypes = []
        L.mita_last_error.restype = ctypes.c_char_p
        L.mita_version.restype = ctypes.c_int
        L.mita_profile_enable.argtypes = [ctypes.c_int]
        L.mita_profile_stage_count.restype = ctypes.c_int
        L.mita_profile_stage_name.argtypes = [ctypes.c_int]
        L.mita_profile_stage_name.restype = ctypes.c_char_p
        L.mita_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        L.mita_release_workspace.argtypes = [ctypes.c_void_p]
        L.mita_release_workspace.restype = ctypes.c_int
        _lib = L
    return _lib


def mita_status_string(status: int) -> str:
    return lib().mita_status_string(int(status)).decode()


def mita_last_error() -> str:
    return lib().mita_last_error().decode()


def mita_version() -> int:
    return int(lib().mita_version())


def _raise(rc: int, what: str) -> None:
    if rc != MITA_OK:
        raise RuntimeError(f"{what}: {mita_status_string(rc)} ({rc}): {mita_last_error()}")


def _check_inputs(Q, K, V):
    import torch

    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must have shape [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (Q.shape == K.shape == V.shape):
        raise ValueError("Q, K and V must have the same shape")
    if not (Q.dtype == K.dtype == V.dtype):
        raise ValueError("Q, K and V must have the same dtype")
    if Q.dtype == torch.bfloat16:
        dt = MITA_BF16
    elif Q.dtype == torch.float32:
        dt = MITA_F32
    else:
        raise ValueError("dtype must be torch.bfloat16 or torch.float32")
    if not (Q.device == K.device == V.device):
        raise ValueError("Q, K and V must be on the same device")
    return dt


def _call(Q, K, V, m: int, k: int, grid, scale, want_dbg: bool, noalloc: bool = False):
    import torch

    dt = _check_inputs(Q, K, V)
    B, H, N, d = Q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    dev = Q.device
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    idx = torch.empty((B, H, m, k), dtype=torch.int32, device=dev)
    route = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    g = None if grid is None else ctypes.byref(MitaGrid(*[int(x) for x in grid]))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        args = [Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N, d, g, int(m), int(k),
                float(scale), out.data_ptr(), idx.data_ptr(), route.data_ptr(), stream]
        if noalloc:
            _raise(lib().mita_forward_noalloc(*args), "mita_forward_noalloc")
            return out, idx, route
        if not want_dbg:
            _raise(lib().mita_forward(*args), "mita_forward")
            return out, idx, route
        dbg = {
            "ql": torch.empty((B, H, m, d), dtype=Q.dtype, device=dev),
            "vl": torch.empty((B, H, m, d), dtype=torch.float32, device=dev),
            "perm": torch.empty((B, H, N), dtype=torch.int32, device=dev),
            "offsets": torch.empty((B, H, m + 1), dtype=torch.int32, device=dev),
        }
        s = MitaIntermediates(dbg["ql"].data_ptr(), dbg["vl"].data_ptr(), dbg["perm"].data_ptr(),
                              dbg["offsets"].data_ptr())
        _raise(lib().mita_forward_ex(*args, ctypes.byref(s)), "mita_forward_ex")
        return out, idx, route, dbg


def mita_forward(Q, K, V, *, m: int, k: int, grid=None, scale=None):
    """MiTA forward of [B, H, N, d] tensors (bf16 or fp32, on the GPU).

    grid: (gh, gw, mh, mw) token and landmark grids (None: 1D, contiguous
    windows).  Returns (out [B,H,N,d] fp32, idx [B,H,m,k] int32 ascending,
    route [B,H,N] int32).  Enqueued on torch's current stream."""
    return _call(Q, K, V, m, k, grid, scale, want_dbg=False)


def mita_forward_ex(Q, K, V, *, m: int, k: int, grid=None, scale=None):
    """Like mita_forward, plus a dict of intermediates: ql (landmark queries),
    vl (landmark values, fp32), perm (queries grouped by expert) and offsets."""
    return _call(Q, K, V, m, k, grid, scale, want_dbg=True)


def mita_forward_noalloc(Q, K, V, *, m: int, k: int, grid=None, scale=None):
    """mita_forward without any device allocation by the library: its work
    space is the library's static 64 MiB scratch array (calls that overlap on
    one GPU race; larger problems raise).  The outputs are still allocated
    here, by torch, before the call."""
    return _call(Q, K, V, m, k, grid, scale, want_dbg=False, noalloc=True)


def mita_forward_s(Q, K, V, *, m: int, k: int, s: int, grid=None, scale=None):
    """MiTA with s experts per query (bf16 inputs for s > 1).  Returns (out
    [B,H,N,d] fp32, idx [B,H,m,k] int32, routes [B,H,N,s] int32, best first)."""
    import torch

    dt = _check_inputs(Q, K, V)
    B, H, N, d = Q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    dev = Q.device
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    idx = torch.empty((B, H, m, k), dtype=torch.int32, device=dev)
    routes = torch.empty((B, H, N, s), dtype=torch.int32, device=dev)
    g = None if grid is None else ctypes.byref(MitaGrid(*[int(x) for x in grid]))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _raise(lib().mita_forward_s(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N, d, g,
                                    int(m), int(k), int(s), float(scale), out.data_ptr(),
                                    idx.data_ptr(), routes.data_ptr(), stream),
               "mita_forward_s")
    return out, idx, routes


def mita_dense_attention(Q, K, V, *, scale=None):
    """Dense attention of [B, H, N, d] bf16 GPU tensors over all N keys (the
    full-attention baseline).  Returns out [B, H, N, d] fp32, enqueued on
    torch's current stream."""
    import torch

    dt = _check_inputs(Q, K, V)
    B, H, N, d = Q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=Q.device)
    with torch.cuda.device(Q.device):
        stream = torch.cuda.current_stream(Q.device).cuda_stream
        _raise(lib().mita_dense_attention(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N, d,
                                          float(scale), out.data_ptr(), stream),
               "mita_dense_attention")
    return out


def mita_backward(Q, K, V, idx, route, dout, *, m: int, k: int, grid=None, scale=None):
    """Gradients (dQ, dK, dV) [B,H,N,d] fp32 of sum(dout * out), out being
    mita_forward's output for the same Q, K, V, with the experts idx
    [B,H,m,k] and the routes [B,H,N] (int32) held fixed.  dout: [B,H,N,d]
    fp32.  Enqueued on torch's current stream."""
    import torch

    dt = _check_inputs(Q, K, V)
    B, H, N, d = Q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    for name, t, shape, dtype in (("idx", idx, (B, H, m, k), torch.int32),
                                  ("route", route, (B, H, N), torch.int32),
                                  ("dout", dout, (B, H, N, d), torch.float32)):
        if not isinstance(t, torch.Tensor) or t.device != Q.device:
            raise ValueError(f"{name} must be a tensor on Q's device")
        if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape}")
    dev = Q.device
    dQ = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    dK = torch.empty_like(dQ)
    dV = torch.empty_like(dQ)
    g = None if grid is None else ctypes.byref(MitaGrid(*[int(x) for x in grid]))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _raise(lib().mita_backward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt, B, H, N, d, g,
                                   int(m), int(k), float(scale), idx.data_ptr(), route.data_ptr(),
                                   dout.data_ptr(), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(),
                                   stream), "mita_backward")
    return dQ, dK, dV


def mita_release_workspace(stream=None, device=None) -> None:
    """Free the library's cached work space of a torch stream (default: the
    current stream of `device`), in that stream's order."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    with torch.cuda.device(stream.device):
        _raise(lib().mita_release_workspace(stream.cuda_stream), "mita_release_workspace")


def mita_profile_enable(enabled: bool) -> None:
    _raise(lib().mita_profile_enable(1 if enabled else 0), "mita_profile_enable")


def mita_profile_read() -> tuple[dict[str, float], int]:
    """Summed milliseconds per stage and the number of profiled calls."""
    L = lib()
    n = int(L.mita_profile_stage_count())
    ms = (ctypes.c_double * n)()
    calls = ctypes.c_int64()
    _raise(L.mita_profile_read(ms, ctypes.byref(calls), n), "mita_profile_read")
    names = [L.mita_profile_stage_name(i).decode() for i in range(n)]
    return dict(zip(names, list(ms))), int(calls.value)

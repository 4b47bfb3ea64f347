"""The no-allocation entry point (mita_forward_noalloc) through the C ABI:
two calls in a row, the second on a smaller input, each bitwise equal to
mita_forward on the same inputs (same kernels, same launch shapes; the only
difference is where the work space lives).  Device memory in use must not
grow across the no-allocation calls, and a call whose work space would
exceed the static array is rejected with nothing enqueued."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

from mixture_top_sparse_amd.inputs import WORKLOADS, generate, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _noalloc(L, mts, w, Qt, Kt, Vt):
    B, H, N, d = Qt.shape
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, w.m, w.k), dtype=torch.int32, device="cuda")
    route = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    dt = mts.MITA_BF16 if Qt.dtype == torch.bfloat16 else mts.MITA_F32
    grid = mts.MitaGrid(*w.grid)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    rc = L.mita_forward_noalloc(Qt.data_ptr(), Kt.data_ptr(), Vt.data_ptr(), dt, B, H, N, d,
                                ctypes.byref(grid), w.m, w.k, w.scale, out.data_ptr(),
                                idx.data_ptr(), route.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert rc == mts.MITA_OK, mts.mita_last_error()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return [t.cpu().numpy() for t in (out, idx, route)], free0 - free1


def test_noalloc_matches_mita_forward_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    L = mts.lib()
    large = WORKLOADS["long1d_16k"].with_(B=2, H=4)
    small = WORKLOADS["deit_s_14x14"].with_(B=4, H=3)
    cases = []
    for w in (large, small):
        cases.append((w, *to_torch(generate(w), w.dtype, "cuda")))
    refs = []
    for w, Qt, Kt, Vt in cases:
        _say(f"case reference mita_forward {w.name} B={w.B} H={w.H} N={w.N}")
        refs.append([t.cpu().numpy() for t in mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k,
                                                               grid=w.grid, scale=w.scale)])
    # a first call loads nothing new afterwards; the two checked calls follow
    w, Qt, Kt, Vt = cases[1]
    _say("case warm-up call of mita_forward_noalloc")
    _noalloc(L, mts, w, Qt, Kt, Vt)
    for (w, Qt, Kt, Vt), ref in zip(cases, refs):
        _say(f"case mita_forward_noalloc {w.name} B={w.B} H={w.H} N={w.N}")
        got, grew = _noalloc(L, mts, w, Qt, Kt, Vt)
        for name, a, b in zip(("out", "idx", "route"), got, ref):
            assert np.array_equal(a, b), f"{w.name}: {name} differs from mita_forward"
        assert grew < (1 << 20), f"device memory in use grew by {grew} bytes"


def test_noalloc_rejects_oversize_and_enqueues_nothing():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    L = mts.lib()
    B, H, N, d = 1, 2, 1 << 23, 64  # the query permutation alone fills the 64 MiB array
    # full-size buffers, so that even a launch would stay in bounds; the fill
    # values must survive because the call launches nothing
    Q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, H, N, d), 3.0, device="cuda")
    idx = torch.full((B, H, 64, 64), -7, dtype=torch.int32, device="cuda")
    route = torch.full((B, H, N), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    _say("case mita_forward_noalloc beyond the static array")
    rc = L.mita_forward_noalloc(Q.data_ptr(), Q.data_ptr(), Q.data_ptr(), mts.MITA_BF16, B, H, N,
                                d, None, 64, 64, 0.125, out.data_ptr(), idx.data_ptr(),
                                route.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == mts.MITA_ERR_UNSUPPORTED
    assert "scratch" in mts.mita_last_error()
    torch.cuda.synchronize()
    assert (out == 3.0).all().item() and (idx == -7).all().item() and (route == -7).all().item()

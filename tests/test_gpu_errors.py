"""Error paths of the C ABI on the GPU: a failed launch reports
MITA_ERR_HIP and enqueues nothing, and the library works normally after it.
The failure is forced from the host (MITA_FAULT_INJECT=launch makes the call
fail where it would launch its first kernel); no kernel ever faults."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from mixture_top_sparse_amd.inputs import WORKLOADS, generate, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-errors] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    mts.lib()


def test_injected_launch_failure_enqueues_nothing(monkeypatch):
    import ctypes

    import mixture_top_sparse_amd as mts

    w = WORKLOADS["deit_s_14x14"].with_(B=1, H=2)
    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
    B, H, N, d = Qt.shape
    _say("case injected launch failure: reference call")
    ref = [t.cpu().numpy() for t in mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid,
                                                     scale=w.scale)]
    out = torch.full((B, H, N, d), float("nan"), device="cuda")
    idx = torch.full((B, H, w.m, w.k), -7, dtype=torch.int32, device="cuda")
    route = torch.full((B, H, N), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    monkeypatch.setenv("MITA_FAULT_INJECT", "launch")
    _say("case injected launch failure: failing call")
    grid = mts.MitaGrid(*w.grid)
    rc = mts.lib().mita_forward(Qt.data_ptr(), Kt.data_ptr(), Vt.data_ptr(), mts.MITA_BF16, B, H,
                                N, d, ctypes.byref(grid), w.m, w.k, w.scale, out.data_ptr(),
                                idx.data_ptr(), route.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert rc == mts.MITA_ERR_HIP, rc
    assert "launch" in mts.mita_last_error()
    torch.cuda.synchronize()
    # nothing ran: the outputs keep their fill values
    assert torch.isnan(out).all().item()
    assert (idx == -7).all().item() and (route == -7).all().item()
    monkeypatch.delenv("MITA_FAULT_INJECT")
    _say("case injected launch failure: next call")
    got = [t.cpu().numpy() for t in mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid,
                                                     scale=w.scale)]
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)

"""GPU parity of several experts per query (s > 1): mita_forward_s through
the C ABI against the oracle's route_s / output_s, on the DeiT-S-shaped
workload in full and the 2^16-token length-scaling workload on sampled
queries; and s = 1 through mita_forward_s equal to mita_forward bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from mixture_top_sparse_amd.inputs import WORKLOADS, generate, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-multi] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    mts.lib()


@pytest.mark.parametrize("s", [2, 3])
@pytest.mark.parametrize("name", ["deit_s_14x14", "len_64k"])
def test_several_experts_per_query(name, s):
    import mixture_top_sparse_amd as mts
    from parity import Report, check_head_s

    w = WORKLOADS[name]
    _say(f"case {name} s={s} B={w.B} H={w.H} N={w.N} m={w.m} k={w.k}")
    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
    out, idx, routes = mts.mita_forward_s(Qt, Kt, Vt, m=w.m, k=w.k, s=s, grid=w.grid,
                                          scale=w.scale)
    torch.cuda.synchronize()
    out, idx, routes = out.cpu().numpy(), idx.cpu().numpy(), routes.cpu().numpy()
    exact = [t.cpu().to(torch.float64).numpy() for t in (Qt, Kt, Vt)]
    rep = Report()
    if w.N <= 4096:
        heads, qsel = [(b, h) for b in range(w.B) for h in range(w.H)], None
    else:
        heads = [(0, 0), (w.B - 1, w.H - 1)]
        rng = np.random.default_rng(17)
        qsel = np.unique(np.concatenate([np.arange(64), np.arange(w.N - 64, w.N),
                                         rng.choice(w.N, 1500, replace=False)]))
    for b, h in heads:
        g = {"out": out[b, h], "idx": idx[b, h], "routes": routes[b, h]}
        check_head_s(w, exact[0][b, h], exact[1][b, h], exact[2][b, h], g, s, rep, qsel=qsel)
    _say(f"{name} s={s}: {rep.summary()} near-tie caps (top-k, route)={rep.caps()}")
    assert rep.ok(), rep.problems()


@pytest.mark.parametrize("name", ["deit_s_14x14", "long1d_16k"])
def test_s1_is_mita_forward(name):
    import mixture_top_sparse_amd as mts

    w = WORKLOADS[name].with_(B=1, H=3)
    _say(f"case s=1 {name}")
    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
    a = mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid, scale=w.scale)
    b = mts.mita_forward_s(Qt, Kt, Vt, m=w.m, k=w.k, s=1, grid=w.grid, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[2], b[2][..., 0])

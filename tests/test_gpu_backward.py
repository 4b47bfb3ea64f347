"""GPU parity of the backward pass: mita_backward through the C ABI against
the fp64 oracle's backward (oracle.backward), both given the same experts
and routes — the ones the oracle's forward selects, or arbitrary ones — and
the same dout.

Tolerance.  The oracle computes in fp64 on the same input values (bf16
inputs are exact in both; the landmark queries are rounded to the input type
by both, bit for bit).  With fp32 inputs the GPU computes in fp32 throughout
(fp32 MFMA products and sums, the hardware exp2): each gradient element is a
sum of at most m + k + N products whose fp32 rounding errors are about 2^-24
relative to the largest of them, and the error stays below 1e-6 of each
tensor's largest element.  With bf16 inputs the expert and cross steps'
products run on bf16 MFMA with the computed operands (dout, the landmark
values and their gradient, the softmax weights and their gradients) split
into bf16 hi + lo parts: each product is then within about 2^-16 of exact,
relative, and the error measures up to 1.3e-5 of the largest element on
these cases.  The test
allows 2e-5 of that maximum (RTOL below).  It checks the same
bound separately on the keys that no expert holds (they receive only the
small cross-attention term), and the cases include windows of 3x3 tokens,
where dQ's pooling term is of the same order as the rest, so that a missing
or wrong small term cannot hide under the large ones.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle as O
from mixture_top_sparse_amd.inputs import (WORKLOADS, Workload, generate, generate_dout,
                                           generate_selection, to_torch)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RTOL = 2e-5


def _say(msg):
    print(f"[gpu-backward] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    mts.lib()


def _round_mode(w):
    return O.ROUND_BF16 if w.dtype == "bf16" else O.ROUND_F32


def _oracle_selection(w, Q, K, b, h):
    ql = O.pool(Q[b, h], *w.grid, _round_mode(w))
    return O.topk(ql, K[b, h], w.k), O.route(Q[b, h], ql)


def _rel(got, ref):
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / den if den > 0 else float(np.max(np.abs(got)))


def _check(w: Workload, selection: str, heads=None):
    import mixture_top_sparse_amd as mts

    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
    dout = torch.from_numpy(generate_dout(w)).cuda()
    Q, K, V = (t.cpu().to(torch.float64).numpy() for t in (Qt, Kt, Vt))
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    if selection == "oracle":
        idx = np.zeros((w.B, w.H, w.m, w.k), np.int32)
        routes = np.zeros((w.B, w.H, w.N), np.int32)
        for b in range(w.B):
            for h in range(w.H):
                if (b, h) in heads or w.B * w.H <= 4:
                    idx[b, h], routes[b, h] = _oracle_selection(w, Q, K, b, h)
    else:
        idx, routes = generate_selection(w, seed=77 + w.seed)
    _say(f"case {w.name} {w.dtype} B={w.B} H={w.H} N={w.N} m={w.m} k={w.k} grid={w.grid} "
         f"selection={selection}")
    dQ, dK, dV = mts.mita_backward(Qt, Kt, Vt, torch.from_numpy(idx).cuda(),
                                   torch.from_numpy(routes).cuda(), dout, m=w.m, k=w.k,
                                   grid=w.grid, scale=w.scale)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in (dQ, dK, dV)]
    G = dout.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b, h in heads:
        ref = O.backward(Q[b, h], K[b, h], V[b, h], w.grid, w.k, w.scale, _round_mode(w),
                         idx[b, h], routes[b, h], G[b, h])
        errs = {}
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            errs[name] = _rel(g[b, h], r)
        held = np.zeros(w.N, bool)
        held[idx[b, h].ravel()] = True
        if not held.all():  # keys only the landmarks see
            for name, g, r in (("dK_free", got[1], ref[1]), ("dV_free", got[2], ref[2])):
                errs[name] = _rel(g[b, h][~held], r[~held])
        worst = max(worst, *errs.values())
        _say(f"  head ({b},{h}): " + " ".join(f"{k_}={v:.2e}" for k_, v in errs.items()))
        bad = {k_: v for k_, v in errs.items() if not v <= RTOL}
        assert not bad, f"{w.name} head ({b},{h}) {selection}: relative errors {bad} > {RTOL}"
    return worst


CASES = [
    WORKLOADS["tiny_f32_14x14"].with_(H=2),
    WORKLOADS["deit_s_14x14"].with_(B=2, H=2),
    Workload("ragged_1d_1000", 1, 2, 1000, 64, "bf16", (1, 1000, 1, 16), 20, "mixture", 32, 0.5,
             seed=21),
    WORKLOADS["seg_40x40"].with_(B=1, H=2),
    WORKLOADS["long1d_16k"].with_(B=1, H=2, N=4096, grid=(1, 4096, 1, 64)),
    Workload("f32_1d_3000", 1, 1, 3000, 64, "f32", (1, 3000, 1, 48), 33, "mixture", 64, 0.5,
             seed=22),
    # bf16 with 40 landmarks: three 16-landmark blocks in the cross step and
    # five 16-pair blocks in the expert step (the odd tails of their bf16
    # MFMA loops)
    Workload("bf16_1d_2000_m40", 1, 2, 2000, 64, "bf16", (1, 2000, 1, 40), 24, "mixture", 64,
             0.5, seed=23),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_with_the_methods_selection(w):
    _check(w, "oracle")


@pytest.mark.parametrize("w", [CASES[1], CASES[2], CASES[4]], ids=lambda w: w.name)
def test_backward_with_arbitrary_selection(w):
    # keys repeated across experts, uneven and empty experts
    _check(w, "random")


def test_backward_one_expert_takes_every_query():
    import mixture_top_sparse_amd as mts

    w = Workload("one_expert", 1, 1, 2048, 64, "bf16", (1, 2048, 1, 32), 32, "mixture", 16, 0.5,
                 seed=23)
    _say(f"case {w.name}: all routes to expert 5")
    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
    dout = torch.from_numpy(generate_dout(w)).cuda()
    Q, K, V = (t.cpu().to(torch.float64).numpy() for t in (Qt, Kt, Vt))
    idx, _ = _oracle_selection(w, Q, K, 0, 0)
    routes = np.full(w.N, 5, np.int32)
    dQ, dK, dV = mts.mita_backward(Qt, Kt, Vt, torch.from_numpy(idx[None, None]).cuda(),
                                   torch.from_numpy(routes[None, None]).cuda(), dout, m=w.m,
                                   k=w.k, grid=w.grid, scale=w.scale)
    torch.cuda.synchronize()
    ref = O.backward(Q[0, 0], K[0, 0], V[0, 0], w.grid, w.k, w.scale, O.ROUND_BF16, idx, routes,
                     dout.cpu().numpy()[0, 0].astype(np.float64))
    for name, g, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        e = _rel(g[0, 0].cpu().numpy().astype(np.float64), r)
        _say(f"  {name} {e:.2e}")
        assert e <= RTOL, (name, e)


def test_backward_full_size_sampled_heads():
    """The 16K-token 1D workload at its full batch (B=4, H=8) in one call;
    the oracle checks the first and the last head."""
    w = WORKLOADS["long1d_16k"]
    _check(w, "oracle", heads=[(0, 0), (w.B - 1, w.H - 1)])


def test_backward_repeatable_dq():
    """dQ has no atomics: two calls give identical bits.  dK and dV (fp32
    atomic adds of the expert step) agree to rounding."""
    import mixture_top_sparse_amd as mts

    w = CASES[4]
    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
    dout = torch.from_numpy(generate_dout(w)).cuda()
    idx, routes = generate_selection(w, seed=5)
    a = mts.mita_backward(Qt, Kt, Vt, torch.from_numpy(idx).cuda(),
                          torch.from_numpy(routes).cuda(), dout, m=w.m, k=w.k, grid=w.grid)
    b = mts.mita_backward(Qt, Kt, Vt, torch.from_numpy(idx).cuda(),
                          torch.from_numpy(routes).cuda(), dout, m=w.m, k=w.k, grid=w.grid)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    for x, y in zip(a[1:], b[1:]):
        assert float((x - y).abs().max()) <= 1e-6 * float(x.abs().max())

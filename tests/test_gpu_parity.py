"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test prints the case it is about to run before touching the GPU."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from mixture_top_sparse_amd.inputs import WORKLOADS, Workload, generate, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    mts.lib()  # fail loudly if the library is missing


def _run(w: Workload, Q, K, V):
    import mixture_top_sparse_amd as mts
    from parity import gpu_results_to_numpy

    Qt, Kt, Vt = to_torch((Q, K, V), w.dtype, "cuda")
    res = mts.mita_forward_ex(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid, scale=w.scale)
    g = gpu_results_to_numpy(res)
    exact = [t.to("cpu").to(torch.float64).numpy() for t in (Qt, Kt, Vt)]
    return g, exact


def _check(w, g, exact, heads=None, qsel=None, exact_ties=False):
    from parity import Report, check_head

    rep = Report()
    Qd, Kd, Vd = exact
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in pairs:
        gh = {key: val[b, h] for key, val in g.items()}
        check_head(w, Qd[b, h], Kd[b, h], Vd[b, h], gh, rep, qsel=qsel, exact_ties=exact_ties)
    _say(f"{w.name}: {rep.summary()} near-tie caps (top-k, route)={rep.caps()}")
    assert rep.ok(), rep.problems()
    return rep


# ---------------------------------------------------------------------------
# the workloads: whole outputs where the oracle is quick, samples at full size
# ---------------------------------------------------------------------------

FULL = ["tiny_f32_14x14", "deit_s_14x14", "seg_40x40", "seg_32x32", "long1d_16k"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full(name):
    w = WORKLOADS[name]
    _say(f"case {name} B={w.B} H={w.H} N={w.N} m={w.m} k={w.k} {w.dtype}")
    Q, K, V = generate(w)
    g, exact = _run(w, Q, K, V)
    heads = None
    if name == "long1d_16k":
        heads = [(0, 0), (1, 3), (3, 7)]
    _check(w, g, exact, heads=heads)


SAMPLED = ["long1d_32k", "long1d_64k", "len_64k", "len_256k", "len_1m"]


@pytest.mark.parametrize("name", SAMPLED)
def test_workload_sampled(name):
    w = WORKLOADS[name]
    _say(f"case {name} B={w.B} H={w.H} N={w.N} m={w.m} k={w.k} {w.dtype} (sampled)")
    Q, K, V = generate(w)
    g, exact = _run(w, Q, K, V)
    rng = np.random.default_rng(123)
    qsel = np.unique(np.concatenate([np.arange(64), np.arange(w.N - 64, w.N),
                                     rng.choice(w.N, 1500, replace=False)]))
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    _check(w, g, exact, heads=heads, qsel=qsel)


@pytest.mark.parametrize("name", ["deit_s_14x14", "len_64k"])
def test_values_scaled_by_8(name):
    """Values 8x larger (a power of two, so bf16 rounding commutes with it):
    the attention's P.V error bound scales with max|V|, and the hi + lo
    operands must keep it inside the 5e-3 tolerance at max|V| near 45."""
    w = WORKLOADS[name]
    _say(f"case {name} with V scaled by 8")
    Q, K, V = generate(w)
    g, exact = _run(w, Q, K, 8.0 * V)
    assert np.abs(exact[2]).max() > 30.0
    if w.N <= 4096:
        rep = _check(w, g, exact)
    else:
        rng = np.random.default_rng(5)
        qsel = np.unique(np.concatenate([np.arange(64), rng.choice(w.N, 2000, replace=False)]))
        rep = _check(w, g, exact, heads=[(0, 0), (w.B - 1, w.H - 1)], qsel=qsel)
    _say(f"{name} x8: out_max_err={rep.out_max_err:.3e}")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------


def _edge(name, B, H, N, grid, k, dtype="bf16", values="iid", seed=100, centres=0):
    return Workload(name, B, H, N, 64, dtype, grid, k, values, centres, 0.5 if centres else 0.0,
                    seed)


EDGES = {
    # N not a multiple of the 64-key tile, m does not divide N (overlapping
    # adaptive 1D windows), k not a multiple of 16
    "ragged_1d": _edge("ragged_1d", 2, 2, 1000, (1, 1000, 1, 10), 7),
    "single_landmark_k1": _edge("single_landmark_k1", 1, 2, 300, (1, 300, 1, 1), 1),
    "k_equals_n": _edge("k_equals_n", 1, 1, 48, (1, 48, 1, 3), 48),
    "m_equals_n": _edge("m_equals_n", 1, 1, 64, (8, 8, 8, 8), 64),
    "grid_12x20": _edge("grid_12x20", 2, 1, 240, (12, 20, 3, 5), 33, values="mixture", centres=16),
    "f32_ragged": _edge("f32_ragged", 1, 3, 777, (1, 777, 1, 40), 50, dtype="f32"),
    "m17_k63": _edge("m17_k63", 1, 2, 5000, (1, 5000, 1, 17), 63, values="mixture", centres=32),
    # the multi-launch path with short work items (64 queries per expert on
    # average) assigned to the attention's blocks by size
    "short_items_2048": _edge("short_items_2048", 2, 2, 2048, (1, 2048, 1, 32), 24,
                              values="mixture", centres=16),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_edge_case(name):
    w = EDGES[name]
    _say(f"case {name} B={w.B} H={w.H} N={w.N} grid={w.grid} k={w.k} {w.dtype}")
    Q, K, V = generate(w)
    g, exact = _run(w, Q, K, V)
    _check(w, g, exact)


# each pre-threshold path of the top-k scan at least once per input type:
# sampled tiles (from 32K keys), 16-key groups (4097-32767 keys), every key
# (up to 4096 keys, the edge cases above)
THRESHOLD_PATHS = {
    "f32_sampled_40000": _edge("f32_sampled_40000", 1, 2, 40000, (1, 40000, 1, 37), 5,
                               dtype="f32", values="mixture", centres=64),
    "f32_groups16_6000": _edge("f32_groups16_6000", 2, 1, 6000, (1, 6000, 1, 20), 40,
                               dtype="f32"),
    "bf16_sampled_k3_50001": _edge("bf16_sampled_k3_50001", 1, 2, 50001, (1, 50001, 1, 37), 3,
                                   values="mixture", centres=128),
}


@pytest.mark.parametrize("name", sorted(THRESHOLD_PATHS))
def test_threshold_paths(name):
    w = THRESHOLD_PATHS[name]
    _say(f"case {name} B={w.B} H={w.H} N={w.N} m={w.m} k={w.k} {w.dtype}")
    Q, K, V = generate(w)
    g, exact = _run(w, Q, K, V)
    rng = np.random.default_rng(321)
    qsel = np.unique(np.concatenate([np.arange(64), np.arange(w.N - 64, w.N),
                                     rng.choice(w.N, 1000, replace=False)]))
    _check(w, g, exact, qsel=qsel)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_ties_resolve_to_lowest_index(dtype):
    """Small-integer inputs: every dot product is exact in fp32 and fp64, so
    equal scores are true ties on both sides and must resolve to the lower
    key (top-k) and the lower landmark (routing) exactly."""
    w = _edge(f"ties_{dtype}", 1, 2, 640, (1, 640, 1, 16), 20, dtype=dtype)
    rng = np.random.default_rng(7)
    Q = rng.integers(-2, 3, size=(1, 2, 640, 64)).astype(np.float32)
    K = rng.integers(-1, 2, size=(1, 2, 640, 64)).astype(np.float32)
    V = rng.integers(-3, 4, size=(1, 2, 640, 64)).astype(np.float32)
    K[:, :, 100:110] = K[:, :, 5:15]  # duplicated keys: equal scores at different indices
    # windows of 40 tokens: make the landmark means exact small values
    Q[:, :, :, :] = np.repeat(Q[:, :, ::40, :], 40, axis=2)
    _say(f"case exact ties {dtype}")
    g, exact = _run(w, Q, K, V)
    _check(w, g, exact, exact_ties=True)


def test_all_queries_one_expert():
    """Constant queries: every landmark is the same vector, every routing
    logit ties, so all N queries go to expert 0 (many tiles of one expert,
    m-1 empty experts)."""
    w = _edge("one_expert", 1, 1, 4000, (1, 4000, 1, 8), 16)
    rng = np.random.default_rng(8)
    Q = np.full((1, 1, 4000, 64), 0.5, np.float32)
    K = rng.standard_normal((1, 1, 4000, 64)).astype(np.float32)
    V = rng.standard_normal((1, 1, 4000, 64)).astype(np.float32)
    _say("case all queries to one expert")
    g, exact = _run(w, Q, K, V)
    assert np.all(g["route"] == 0)
    assert g["offsets"][0, 0].tolist() == [0] + [4000] * 8
    _check(w, g, exact, exact_ties=False)


def test_deterministic():
    """Two runs give bitwise-identical results (no races in merges or scatter)."""
    w = WORKLOADS["len_64k"]
    _say("case determinism len_64k")
    Q, K, V = generate(w)
    g1, _ = _run(w, Q, K, V)
    g2, _ = _run(w, Q, K, V)
    for key in g1:
        assert np.array_equal(g1[key], g2[key]), key


def test_streams_and_workspace_growth():
    """Calls on two streams at once, and a stream whose cached work space
    must grow and then serves a smaller call again, give the bitwise results
    of the same calls made one at a time on the default stream."""
    import mixture_top_sparse_amd as mts

    small = WORKLOADS["seg_32x32"].with_(B=2, H=2)
    large = WORKLOADS["long1d_16k"].with_(B=1, H=2)
    cases = []
    for w in (small, large):
        Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")
        cases.append((w, Qt, Kt, Vt))

    def fwd(c):
        w, Qt, Kt, Vt = c
        return mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid, scale=w.scale)

    def host(res):
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in res]

    _say("case streams: references on the default stream")
    ref = [host(fwd(c)) for c in cases]

    _say("case streams: small and large on two streams at once")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        r1 = fwd(cases[0])
    with torch.cuda.stream(s2):
        r2 = fwd(cases[1])
    for got, want in ((host(r1), ref[0]), (host(r2), ref[1])):
        for a, b in zip(got, want):
            assert np.array_equal(a, b)

    _say("case streams: small, large, small on a fresh stream (work space grows)")
    s3 = torch.cuda.Stream()
    with torch.cuda.stream(s3):
        seq = [fwd(cases[0]), fwd(cases[1]), fwd(cases[0])]
    for got, want in zip([host(r) for r in seq], [ref[0], ref[1], ref[0]]):
        for a, b in zip(got, want):
            assert np.array_equal(a, b)


def test_workspace_eviction_and_release():
    """Ten streams (two more than the library caches blocks for, so later
    calls take over least recently used blocks), then early release of some
    streams' blocks and calls on them again: every result is bitwise the
    result of the same call on the default stream."""
    import mixture_top_sparse_amd as mts

    w = WORKLOADS["seg_32x32"].with_(B=2, H=2)
    Qt, Kt, Vt = to_torch(generate(w), w.dtype, "cuda")

    def fwd():
        return mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid, scale=w.scale)

    def host(res):
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in res]

    _say("case eviction: reference on the default stream")
    ref = host(fwd())
    streams = [torch.cuda.Stream() for _ in range(10)]
    assert len({s.cuda_stream for s in streams}) == 10
    for rnd in range(2):
        _say(f"case eviction: round {rnd}, one call on each of 10 streams")
        got = []
        for s in streams:
            with torch.cuda.stream(s):
                got.append(fwd())
        for r in got:
            for a, b in zip(host(r), ref):
                assert np.array_equal(a, b)
    _say("case eviction: release three streams' blocks, call again")
    for s in streams[:3]:
        mts.mita_release_workspace(s)
        mts.mita_release_workspace(s)  # nothing cached any more: not an error
    got = []
    for s in streams[:4]:
        with torch.cuda.stream(s):
            got.append(fwd())
    for r in got:
        for a, b in zip(host(r), ref):
            assert np.array_equal(a, b)
    for s in streams:
        mts.mita_release_workspace(s)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_golden_pair_count_closed_form(dtype):
    """The pages' count at m = k = 25 (tests/golden/pair_count_m25_k25.json:
    25 compressed + 25 raw pairs) on the GPU path, independent of the oracle.
    With Q = 0 every logit ties: every query goes to landmark 0, every expert
    holds keys 0..k-1 (ties to the lower index), V_l is the mean of V, and
    every output row is (m * mean(V) + sum of V[0..k-1]) / total_pairs."""
    import json
    import os

    from parity import TOL

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "pair_count_m25_k25.json")))
    gh, gw, mh, mw = g["grid"]
    m, k, N = g["m"], g["k"], gh * gw
    w = _edge(f"golden_pairs_{dtype}", 1, 2, N, tuple(g["grid"]), k, dtype=dtype)
    rng = np.random.default_rng(11)
    Q = np.zeros((1, 2, N, 64), np.float32)
    K = rng.standard_normal((1, 2, N, 64)).astype(np.float32)
    V = rng.standard_normal((1, 2, N, 64)).astype(np.float32)
    _say(f"case golden pair count m={m} k={k} {dtype}")
    res, exact = _run(w, Q, K, V)
    Vd = exact[2]
    assert np.all(res["route"] == 0)
    assert np.array_equal(res["idx"], np.broadcast_to(np.arange(k, dtype=np.int32),
                                                      res["idx"].shape))
    for h in range(2):
        want = (g["compressed_pairs"] * Vd[0, h].mean(0) + Vd[0, h, :g["raw_pairs"]].sum(0)) \
            / g["total_pairs"]
        err = np.abs(res["out"][0, h] - want[None, :]).max()
        assert err <= TOL[dtype], err

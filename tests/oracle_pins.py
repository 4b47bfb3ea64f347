"""Pins for the fp64 oracle: each check compares the oracle with something
other than itself — a library routine, a closed form, an invariant of the
definition, or brute force on inputs whose dot products are exact.

Each ``check_*`` raises AssertionError on failure.  They are collected as
tests by ``test_oracle_pins.py`` and re-run against deliberately broken
builds of the oracle by ``test_oracle_mutants.py`` (which asserts that every
planted mistake trips at least one of them).

Where a pin follows a statement of the pages it names the page and section:
  [P1] "NeurIPS'26：注意力也是FFN？…", section "用少量地标查询，同时构造全局概括与细节专家"
  [P2] "NeurIPS 2026 | Mixture-of-Top-k 注意力…", section "MiTA：用少量地标查询，同时完成压缩与专家构造"
  [P3] "And attention is also FFN? …", Figure 3 and Algorithm 1
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

import oracle as O

# ---------------------------------------------------------------------------
# helpers (no MiTA arithmetic: only data construction)
# ---------------------------------------------------------------------------


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _int_data(rng, shape, lo=-3, hi=3):
    """Small integers: every dot product of such vectors is exact in fp64 in
    any summation order, so equal scores are real ties."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def _bf16_bits(x: float) -> int:
    f = np.array([x], dtype=np.float32)
    u = int(f.view(np.uint32)[0])
    assert float(f[0]) == x, "result is not an fp32 value"
    assert u & 0xFFFF == 0, "result has more than 8 significant bits"
    return u >> 16


def _bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


# ---------------------------------------------------------------------------
# rounding into bfloat16 (the landmark queries are stored in the input type)
# ---------------------------------------------------------------------------


def check_round_bf16_definition():
    """Round-to-nearest, ties-to-even into bf16, checked against the IEEE
    definition with exact rational arithmetic: the result is a bf16 value and
    no neighbouring bf16 value is closer (on a tie the result is even)."""
    rng = _rng(11)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000)))
    # exact midpoints between neighbouring bf16 values, and points just off them
    for b in rng.integers(0x3C00, 0x4400, 300):
        lo, hi = _bf16_value(int(b)), _bf16_value(int(b) + 1)
        mid = (lo + hi) / 2
        xs += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), -mid]
    for x in xs:
        r = O.round_bf16(float(x))
        bits = _bf16_bits(r)
        dist = abs(Fraction(x) - Fraction(r))
        for nb in (bits - 1, bits + 1):
            if (nb & 0x7F80) == 0x7F80:  # infinities / NaN are not neighbours
                continue
            dn = abs(Fraction(x) - Fraction(_bf16_value(nb)))
            assert dist <= dn, (x, r)
            if dist == dn:
                assert bits % 2 == 0, ("tie not to even", x, r)


def check_round_bf16_cases():
    """Hand-derived cases.  1 + 2^-8 lies halfway between the bf16 values 1
    and 1 + 2^-7, so ties-to-even gives 1; 1 + 3*2^-8 lies halfway between
    1 + 2^-7 and 1 + 2^-6 and goes to the even 1 + 2^-6.  1 + 2^-8 + 2^-40
    is above the midpoint and must round up to 1 + 2^-7 — rounding first to
    fp32 would drop the 2^-40 and then tie down to 1 (double rounding)."""
    assert O.round_bf16(1 + 2.0**-8) == 1.0
    assert O.round_bf16(1 + 3 * 2.0**-8) == 1 + 2.0**-6
    assert O.round_bf16(1 + 2.0**-8 + 2.0**-40) == 1 + 2.0**-7
    assert O.round_bf16(-(1 + 2.0**-8 + 2.0**-40)) == -(1 + 2.0**-7)
    assert O.round_bf16(2.0**-133) == 2.0**-133  # smallest subnormal
    assert O.round_bf16(2.0**-135) == 0.0  # below half of it
    assert O.round_bf16(3 * 2.0**-135) == 2.0**-133  # above half of it
    assert O.round_bf16(2.0**128) == float("inf")


# ---------------------------------------------------------------------------
# step 1: landmark queries by local average pooling [P1][P2]
# ---------------------------------------------------------------------------


def check_pool_bins_14_to_5():
    """Adaptive bins of a 14-token side into 5: start = floor(i*14/5),
    end = ceil((i+1)*14/5): 0..3, 2..6, 5..9, 8..12, 11..14 (they overlap)."""
    want = [(0, 3), (2, 6), (5, 9), (8, 12), (11, 14)]
    for a in range(5):
        for c in range(5):
            r0, r1, c0, c1 = O.window(14, 14, 5, 5, a * 5 + c)
            assert (r0, r1) == want[a] and (c0, c1) == want[c]
    # 1D: gh = mh = 1; windows of N/m tokens when m divides N
    for i in range(64):
        assert O.window(1, 4096, 1, 64, i) == (0, 1, 64 * i, 64 * (i + 1))


def check_pool_vs_adaptive_avg_pool():
    """Before rounding, the pooled landmarks equal torch's adaptive average
    pooling in fp64 (a library routine with the same bin rule)."""
    rng = _rng(12)
    for gh, gw, mh, mw in [(14, 14, 5, 5), (40, 40, 7, 7), (32, 32, 7, 7), (9, 13, 4, 3),
                           (1, 100, 1, 7), (1, 4096, 1, 64)]:
        N, d = gh * gw, 8
        Q = rng.standard_normal((N, d))
        got = O.pool(Q, gh, gw, mh, mw, O.ROUND_NONE)
        img = torch.from_numpy(Q.T.reshape(d, gh, gw).copy())
        ref = F.adaptive_avg_pool2d(img, (mh, mw)).reshape(d, mh * mw).T.numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def check_pool_special_cases():
    rng = _rng(13)
    # constant tokens give constant landmarks
    Q = np.full((196, 4), 0.75)
    assert np.all(O.pool(Q, 14, 14, 5, 5) == 0.75)
    # one landmark per token: identity
    Q = rng.standard_normal((12, 5))
    assert np.array_equal(O.pool(Q, 3, 4, 3, 4), Q)
    # a single landmark: the global mean
    Q = rng.standard_normal((60, 6))
    np.testing.assert_allclose(O.pool(Q, 6, 10, 1, 1)[0], Q.mean(0), rtol=1e-13, atol=1e-15)
    # 1D windows of N/m contiguous tokens
    Q = rng.standard_normal((512, 3))
    np.testing.assert_allclose(O.pool(Q, 1, 512, 1, 16), Q.reshape(16, 32, 3).mean(1),
                               rtol=1e-13, atol=1e-15)


def check_pool_rounding_modes():
    """Rounded landmarks are exactly representable in the target type and are
    the nearest such value to the fp64 mean."""
    rng = _rng(14)
    Qf = torch.randn(196, 16, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    Q = Qf.to(torch.float64).numpy()
    exact = O.pool(Q, 14, 14, 5, 5, O.ROUND_NONE)
    rb = O.pool(Q, 14, 14, 5, 5, O.ROUND_BF16)
    assert np.array_equal(torch.from_numpy(rb).to(torch.bfloat16).to(torch.float64).numpy(), rb)
    for x, r in zip(exact.ravel()[:200], rb.ravel()[:200]):
        bits = _bf16_bits(float(r))
        for nb in (bits - 1, bits + 1):
            assert abs(Fraction(float(x)) - Fraction(float(r))) <= abs(
                Fraction(float(x)) - Fraction(_bf16_value(nb)))
    Q = rng.standard_normal((196, 16)).astype(np.float32).astype(np.float64)
    r32 = O.pool(Q, 14, 14, 5, 5, O.ROUND_F32)
    e64 = O.pool(Q, 14, 14, 5, 5, O.ROUND_NONE)
    assert np.array_equal(r32, e64.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# step 2a: routed experts = per-landmark top-k keys [P1][P2]
# ---------------------------------------------------------------------------


def _bruteforce_topk(S, k):
    """Full sort of every row by (larger score, then lower index)."""
    m, N = S.shape
    out = np.empty((m, k), np.int64)
    for i in range(m):
        order = np.lexsort((np.arange(N), -S[i]))  # last key is primary
        out[i] = np.sort(order[:k])
    return out


def check_topk_bruteforce_with_ties():
    rng = _rng(21)
    for N, d, m, k in [(37, 4, 5, 6), (64, 8, 3, 64), (100, 3, 7, 1), (23, 2, 4, 11)]:
        Ql = _int_data(rng, (m, d))
        K = _int_data(rng, (N, d))
        got = O.topk(Ql, K, k)
        S = Ql @ K.T  # exact: small integers
        assert np.array_equal(got, _bruteforce_topk(S, k)), (N, d, m, k)
        assert np.all(np.diff(got, axis=1) > 0)  # ascending, distinct


def check_topk_gaussian_vs_torch():
    rng = _rng(22)
    Ql = rng.standard_normal((9, 16))
    K = rng.standard_normal((300, 16))
    got = O.topk(Ql, K, 17)
    ref = torch.topk(torch.from_numpy(Ql @ K.T), 17, dim=1).indices.numpy()
    for i in range(9):
        assert set(got[i].tolist()) == set(ref[i].tolist())


def check_topk_k_equals_n_and_duplicates():
    rng = _rng(23)
    Ql = rng.standard_normal((4, 8))
    K = rng.standard_normal((50, 8))
    assert np.array_equal(O.topk(Ql, K, 50), np.tile(np.arange(50), (4, 1)))
    # two identical key rows that beat every other key: with k = 1 the lower
    # index wins
    K[17] = K[31] = 10.0 * Ql[0]
    got = O.topk(Ql[:1], K, 1)
    assert got[0, 0] == 17
    got = O.topk(Ql[:1], K, 2)
    assert got[0].tolist() == [17, 31]


def check_topk_permutation_equivariance():
    rng = _rng(24)
    Ql = rng.standard_normal((6, 8))
    K = rng.standard_normal((120, 8))
    p = rng.permutation(120)
    a = O.topk(Ql, K, 13)
    b = O.topk(Ql, K[p], 13)
    for i in range(6):
        assert set(p[b[i]].tolist()) == set(a[i].tolist())


def _abs_product_sum(a, b):
    """Sum over coordinates of |a_j * b_j|, written out term by term."""
    return float(sum(abs(float(x) * float(y)) for x, y in zip(a, b)))


def check_topk_gap_report():
    """The near-tie report of the top-k step: the k-th and (k+1)-th scores in
    the order (larger score, then lower key) and, for those two keys, the sum
    of |products| of their dot products (the bound the comparison protocol
    scales its fp32 band by).  Computed here from a lexicographic sort and
    term-by-term sums; integer data make some scores tie exactly, so the tie
    rule decides which key sits at each of the two places."""
    rng = _rng(25)
    cases = [(rng.standard_normal((5, 8)), rng.standard_normal((90, 8)), 10),
             (_int_data(rng, (7, 6), -2, 2), _int_data(rng, (80, 6), -2, 2), 13),
             (_int_data(rng, (4, 5), -1, 1), _int_data(rng, (40, 5), -3, 3), 1)]
    for Ql, K, k in cases:
        _, gap = O.topk(Ql, K, k, with_gap=True)
        S = Ql @ K.T
        for i in range(Ql.shape[0]):
            order = np.lexsort((np.arange(K.shape[0]), -S[i]))  # score desc, index asc
            tk, tn = order[k - 1], order[k]
            assert np.isclose(gap[i, 0], S[i, tk], rtol=1e-12, atol=1e-12)
            assert np.isclose(gap[i, 1], S[i, tn], rtol=1e-12, atol=1e-12)
            assert np.isclose(gap[i, 2], _abs_product_sum(Ql[i], K[tk]), rtol=1e-13, atol=0)
            assert np.isclose(gap[i, 3], _abs_product_sum(Ql[i], K[tn]), rtol=1e-13, atol=0)
            assert gap[i, 2] >= abs(gap[i, 0]) and gap[i, 3] >= abs(gap[i, 1])
    # k = N: no (k+1)-th key, so no near-tie is possible
    Ql, K = rng.standard_normal((3, 4)), rng.standard_normal((12, 4))
    _, gap = O.topk(Ql, K, 12, with_gap=True)
    S = Ql @ K.T
    assert np.all(gap[:, 1] == -np.inf) and np.all(gap[:, 3] == 0.0)
    for i in range(3):
        last = np.lexsort((np.arange(12), -S[i]))[11]
        assert np.isclose(gap[i, 2], _abs_product_sum(Ql[i], K[last]), rtol=1e-13, atol=0)


# ---------------------------------------------------------------------------
# step 2b: landmark values = cross-attention of landmarks over all keys [P1][P2]
# ---------------------------------------------------------------------------


def check_landmark_values_vs_torch_softmax():
    rng = _rng(31)
    for N, d, m, scale in [(196, 16, 25, 0.25), (1000, 8, 3, 1.0), (7, 4, 2, 0.125)]:
        Ql = rng.standard_normal((m, d))
        K = rng.standard_normal((N, d))
        V = rng.standard_normal((N, d))
        got = O.landmark_values(Ql, K, V, scale)
        A = torch.softmax(torch.from_numpy(scale * (Ql @ K.T)), dim=-1)
        ref = (A @ torch.from_numpy(V)).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def check_landmark_values_invariants():
    rng = _rng(32)
    N, d, m = 150, 8, 6
    Ql = rng.standard_normal((m, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    Vl = O.landmark_values(Ql, K, V, 0.3)
    # convex combination of value rows
    assert np.all(Vl <= V.max(0) + 1e-12) and np.all(Vl >= V.min(0) - 1e-12)
    # equal keys: uniform weights, the mean value
    Ke = np.tile(K[:1], (N, 1))
    np.testing.assert_allclose(O.landmark_values(Ql, Ke, V, 0.3), np.tile(V.mean(0), (m, 1)),
                               rtol=1e-12, atol=1e-13)
    # weights sum to one: affine maps of V carry through
    c = rng.standard_normal(d)
    np.testing.assert_allclose(O.landmark_values(Ql, K, 2.5 * V + c, 0.3), 2.5 * Vl + c,
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# step 3: routing to the best-matching landmark [P1][P2]
# ---------------------------------------------------------------------------


def check_route_vs_argmax_with_ties():
    rng = _rng(41)
    Q = _int_data(rng, (400, 4), -2, 2)
    Ql = _int_data(rng, (9, 4), -1, 1)
    got = O.route(Q, Ql)
    ref = np.argmax(Q @ Ql.T, axis=1)  # first occurrence of the maximum
    assert np.array_equal(got, ref)
    # a single landmark takes every query
    assert np.all(O.route(Q, Ql[:1]) == 0)
    # routing a subset gives the same answers
    sel = rng.choice(400, 37, replace=False)
    assert np.array_equal(O.route(Q, Ql, qsel=sel), ref[sel])


def check_route_top2_report():
    """The near-tie report of routing: the best and second-best logits (each
    the first occurrence in landmark order, the best one excluded from the
    search for the second) and the sums of |products| of those two dot
    products, from an independent sort and term-by-term sums."""
    rng = _rng(42)
    cases = [(rng.standard_normal((50, 8)), rng.standard_normal((6, 8))),
             (_int_data(rng, (120, 4), -2, 2), _int_data(rng, (9, 4), -1, 1))]
    for Q, Ql in cases:
        sel = np.arange(Q.shape[0])[::3]
        for qsel in (None, sel):
            r, top2 = O.route(Q, Ql, qsel=qsel, with_top2=True)
            qs = np.arange(Q.shape[0]) if qsel is None else sel
            R = Q[qs] @ Ql.T
            for p, q in enumerate(qs):
                order = np.lexsort((np.arange(Ql.shape[0]), -R[p]))
                best, second = order[0], order[1]
                assert r[p] == best
                assert np.isclose(top2[p, 0], R[p, best], rtol=1e-12, atol=1e-12)
                assert np.isclose(top2[p, 1], R[p, second], rtol=1e-12, atol=1e-12)
                assert np.isclose(top2[p, 2], _abs_product_sum(Q[q], Ql[best]), rtol=1e-13,
                                  atol=0)
                assert np.isclose(top2[p, 3], _abs_product_sum(Q[q], Ql[second]), rtol=1e-13,
                                  atol=0)
    # a single landmark: no runner-up
    Q, Ql = rng.standard_normal((10, 4)), rng.standard_normal((1, 4))
    r, top2 = O.route(Q, Ql, with_top2=True)
    assert np.all(r == 0) and np.all(top2[:, 1] == -np.inf) and np.all(top2[:, 3] == 0.0)
    for q in range(10):
        assert np.isclose(top2[q, 2], _abs_product_sum(Q[q], Ql[0]), rtol=1e-13, atol=0)


# ---------------------------------------------------------------------------
# step 4: grouping queries by expert [P1][P2]
# ---------------------------------------------------------------------------


def check_bucket_vs_stable_argsort():
    rng = _rng(51)
    for N, m in [(1000, 7), (5, 9), (64, 1)]:
        r = rng.integers(0, m, N).astype(np.int32)
        off, perm = O.bucket(r, m)
        assert np.array_equal(perm, np.argsort(r, kind="stable"))
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(r, minlength=m))]))


# ---------------------------------------------------------------------------
# step 5: one softmax over m compressed + k raw pairs [P1][P2][P3]
# ---------------------------------------------------------------------------


def check_output_k_equals_n_is_dense_attention():
    """With k = N every expert holds all keys, so each query attends densely
    over the m compressed pairs plus all N raw pairs: fp64 scaled dot-product
    attention over the concatenated keys [Ql; K] and values [Vl; V]."""
    rng = _rng(61)
    for N, d, m, scale in [(60, 8, 5, 0.35), (196, 16, 25, 0.25)]:
        Q = rng.standard_normal((N, d))
        K = rng.standard_normal((N, d))
        V = rng.standard_normal((N, d))
        Ql = rng.standard_normal((m, d))
        Vl = rng.standard_normal((m, d))
        idx = np.tile(np.arange(N, dtype=np.int32), (m, 1))
        r = rng.integers(0, m, N).astype(np.int32)
        got = O.output(Q, K, V, Ql, Vl, idx, r, scale)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
        ref = F.scaled_dot_product_attention(t(Q), t(np.vstack([Ql, K])), t(np.vstack([Vl, V])),
                                             scale=scale)[0, 0].numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def check_output_pair_count_closed_form():
    """With all logits equal, every one of the m + k pairs gets weight
    1/(m+k): 25 + 25 = 50 pairs at m = k = 25 (the pages' ImageNet count),
    none merged or dropped, even when the expert's keys repeat."""
    rng = _rng(62)
    N, d, m, k = 196, 8, 25, 25
    Q = np.zeros((N, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    Ql = rng.standard_normal((m, d))
    Vl = rng.standard_normal((m, d))
    idx = np.tile(np.arange(k, dtype=np.int32), (m, 1))
    r = rng.integers(0, m, N).astype(np.int32)
    got = O.output(Q, K, V, Ql, Vl, idx, r, 0.125)
    want = (Vl.sum(0) + V[:k].sum(0)) / (m + k)
    np.testing.assert_allclose(got, np.tile(want, (N, 1)), rtol=1e-12, atol=1e-14)


def check_golden_pair_count_m25_k25():
    """The pages' worked count (tests/golden/pair_count_m25_k25.json): at
    m = k = 25 a query attends over 25 compressed and 25 raw pairs, 50 in
    all.  One-hot values (a column per landmark and per key) make each
    pair's softmax weight appear in its own output column, so the pairs a
    query attends over can be counted; with equal logits each weighs 1/50."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "pair_count_m25_k25.json")))
    m, k = g["m"], g["k"]
    gh, gw, mh, mw = g["grid"]
    N = gh * gw
    assert mh * mw == m and g["compressed_pairs"] + g["raw_pairs"] == g["total_pairs"]
    rng = _rng(65)
    d = m + N
    Q = np.zeros((N, d))  # equal logits for every pair
    K = rng.standard_normal((N, d))
    Vl = np.eye(m, d)
    V = np.eye(N, d, k=m)
    Ql = rng.standard_normal((m, d))
    idx = np.sort(np.stack([rng.choice(N, k, replace=False) for _ in range(m)]), 1).astype(
        np.int32)
    r = rng.integers(0, m, N).astype(np.int32)
    out = O.output(Q, K, V, Ql, Vl, idx, r, 0.125)
    for q in range(N):
        used = np.flatnonzero(out[q] > 0)
        assert used.size == g["total_pairs"]
        assert np.count_nonzero(used < m) == g["compressed_pairs"]
        assert np.array_equal(used[used >= m] - m, idx[r[q]])
        np.testing.assert_allclose(out[q, used], 1.0 / g["total_pairs"], rtol=1e-14)


def check_output_uses_routed_expert():
    """Each query reads exactly the expert it is routed to: compare against
    dense attention over [Ql; K[idx[route[q]]]] computed per query with
    torch."""
    rng = _rng(63)
    N, d, m, k, scale = 80, 8, 4, 9, 0.4
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Ql, Vl = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    idx = np.sort(np.stack([rng.choice(N, k, replace=False) for _ in range(m)]), 1).astype(
        np.int32)
    r = rng.integers(0, m, N).astype(np.int32)
    got = O.output(Q, K, V, Ql, Vl, idx, r, scale)
    for q in range(N):
        kk = torch.from_numpy(np.vstack([Ql, K[idx[r[q]]]]))
        vv = torch.from_numpy(np.vstack([Vl, V[idx[r[q]]]]))
        w = torch.softmax(scale * (kk @ torch.from_numpy(Q[q])), 0)
        np.testing.assert_allclose(got[q], (w @ vv).numpy(), rtol=1e-11, atol=1e-13)
    # a query subset gives the same rows
    sel = np.array([3, 77, 0, 41])
    np.testing.assert_array_equal(O.output(Q, K, V, Ql, Vl, idx, r, scale, qsel=sel), got[sel])


def check_output_invariants():
    rng = _rng(64)
    N, d, m, k = 100, 8, 5, 12
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Ql, Vl = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    idx = np.sort(np.stack([rng.choice(N, k, replace=False) for _ in range(m)]), 1).astype(
        np.int32)
    r = rng.integers(0, m, N).astype(np.int32)
    out = O.output(Q, K, V, Ql, Vl, idx, r, 0.3)
    for q in range(N):
        pool_v = np.vstack([Vl, V[idx[r[q]]]])
        assert np.all(out[q] <= pool_v.max(0) + 1e-12)
        assert np.all(out[q] >= pool_v.min(0) - 1e-12)
    # relabelling the keys (K, V rows and the expert indices) changes nothing
    p = rng.permutation(N)
    inv = np.argsort(p)
    idx2 = np.sort(inv[idx], 1).astype(np.int32)
    out2 = O.output(Q, K[p], V[p], Ql, Vl, idx2, r, 0.3)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# several experts per query (s > 1): the pages name s and run only s = 1
# ([P2], the remark on the experiments' routing; [P3], the configuration named
# before the concatenation).  Reading: the s best landmarks (ties to the lower
# index, best first), and one softmax over the m compressed pairs and the k
# pairs of every routed expert, a key shared by two experts counted once per
# expert, which is what [P3] Algorithm 1's per-expert attention combined by
# online softmax gives.
# ---------------------------------------------------------------------------


def check_route_s_vs_lexsort_with_ties():
    """The s experts are the first s landmarks in the order (larger logit,
    then lower index), from numpy's lexsort over exact integer logits with
    many ties; s = 1 is the single-expert routing; s = m lists every
    landmark once."""
    rng = _rng(81)
    Q = _int_data(rng, (300, 4), -2, 2)
    Ql = _int_data(rng, (7, 4), -1, 1)
    R = Q @ Ql.T
    order = np.stack([np.lexsort((np.arange(7), -R[q])) for q in range(300)])
    for s in (1, 2, 3, 7):
        assert np.array_equal(O.route_s(Q, Ql, s), order[:, :s])
    assert np.array_equal(O.route_s(Q, Ql, 1)[:, 0], O.route(Q, Ql))
    sel = rng.choice(300, 23, replace=False)
    assert np.array_equal(O.route_s(Q, Ql, 3, qsel=sel), order[sel, :3])


def check_bucket_s_vs_stable_argsort():
    """Every (query, expert) assignment, grouped by expert with queries in
    index order: a stable argsort of the flattened routes, each entry mapped
    back to its query."""
    rng = _rng(82)
    for N, m, s in [(500, 9, 3), (40, 4, 4), (7, 5, 1)]:
        routes = np.stack([rng.permutation(m)[:s] for _ in range(N)]).astype(np.int32)
        off, perm = O.bucket_s(routes, m)
        flat = routes.reshape(-1)
        assert np.array_equal(perm, np.argsort(flat, kind="stable") // s)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=m))]))
    # one query listing the same expert twice is rejected
    try:
        O.bucket_s(np.array([[1, 1]], np.int32), 3)
    except ValueError:
        pass
    else:
        raise AssertionError("repeated expert accepted")


def _s_case(rng, N=70, d=8, m=6, k=9, s=3):
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Ql, Vl = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    # overlapping experts: keys drawn from the first half of the sequence
    idx = np.sort(np.stack([rng.choice(N // 2, k, replace=False) for _ in range(m)]), 1)
    routes = np.stack([rng.permutation(m)[:s] for _ in range(N)])
    return Q, K, V, Ql, Vl, idx.astype(np.int32), routes.astype(np.int32)


def check_output_s_vs_concatenated_attention():
    """Per query, torch's softmax attention over the stacked keys
    [Ql; K[idx[e1]]; ...; K[idx[es]]] and values [Vl; V[...]; ...]."""
    rng = _rng(83)
    Q, K, V, Ql, Vl, idx, routes = _s_case(rng)
    scale = 0.37
    got = O.output_s(Q, K, V, Ql, Vl, idx, routes, scale)
    for q in range(Q.shape[0]):
        kk = torch.from_numpy(np.vstack([Ql] + [K[idx[e]] for e in routes[q]]))
        vv = torch.from_numpy(np.vstack([Vl] + [V[idx[e]] for e in routes[q]]))
        w = torch.softmax(scale * (kk @ torch.from_numpy(Q[q])), 0)
        np.testing.assert_allclose(got[q], (w @ vv).numpy(), rtol=1e-11, atol=1e-13)
    sel = np.array([5, 0, 69])
    np.testing.assert_array_equal(O.output_s(Q, K, V, Ql, Vl, idx, routes, scale, qsel=sel),
                                  got[sel])


def check_output_s_is_online_softmax_of_expert_partials():
    """[P3] Algorithm 1: attend each routed expert's pairs separately, keep
    (max, sum, weighted sum) per part, and combine the parts (the compressed
    pairs and the s experts) by rescaling to a common maximum."""
    rng = _rng(84)
    Q, K, V, Ql, Vl, idx, routes = _s_case(rng, N=40, s=4)
    scale = 0.5
    got = O.output_s(Q, K, V, Ql, Vl, idx, routes, scale)
    for q in range(Q.shape[0]):
        parts = [(Ql, Vl)] + [(K[idx[e]], V[idx[e]]) for e in routes[q]]
        mx, tot, acc = -np.inf, 0.0, np.zeros(Q.shape[1])
        for kp, vp in parts:
            lg = scale * (kp @ Q[q])
            pm = lg.max()
            pe = np.exp(lg - pm)
            nm = max(mx, pm)
            tot = tot * np.exp(mx - nm) + pe.sum() * np.exp(pm - nm)
            acc = acc * np.exp(mx - nm) + (pe @ vp) * np.exp(pm - nm)
            mx = nm
        np.testing.assert_allclose(got[q], acc / tot, rtol=1e-11, atol=1e-13)


def check_output_s_shared_keys_count_per_expert():
    """With k = N every expert holds every key, so the s experts repeat all N
    pairs s times: closed form softmax over the compressed logits and the raw
    logits raised by log(s).  A union that merged repeated keys, or a drop of
    any expert, fails this."""
    rng = _rng(85)
    N, d, m, s, scale = 50, 8, 5, 3, 0.3
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Ql, Vl = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    idx = np.tile(np.arange(N, dtype=np.int32), (m, 1))
    routes = np.stack([rng.permutation(m)[:s] for _ in range(N)]).astype(np.int32)
    got = O.output_s(Q, K, V, Ql, Vl, idx, routes, scale)
    lc = scale * (Q @ Ql.T)
    lr = scale * (Q @ K.T) + np.log(s)
    lg = np.hstack([lc, lr])
    w = np.exp(lg - lg.max(1, keepdims=True))
    want = (w[:, :m] @ Vl + w[:, m:] @ V) / w.sum(1, keepdims=True)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


def check_output_s_reduces_and_is_order_free():
    """s = 1 is the single-expert output bit for bit; reordering a query's
    experts changes only the summation order."""
    rng = _rng(86)
    Q, K, V, Ql, Vl, idx, routes = _s_case(rng, s=3)
    one = O.output_s(Q, K, V, Ql, Vl, idx, routes[:, :1], 0.4)
    np.testing.assert_array_equal(one, O.output(Q, K, V, Ql, Vl, idx, routes[:, 0], 0.4))
    a = O.output_s(Q, K, V, Ql, Vl, idx, routes, 0.4)
    b = O.output_s(Q, K, V, Ql, Vl, idx, routes[:, ::-1], 0.4)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# the dense-attention baseline (the full attention the pages time MiTA
# against: "NeurIPS 2026 | Mixture-of-Top-k 注意力…", section
# "长序列建模：实际运行时间也能明显缩短")
# ---------------------------------------------------------------------------


def check_dense_vs_torch_sdpa():
    """fp64 dense attention equals torch's scaled_dot_product_attention in
    float64 on the CPU (a library routine of the same definition)."""
    rng = _rng(71)
    for N, d, scale in [(1, 4, 0.5), (37, 8, 0.3), (200, 16, 0.125)]:
        Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
        got = O.dense(Q, K, V, scale)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
        ref = F.scaled_dot_product_attention(t(Q), t(K), t(V), scale=scale)[0, 0].numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def check_dense_is_output_over_every_key():
    """Step 5 with k = N attends over [Ql; K] and [Vl; V]: exactly dense
    attention over those concatenated pairs (queries taken from a padded
    array through the query selection)."""
    rng = _rng(72)
    N, d, m, scale = 90, 8, 6, 0.3
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    Ql, Vl = rng.standard_normal((m, d)), rng.standard_normal((m, d))
    idx = np.tile(np.arange(N, dtype=np.int32), (m, 1))
    r = rng.integers(0, m, N).astype(np.int32)
    want = O.output(Q, K, V, Ql, Vl, idx, r, scale)
    Qpad = np.vstack([np.zeros((m, d)), Q])
    got = O.dense(Qpad, np.vstack([Ql, K]), np.vstack([Vl, V]), scale, qsel=np.arange(m, m + N))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def check_dense_invariants():
    rng = _rng(73)
    N, d = 120, 8
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    out = O.dense(Q, K, V, 0.4)
    # a convex combination of the value rows
    assert np.all(out <= V.max(0) + 1e-12) and np.all(out >= V.min(0) - 1e-12)
    # zero queries see equal logits: the plain mean of the values (closed form)
    np.testing.assert_allclose(O.dense(np.zeros((N, d)), K, V, 0.4), np.tile(V.mean(0), (N, 1)),
                               rtol=1e-12, atol=1e-14)
    # relabelling keys and values together changes nothing
    p = rng.permutation(N)
    np.testing.assert_allclose(O.dense(Q, K[p], V[p], 0.4), out, rtol=1e-12, atol=1e-13)
    # one key far above the rest takes all the weight
    K2 = K.copy()
    K2[17] = 50.0 * Q[3] / np.linalg.norm(Q[3])
    np.testing.assert_allclose(O.dense(Q, K2, V, 1.0, qsel=[3])[0], V[17], rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# whole pipeline
# ---------------------------------------------------------------------------


def check_forward_composes_steps():
    rng = _rng(71)
    B, H, N, d, grid, k = 2, 2, 196, 16, (14, 14, 5, 5), 25
    Q, K, V = (torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32))
               .to(torch.bfloat16).to(torch.float64).numpy() for _ in range(3))
    res = O.forward(Q, K, V, grid, k, 0.125, O.ROUND_BF16)
    for b in range(B):
        for h in range(H):
            ql = O.pool(Q[b, h], *grid, O.ROUND_BF16)
            assert np.array_equal(res["ql"][b, h], ql)
            idx = O.topk(ql, K[b, h], k)
            assert np.array_equal(res["idx"][b, h], idx)
            vl = O.landmark_values(ql, K[b, h], V[b, h], 0.125)
            np.testing.assert_array_equal(res["vl"][b, h], vl)
            r = O.route(Q[b, h], ql)
            assert np.array_equal(res["route"][b, h], r)
            off, perm = O.bucket(r, 25)
            assert np.array_equal(res["offsets"][b, h], off)
            assert np.array_equal(res["perm"][b, h], perm)
            out = O.output(Q[b, h], K[b, h], V[b, h], ql, vl, idx, r, 0.125)
            np.testing.assert_array_equal(res["out"][b, h], out)


# ---------------------------------------------------------------------------
# backward pass (training): the experts and routes held fixed [P1 section
# "长序列建模：训练时间从10.6小时降至2.4小时" — the pages' wall-clock results are
# training times]
# ---------------------------------------------------------------------------


def _bw_case(rng, N, d, grid, k, scale):
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    ql = O.pool(Q, *grid, O.ROUND_NONE)
    idx = O.topk(ql, K, k)
    r = O.route(Q, ql)
    G = rng.standard_normal((N, d))
    return Q, K, V, idx, r, G


def _torch_forward_fixed(Q, K, V, grid, idx, r, scale):
    """The forward written with torch's own operators (adaptive average
    pooling, softmax, matmul) for autograd, with the experts and routes
    given (not re-selected)."""
    gh, gw, mh, mw = grid
    N, d = Q.shape
    ql = F.adaptive_avg_pool2d(Q.T.reshape(d, gh, gw), (mh, mw)).reshape(d, mh * mw).T
    A = torch.softmax(scale * (ql @ K.T), dim=-1)
    vl = A @ V
    outs = []
    for q in range(N):
        ex = torch.as_tensor(idx[r[q]].astype(np.int64))
        logits = scale * torch.cat([ql @ Q[q], K[ex] @ Q[q]])
        w = torch.softmax(logits, dim=0)
        outs.append(w[:ql.shape[0]] @ vl + w[ql.shape[0]:] @ V[ex])
    return torch.stack(outs)


def check_backward_vs_autograd():
    """The hand-derived backward against torch autograd of the same forward
    (fp64), on a 1D grid and an overlapping 2D grid (14x14 -> 5x5 bins)."""
    rng = _rng(81)
    for N, d, grid, k, scale in [(30, 8, (1, 30, 1, 5), 4, 0.35),
                                 (196, 4, (14, 14, 5, 5), 6, 0.5)]:
        Q, K, V, idx, r, G = _bw_case(rng, N, d, grid, k, scale)
        dQ, dK, dV = O.backward(Q, K, V, grid, k, scale, O.ROUND_NONE, idx, r, G)
        Qt, Kt, Vt = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        out = _torch_forward_fixed(Qt, Kt, Vt, grid, idx, r, scale)
        # the torch forward is the oracle's forward (pinned elsewhere)
        vl = O.landmark_values(O.pool(Q, *grid, O.ROUND_NONE), K, V, scale)
        ref_out = O.output(Q, K, V, O.pool(Q, *grid, O.ROUND_NONE), vl, idx, r, scale)
        np.testing.assert_allclose(out.detach().numpy(), ref_out, rtol=1e-11, atol=1e-12)
        (out * torch.from_numpy(G)).sum().backward()
        for got, t in ((dQ, Qt), (dK, Kt), (dV, Vt)):
            np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_backward_finite_differences():
    """Central differences of sum(dout * out) through the oracle's own
    forward steps (fixed experts and routes) on every entry of Q, K, V."""
    rng = _rng(82)
    N, d, grid, k, scale = 12, 3, (3, 4, 2, 2), 3, 0.7
    Q, K, V, idx, r, G = _bw_case(rng, N, d, grid, k, scale)
    dQ, dK, dV = O.backward(Q, K, V, grid, k, scale, O.ROUND_NONE, idx, r, G)

    def loss(Q, K, V):
        ql = O.pool(Q, *grid, O.ROUND_NONE)
        vl = O.landmark_values(ql, K, V, scale)
        return float((O.output(Q, K, V, ql, vl, idx, r, scale) * G).sum())

    eps = 1e-6
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        for t in range(N):
            for a in range(d):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][t, a] += eps
                up = loss(*args)
                args[which][t, a] -= 2 * eps
                down = loss(*args)
                fd = (up - down) / (2 * eps)
                assert abs(fd - grad[t, a]) <= 1e-6 * (1 + abs(fd)), (which, t, a, fd, grad[t, a])


def check_backward_invariants():
    """Each output row is a convex combination of value rows (the landmark
    values being convex combinations of V), so the value gradients sum to the
    output gradients; the gradients are linear in dout; the rounding of the
    landmark queries changes the point of evaluation, not the rule."""
    rng = _rng(83)
    N, d, grid, k, scale = 40, 6, (1, 40, 1, 6), 5, 0.4
    Q, K, V, idx, r, G = _bw_case(rng, N, d, grid, k, scale)
    dQ, dK, dV = O.backward(Q, K, V, grid, k, scale, O.ROUND_NONE, idx, r, G)
    np.testing.assert_allclose(dV.sum(0), G.sum(0), rtol=1e-12, atol=1e-12)
    d2 = O.backward(Q, K, V, grid, k, scale, O.ROUND_NONE, idx, r, -2.5 * G)
    for a, b in zip((dQ, dK, dV), d2):
        np.testing.assert_allclose(b, -2.5 * a, rtol=1e-12, atol=1e-13)
    z = O.backward(Q, K, V, grid, k, scale, O.ROUND_NONE, idx, r, 0 * G)
    assert all(np.all(t == 0) for t in z)
    # bf16 rounding of Ql: the gradients are those at the rounded landmarks
    Qb = np.vectorize(O.round_bf16)(Q)
    b16 = O.backward(Qb, K, V, grid, k, scale, O.ROUND_BF16, idx, r, G)
    Qt, Kt, Vt = (torch.tensor(x, requires_grad=True) for x in (Qb, K, V))
    gh, gw, mh, mw = grid
    ql = F.adaptive_avg_pool2d(Qt.T.reshape(d, gh, gw), (mh, mw)).reshape(d, mh * mw).T
    qlr = torch.from_numpy(O.pool(Qb, *grid, O.ROUND_BF16))
    ql = ql + (qlr - ql).detach()  # rounded values, identity derivative
    A = torch.softmax(scale * (ql @ Kt.T), dim=-1)
    vl = A @ Vt
    outs = []
    for q in range(N):
        ex = torch.as_tensor(idx[r[q]].astype(np.int64))
        w = torch.softmax(scale * torch.cat([ql @ Qt[q], Kt[ex] @ Qt[q]]), dim=0)
        outs.append(w[:ql.shape[0]] @ vl + w[ql.shape[0]:] @ Vt[ex])
    (torch.stack(outs) * torch.from_numpy(G)).sum().backward()
    for got, t in zip(b16, (Qt, Kt, Vt)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


ALL_CHECKS = [v for k_, v in sorted(globals().items()) if k_.startswith("check_")]

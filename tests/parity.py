"""GPU-vs-oracle comparison protocol.

Per (batch, head):
  1. landmark queries: bit-exact;
  2. expert index sets: equal, except where the oracle's k-th and (k+1)-th
     scores form a near-tie (counted); a differing GPU set must still consist
     of keys scoring within the near-tie band of the oracle's k-th score;
  3. landmark values: max |diff| <= tol;
  4. routes: equal, except near-ties of the best two routing logits (counted);
     the GPU's choice must score within the band of the best;
  5. perm and offsets: bit-exact against a stable sort of the GPU's routes;
  6. outputs: the oracle's output step re-run with the GPU's expert sets and
     routes (identical to the oracle's own wherever there is no near-tie):
     max |diff| <= tol.
Near-tie (top-k and routing alike): gap between the two fp64 scores below
max(1e-4 * max(|a|, |b|), 2 * d * 2^-24 * max(A_a, A_b)), where A is the sum
of |products| of the dot product (the fp32 accumulation error bound).
Near-ties are rare for continuous inputs, so their counts are capped: at
most max(1, 1% of the experts checked) top-k near-ties and max(1, 0.1% of
the queries checked) routing near-ties per comparison.  A band that grew too
wide (and so excused real selection or routing errors) would break a cap.
Tolerance: 1e-5 absolute for fp32 inputs, 5e-3 for bf16 inputs (fp32
accumulation).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle as O

TOL = {"f32": 1e-5, "bf16": 5e-3}


def near_tie_threshold(a, b, A_a, A_b, d):
    return max(1e-4 * max(abs(a), abs(b)), 2 * d * 2.0**-24 * max(A_a, A_b))


@dataclass
class Report:
    heads: int = 0
    ql_mismatch: int = 0
    topk_near_ties: int = 0
    route_near_ties: int = 0
    vl_max_err: float = 0.0
    out_max_err: float = 0.0
    queries_checked: int = 0
    experts_checked: int = 0
    failures: list = field(default_factory=list)

    def fail(self, msg):
        if len(self.failures) < 20:
            self.failures.append(msg)

    def caps(self):
        """(top-k cap, routing cap) on the near-tie counts."""
        return max(1, self.experts_checked // 100), max(1, self.queries_checked // 1000)

    def cap_failures(self):
        tcap, rcap = self.caps()
        msgs = []
        if self.topk_near_ties > tcap:
            msgs.append(f"{self.topk_near_ties} top-k near-ties over {self.experts_checked} "
                        f"experts exceed the cap {tcap}")
        if self.route_near_ties > rcap:
            msgs.append(f"{self.route_near_ties} routing near-ties over {self.queries_checked} "
                        f"queries exceed the cap {rcap}")
        return msgs

    def ok(self):
        return not self.failures and not self.cap_failures()

    def problems(self):
        return self.failures + self.cap_failures()

    def summary(self):
        return (f"heads={self.heads} queries={self.queries_checked} experts={self.experts_checked} "
                f"ql_mismatch={self.ql_mismatch} "
                f"topk_near_ties={self.topk_near_ties} route_near_ties={self.route_near_ties} "
                f"vl_max_err={self.vl_max_err:.3e} out_max_err={self.out_max_err:.3e}")


def gpu_results_to_numpy(res):
    """Convert mita_forward_ex results (torch, on the GPU) to numpy."""
    import torch

    out, idx, route, dbg = res
    torch.cuda.synchronize()
    return {
        "out": out.cpu().numpy(),
        "idx": idx.cpu().numpy(),
        "route": route.cpu().numpy(),
        "ql": dbg["ql"].cpu().to(torch.float64).numpy(),
        "vl": dbg["vl"].cpu().numpy().astype(np.float64),
        "perm": dbg["perm"].cpu().numpy(),
        "offsets": dbg["offsets"].cpu().numpy(),
    }


def check_head(w, Qh, Kh, Vh, g, rep: Report, qsel=None, exact_ties=False):
    """Compare one head.  Qh, Kh, Vh: [N, d] exact fp64 inputs; g: dict of this
    head's GPU results; qsel: optional query sample; exact_ties: demand
    identical sets/routes even at near-ties (for inputs whose scores are
    exact in fp32, where ties must resolve by index on both sides).  Adds
    this head's counts to rep (near-ties, experts and queries checked) and
    returns it."""
    tol = TOL[w.dtype]
    N, d = Qh.shape
    m, k = w.m, w.k
    rmode = O.ROUND_BF16 if w.dtype == "bf16" else O.ROUND_F32
    rep.heads += 1

    ql = O.pool(Qh, *w.grid, rmode)
    if not np.array_equal(ql, g["ql"]):
        bad = int(np.sum(ql != g["ql"]))
        rep.ql_mismatch += bad
        rep.fail(f"landmark queries differ in {bad} elements")

    idx_o, gap = O.topk(ql, Kh, k, with_gap=True)
    rep.experts_checked += m
    for i in range(m):
        if np.array_equal(idx_o[i], g["idx"][i]):
            continue
        if exact_ties:
            rep.fail(f"expert {i}: index set differs (exact-tie input)")
            continue
        thr = near_tie_threshold(gap[i, 0], gap[i, 1], gap[i, 2], gap[i, 3], d)
        gi = g["idx"][i]
        if (len(set(gi.tolist())) != k or gi.min() < 0 or gi.max() >= N
                or np.any(np.diff(gi) <= 0)):
            rep.fail(f"expert {i}: GPU indices invalid")
            continue
        if not (gap[i, 0] - gap[i, 1] < thr):
            rep.fail(f"expert {i}: index set differs without a near-tie "
                     f"(gap {gap[i, 0] - gap[i, 1]:.3e}, band {thr:.3e})")
            continue
        s_gpu = Kh[gi] @ ql[i]
        if np.min(s_gpu) < gap[i, 0] - thr:
            rep.fail(f"expert {i}: GPU picked a key below the near-tie band")
            continue
        rep.topk_near_ties += 1

    vl = O.landmark_values(ql, Kh, Vh, w.scale)
    err = float(np.max(np.abs(vl - g["vl"])))
    rep.vl_max_err = max(rep.vl_max_err, err)
    if not err <= tol:
        rep.fail(f"landmark values max err {err:.3e} > {tol}")

    qs = np.arange(N) if qsel is None else np.asarray(qsel)
    r_o, top2 = O.route(Qh, ql, qsel=qs, with_top2=True)
    r_g = g["route"][qs]
    if np.any((g["route"] < 0) | (g["route"] >= m)):
        rep.fail("route out of range")
        return rep
    for j in np.nonzero(r_o != r_g)[0]:
        q = qs[j]
        if exact_ties:
            rep.fail(f"query {q}: route differs (exact-tie input)")
            continue
        thr = near_tie_threshold(top2[j, 0], top2[j, 1], top2[j, 2], top2[j, 3], d)
        chosen = float(Qh[q] @ ql[r_g[j]])
        if top2[j, 0] - top2[j, 1] < thr and chosen >= top2[j, 0] - thr:
            rep.route_near_ties += 1
        else:
            rep.fail(f"query {q}: route {r_g[j]} vs oracle {r_o[j]} without a near-tie")

    perm_ref = np.argsort(g["route"], kind="stable").astype(np.int32)
    if not np.array_equal(perm_ref, g["perm"]):
        rep.fail("perm differs from the stable sort of the GPU routes")
    off_ref = np.concatenate([[0], np.cumsum(np.bincount(g["route"], minlength=m))]).astype(np.int32)
    if not np.array_equal(off_ref, g["offsets"]):
        rep.fail("offsets differ from the GPU routes' counts")

    out_o = O.output(Qh, Kh, Vh, ql, vl, g["idx"], g["route"], w.scale, qsel=qs)
    err = float(np.max(np.abs(out_o - g["out"][qs])))
    rep.out_max_err = max(rep.out_max_err, err)
    rep.queries_checked += len(qs)
    if not err <= tol:
        rep.fail(f"output max err {err:.3e} > {tol}")
    return rep


def check_head_s(w, Qh, Kh, Vh, g, s, rep: Report, qsel=None):
    """One head of a forward with s experts per query (g: out [N, d], idx
    [m, k], routes [N, s] of the GPU).  Experts as in check_head.  Routes:
    each query's list equals the oracle's (route_s), or differs only where
    the oracle's sorted logits are near-tied: the GPU's j-th choice must then
    score within the band of the oracle's j-th best (counted as a routing
    near-tie).  Outputs: the oracle's output_s re-run with the GPU's experts
    and routes, within the tolerance."""
    tol = TOL[w.dtype]
    N, d = Qh.shape
    m, k = w.m, w.k
    rmode = O.ROUND_BF16 if w.dtype == "bf16" else O.ROUND_F32
    rep.heads += 1
    ql = O.pool(Qh, *w.grid, rmode)
    idx_o, gap = O.topk(ql, Kh, k, with_gap=True)
    rep.experts_checked += m
    for i in range(m):
        if np.array_equal(idx_o[i], g["idx"][i]):
            continue
        thr = near_tie_threshold(gap[i, 0], gap[i, 1], gap[i, 2], gap[i, 3], d)
        if not (gap[i, 0] - gap[i, 1] < thr):
            rep.fail(f"expert {i}: index set differs without a near-tie")
            continue
        if np.min(Kh[g["idx"][i]] @ ql[i]) < gap[i, 0] - thr:
            rep.fail(f"expert {i}: GPU picked a key below the near-tie band")
            continue
        rep.topk_near_ties += 1
    vl = O.landmark_values(ql, Kh, Vh, w.scale)
    qs = np.arange(N) if qsel is None else np.asarray(qsel)
    r_o = O.route_s(Qh, ql, s, qsel=qs)
    r_g = g["routes"][qs]
    if np.any((r_g < 0) | (r_g >= m)):
        rep.fail("route out of range")
        return rep
    for jq in np.nonzero(np.any(r_o != r_g, axis=1))[0]:
        q = qs[jq]
        if len(set(r_g[jq].tolist())) != s:
            rep.fail(f"query {q}: repeated expert in {r_g[jq]}")
            continue
        R = Qh[q] @ ql.T
        A = np.abs(Qh[q][None, :] * ql).sum(1)
        order = r_o[jq]
        ok = True
        for j in range(s):
            if r_g[jq, j] == order[j]:
                continue
            # the oracle's j-th and the next best logit must be near-tied,
            # and the GPU's choice must score within that band
            nxt = np.sort(R)[::-1][j + 1] if j + 1 < m else -np.inf
            thr = near_tie_threshold(R[order[j]], nxt, A[order[j]], A.max(), d)
            if not (R[order[j]] - nxt < thr and R[r_g[jq, j]] >= R[order[j]] - thr):
                ok = False
        if ok:
            rep.route_near_ties += 1
        else:
            rep.fail(f"query {q}: routes {r_g[jq]} vs oracle {order} without a near-tie")
    out_o = O.output_s(Qh, Kh, Vh, ql, vl, g["idx"], g["routes"], w.scale, qsel=qs)
    err = float(np.max(np.abs(out_o - g["out"][qs])))
    rep.out_max_err = max(rep.out_max_err, err)
    rep.queries_checked += len(qs)
    if not err <= tol:
        rep.fail(f"output max err {err:.3e} > {tol}")
    return rep

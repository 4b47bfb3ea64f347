#!/usr/bin/env python3
"""Throughput of the MiTA forward pass on one MI355X (and, beside it, of the
backward pass used in training).

One step = one complete forward (all five stages: pool, landmark scan +
merge, route, bucket, expert attention) over one batch of synthetic inputs
already resident in HBM.  Default workload: the 1M-token length-scaling
configuration (B=1, H=4, N=1048576, d=64, bf16, m=k=64, 1D windows).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MiTA fwd Mtokens·heads/s at N=64K–1M; % of HBM roofline (gather-bound)"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
TOL_BY_DTYPE = {"f32": 1e-5, "bf16": 5e-3}  # the parity tolerance of each input type
# profiler stages that are exactly one kernel launch, with that kernel's name
SINGLE_KERNEL_STAGES = {"landmark_scan": "k_scan", "route": "k_route",
                        "expert_attend": "k_attend", "single_launch": "k_small"}
KERNEL_SOURCES = {"k_scan": "kernels_scan.hip", "k_route": "kernels_route.hip",
                  "k_attend": "kernels_attend.hip", "k_small": "kernels_small.hip",
                  "k_medium": "kernels_medium.hip"}
# bf16 heads of 257 .. MEDIUM_MAX_N tokens (one expert per query) run steps 2
# to 4 in one launch, which the stage profiler books as landmark_scan
MEDIUM_MAX_N = 1600


def medium_path(w, s: int = 1) -> bool:
    return w.dtype == "bf16" and s == 1 and 256 < w.N <= MEDIUM_MAX_N and w.m <= 64 and w.k <= 64


def stage_kernel(stage: str, w, s: int = 1) -> str:
    """The kernel that makes up a single-launch stage on this workload."""
    if stage == "landmark_scan" and medium_path(w, s):
        return "k_medium"
    return SINGLE_KERNEL_STAGES[stage]
# HBM bytes per launch on the 1M-token workload from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (scaled by 2.0 and 1.0, the factors a 1 GiB copy kernel gives),
# with the sha1 of the kernel's sources (kernel_sha) when the counters were
# taken: a kernel whose sources changed since reports traffic null.
COUNTED_TRAFFIC = {
    "len_1m": {
        "k_scan": {"sha": "b07459056d71", "bytes": 1093190594},
        "k_route": {"sha": "26ed5810c057", "bytes": 565138667},
        "k_attend": {"sha": "9113e1ae126b", "bytes": 1635330403},
    },
}


def kernel_sources(symbol: str) -> list[str]:
    """A kernel's source file, then every local header it includes, directly
    or through other local headers, in name order."""
    import re

    csrc = os.path.join(ROOT, "mixture_top_sparse_amd", "csrc")
    seen, todo = set(), [KERNEL_SOURCES[symbol]]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        with open(os.path.join(csrc, f)) as fh:
            todo += [h for h in re.findall(r'^#include "([^"]+)"', fh.read(), flags=re.M)
                     if os.path.exists(os.path.join(csrc, h))]
    return [KERNEL_SOURCES[symbol]] + sorted(seen - {KERNEL_SOURCES[symbol]})


def kernel_sha(symbol: str) -> str:
    """sha1 (12 hex digits) of a kernel's source file and its local headers."""
    import hashlib

    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "mixture_top_sparse_amd", "csrc")
    for f in kernel_sources(symbol):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def counted_traffic(workload: str, symbol: str):
    rec = COUNTED_TRAFFIC.get(workload, {}).get(symbol)
    if rec is None or rec["sha"] != kernel_sha(symbol):
        return None
    return rec["bytes"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def threshold_tiles(w) -> int:
    """Key tiles of 64 the top-k pre-threshold reads per head (the library's
    rule: a quarter of the tiles, at most 1024, when that gives at least 256
    samples, else half of them when that does; below that every tile; none
    when there are fewer than k keys)."""
    ktiles = -(-w.N // 64)
    if w.N < w.k:
        return 0
    if ktiles // 4 >= 256:
        return min(ktiles // 4, 1024)
    return ktiles // 2 if ktiles // 2 >= 256 else ktiles


def stage_bytes(w, s: int = 1) -> dict[str, float]:
    """Algorithmic HBM bytes per launch of each stage: what the stage must
    read and write at minimum (inputs once, outputs once), not what the
    implementation happens to move."""
    e = 2 if w.dtype == "bf16" else 4
    BH, N, d, m, k = w.B * w.H, w.N, w.d, w.m, w.k
    rows = min(m * k, N)
    # the mid-length launch: K, V and Q read, experts, landmark values,
    # routes and the bucket order written
    scan = (BH * (3 * N * d * e + 4 * m * k + 4 * m * d + 4 * N + 4 * N) if medium_path(w, s)
            else BH * (2 * N * d * e))
    # step 4 (bucketing: read the routes, write perm) rides in the merge
    # launch; its prefix over the routing counts in the scan launch moves
    # no per-token bytes
    return {
        "pool": BH * (N * d * e + m * d * e),
        "landmark_threshold": BH * (threshold_tiles(w) * 64 * d * e + m * d * e),
        "route": BH * (N * d * e + 4 * N),
        "landmark_scan": scan,
        "landmark_merge": BH * (4 * m * k + 4 * m * d + 4 * N + 4 * N),
        "expert_attend": BH * (N * d * e + 4 * N * d + 4 * N + rows * 2 * d * e),
        # the one-launch path of short sequences runs all five steps
        "single_launch": path_bytes(w),
    }


def path_bytes(w) -> float:
    """Algorithmic bytes of the whole path: read Q, K, V once, write the fp32
    output and the routes once, plus the expert table and one re-gather of the
    selected key/value rows per head."""
    e = 2 if w.dtype == "bf16" else 4
    BH, N, d, m, k = w.B * w.H, w.N, w.d, w.m, w.k
    return BH * (N * (3 * d * e + 4 * d + 4) + 4 * m * k + min(m * k, N) * 2 * d * e)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, Qt, Kt, Vt, g_out, g_idx, g_route):
    """The fp64 oracle on the host cores, on one (batch, head) slice of the
    same workload; also compares that slice with the GPU's results under the
    parity protocol (every expert, a sample of 4096 queries)."""
    import numpy as np
    import torch

    import oracle as O

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import Report, check_head

    Q, K, V = (t[0:1, 0:1].cpu().to(torch.float64).numpy() for t in (Qt, Kt, Vt))  # [1,1,N,d]
    rmode = O.ROUND_BF16 if w.dtype == "bf16" else O.ROUND_F32
    host_cores = len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle on 1 of {w.B * w.H} heads, N={w.N}, {O.threads()} threads "
        f"({host_cores} host cores available)")
    t0 = time.perf_counter()
    res = O.forward(Q, K, V, w.grid, w.k, w.scale, rmode)
    dt = time.perf_counter() - t0
    idx_g = g_idx[0, 0].cpu().numpy()
    route_g = g_route[0, 0].cpu().numpy()
    sel = np.sort(np.random.default_rng(0).choice(w.N, min(w.N, 4096), replace=False))
    # the parity protocol needs the intermediates too: recompute them on the
    # GPU for this slice (mita_forward_ex on the same inputs)
    import mixture_top_sparse_amd as mts
    from parity import gpu_results_to_numpy

    sl = [t[0:1, 0:1].contiguous() for t in (Qt, Kt, Vt)]
    g = gpu_results_to_numpy(mts.mita_forward_ex(*sl, m=w.m, k=w.k, grid=w.grid, scale=w.scale))
    g = {key: val[0, 0] for key, val in g.items()}
    # the one-slice call splits the key scan differently (more splits per
    # head), so its landmark values may differ from the full call's in the
    # last bits; experts and routes must not
    same_as_full = np.array_equal(g["idx"], idx_g) and np.array_equal(g["route"], route_g)
    slice_vs_full = float(np.max(np.abs(g["out"] - g_out[0, 0].cpu().numpy())))
    rep = check_head(w, Q[0, 0], K[0, 0], V[0, 0], g, Report(), qsel=sel)
    same_idx = int(sum(np.array_equal(a, b) for a, b in zip(res["idx"][0, 0], idx_g)))
    log(f"cpu baseline slice parity: {rep.summary()}")
    return {
        "value": w.N / dt / 1e6,
        "unit": "Mtokens·heads/s",
        "cores": O.threads(),
        "host_cores": host_cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"one (batch, head) slice of the same workload: N={w.N}, m={w.m}, k={w.k}; "
                  f"full fp64 forward (all five steps) in {dt:.2f} s on {O.threads()} OpenMP "
                  f"threads",
        "seconds": dt,
        "parity_slice": {
            "experts_identical": f"{same_idx}/{w.m}",
            "routes_identical": float(np.mean(res["route"][0, 0] == route_g)),
            "topk_near_ties": rep.topk_near_ties,
            "route_near_ties_sampled": rep.route_near_ties,
            "queries_sampled": rep.queries_checked,
            "vl_max_err": rep.vl_max_err,
            "out_max_err_sampled": rep.out_max_err,
            "tolerance": TOL_BY_DTYPE[w.dtype],
            "slice_call_experts_routes_match_full_call": bool(same_as_full),
            "slice_call_out_max_diff_vs_full_call": slice_vs_full,
            "pass": rep.ok(),
        },
    }


def copy_probe(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """A plain elementwise copy (torch.neg of 1 GiB of fp32 into another
    buffer): nbytes read + nbytes written per launch."""
    import torch

    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(x, out=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 4),
            "GBs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def device_warmup(ms: float) -> dict | None:
    """A plain 256 MiB fp32 copy kernel (torch.neg) repeated for about `ms`
    milliseconds of GPU time: brings the memory clocks out of their idle
    state before the timed MiTA steps (no MiTA work, nothing timed)."""
    import torch

    if ms <= 0:
        return None
    x = torch.ones((64 << 20,), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    launches, spent = 0, 0.0
    while spent < ms:
        e0.record()
        for _ in range(10):
            torch.neg(x, out=y)
        e1.record()
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        launches += 10
    del x, y
    log(f"device warm-up: {launches} copy launches of 256 MiB in {spent:.1f} ms")
    return {"kind": "fp32 copy kernel (torch.neg), 256 MiB per launch", "launches": launches,
            "ms": round(spent, 2)}


def dense_baseline(w, Qt, Kt, Vt) -> dict:
    """Dense (full) attention on the same inputs with the library's own
    flash-attention kernel: time per forward and MFMA throughput (MiTA's
    speedup over it, the ratio the pages report against full attention, is
    added once the MiTA step is timed)."""
    import torch

    import mixture_top_sparse_amd as mts

    step = lambda: mts.mita_dense_attention(Qt, Kt, Vt, scale=w.scale)
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    once = time.perf_counter() - t0
    reps = max(1, min(5, int(2.0 / max(once, 1e-3))))  # about 2 s of timed work at most
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4.0 * w.B * w.H * float(w.N) ** 2 * w.d
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"dense attention: {ms:.3f} ms/forward ({reps} timed), {tflops:.0f} TFLOP/s")
    return {"kernel": "k_dense_bf16", "ms_per_step": round(ms, 4), "steps": reps,
            "flops": flops, "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
            "frac": round(tflops / 2500.0, 4)}


FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix rate, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix rate, published


def backward_peaks(w) -> dict[str, float]:
    """The matrix rate each backward contraction kernel runs on: bf16 MFMAs
    for bf16 inputs (their fp32 operands split into bf16 hi + lo parts),
    fp32 MFMAs for fp32 inputs."""
    peak = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    return {"bw_attend": peak, "bw_cross": peak, "bw_landmark_fwd": peak}


def backward_flops(w) -> dict[str, float]:
    """Algorithmic flops per launch of the backward's contraction
    kernels: the expert step does five (m + k) x d products per query (logits,
    dout . values, dQ, and the pair-side sums for keys and values), the
    cross-attention step five m x d products per key, the recomputed
    landmark forward two per key."""
    BH, N, d, m, k = w.B * w.H, w.N, w.d, w.m, w.k
    return {"bw_attend": BH * N * 10.0 * (m + k) * d,
            "bw_cross": BH * N * 10.0 * m * d,
            "bw_landmark_fwd": BH * N * 4.0 * m * d}


def backward_bench(w, Qt, Kt, Vt, idx, route) -> dict:
    """The backward pass (mita_backward, experts and routes from the forward
    just timed) on the same inputs: time per call, per-step times from the
    stage profiler, and its dominant kernel against the peak of the matrix
    instructions it issues (backward_peaks)."""
    import torch

    import mixture_top_sparse_amd as mts
    from mixture_top_sparse_amd.inputs import generate_dout

    dout = torch.from_numpy(generate_dout(w)).cuda()
    call = lambda: mts.mita_backward(Qt, Kt, Vt, idx, route, dout, m=w.m, k=w.k, grid=w.grid,
                                     scale=w.scale)
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    once = time.perf_counter() - t0
    reps = max(3, min(20, int(1.0 / max(once, 1e-4))))
    for _ in range(2):
        call()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    mts.mita_profile_enable(True)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    mts.mita_profile_enable(False)
    stage_ms, calls = mts.mita_profile_read()
    st = {k_: v / max(calls, 1) for k_, v in stage_ms.items() if k_.startswith("bw_")}
    fl = backward_flops(w)
    tf = {k_: fl[k_] / (st[k_] * 1e-3) / 1e12 for k_ in fl if st.get(k_, 0) > 0}
    dom = max(fl, key=lambda k_: st.get(k_, 0.0))
    value = w.B * w.H * w.N / (ms * 1e-3) / 1e6
    peak = backward_peaks(w)[dom]
    log(f"backward: {ms:.3f} ms/call ({reps} timed), {value:.1f} Mtokens.heads/s; "
        f"{dom} {st[dom]:.3f} ms at {tf[dom]:.1f} TFLOP/s (peak {peak:.1f})")
    return {"ms_per_call": round(ms, 4), "calls": reps, "value": round(value, 2),
            "unit": "Mtokens·heads/s", "stages_ms": {k_: round(v, 4) for k_, v in st.items()},
            "stages_TFLOPs": {k_: round(v, 1) for k_, v in tf.items()},
            "roofline": {"scope": "dominant backward kernel", "bound": "mfma", "kernel": dom,
                         "flops": fl[dom], "launch_ms": round(st[dom], 4),
                         "achieved": round(tf[dom], 1), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(tf[dom] / peak, 4),
                         "traffic": None}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="len_1m")
    ap.add_argument("--experts-per-query", type=int, default=1, metavar="S",
                    help="route each query to its S best landmarks (mita_forward_s; S > 1 is "
                         "the several-experts reading, timed for context, not the metric)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense", choices=["auto", "on", "off"], default="auto",
                    help="also time the hand-written dense (full) attention kernel on the same "
                         "inputs and report the speedup (auto: bf16 workloads with N >= 65536)")
    ap.add_argument("--device-warmup-ms", type=float, default=60.0,
                    help="before MiTA's own warm-up steps, run a plain memory-bound copy kernel "
                         "for this long: HBM and fabric clocks ramp over the first 10-15 ms of "
                         "memory-bound work after idling, which a few warm-up steps do not "
                         "cover (0 disables)")
    ap.add_argument("--backward", choices=["on", "off"], default="on",
                    help="after the forward, time mita_backward (the training pass, with the "
                         "forward's experts and routes) and report it beside the metric")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also time a plain 1 GiB device copy kernel (bandwidth context and the "
                         "calibration kernel for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the MiTA forward here runs on a single MI355X "
              "(multi-GPU sharding is a design note, not a measured path); use --gpus 1",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mixture_top_sparse_amd as mts
    from mixture_top_sparse_amd.inputs import WORKLOADS, generate, to_torch

    w = WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} k={w.k} {w.dtype}")
    t0 = time.perf_counter()
    Q, K, V = generate(w)
    Qt, Kt, Vt = to_torch((Q, K, V), w.dtype, "cuda")
    del Q, K, V
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    S = args.experts_per_query
    if S == 1:
        def step():
            return mts.mita_forward(Qt, Kt, Vt, m=w.m, k=w.k, grid=w.grid, scale=w.scale)
    else:
        def step():
            out, idx, routes = mts.mita_forward_s(Qt, Kt, Vt, m=w.m, k=w.k, s=S, grid=w.grid,
                                                  scale=w.scale)
            return out, idx, routes[..., 0]

    warm = device_warmup(args.device_warmup_ms)
    # The dense-attention baseline runs first (it is part of the report, and
    # it takes the GPU out of its idle clock state before MiTA's warm-up).
    dense = None
    if args.dense == "on" or (args.dense == "auto" and w.dtype == "bf16" and w.N >= 65536):
        dense = dense_baseline(w, Qt, Kt, Vt)

    for _ in range(args.warmup):
        res = step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # the timed region: K steps, nothing else enqueued between them
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    h0 = time.perf_counter()
    for _ in range(args.steps):
        res = step()
    host_ms = (time.perf_counter() - h0) * 1e3 / args.steps  # host time to enqueue one step
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    # per-kernel durations: the same K steps again with the library's stage
    # profiler (HIP events around each stage on the stream it runs on); kept
    # out of the timed region because the extra event records add gaps
    mts.mita_profile_enable(True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        res = step()
    ev1.record()
    torch.cuda.synchronize()
    mts.mita_profile_enable(False)
    ms_profiled = ev0.elapsed_time(ev1) / args.steps
    stage_ms, calls = mts.mita_profile_read()
    tokens_heads = w.B * w.H * w.N
    value = tokens_heads / (ms_per_step * 1e-3) / 1e6
    log(f"{ms_per_step:.3f} ms/step, {value:.1f} Mtokens.heads/s "
        f"({ms_profiled:.3f} ms/step with the stage profiler on)")

    avg_stage = {k: v / max(calls, 1) for k, v in stage_ms.items() if not k.startswith("bw_")}
    sbytes = stage_bytes(w, S)
    # the dominant kernel: the slowest of the single-launch stages
    dominant = max(SINGLE_KERNEL_STAGES, key=lambda st: avg_stage.get(st, 0.0))
    ach = sbytes[dominant] / (avg_stage[dominant] * 1e-3) / 1e9
    pbytes = path_bytes(w)
    path_gbs = pbytes / (ms_per_step * 1e-3) / 1e9

    out, idx, route = res
    idx_np = idx.cpu().numpy()
    route_np = route.cpu().numpy()
    union = [int(len(np.unique(idx_np[b, h]))) for b in range(w.B) for h in range(w.H)]
    sizes = np.concatenate([np.bincount(route_np[b, h], minlength=w.m)
                            for b in range(w.B) for h in range(w.H)])

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "Mtokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian-mixture tokens; no dataset, no weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "m": w.m,
                   "k": w.k, "s": S, "grid": list(w.grid), "values": w.values, "centres": w.centres,
                   "noise": w.noise, "seed": w.seed},
        # the metric's own fraction: algorithmic bytes of the whole step over
        # the step time, against the 8 TB/s peak
        "path_roofline": {"scope": "whole step (the metric)", "algorithmic_bytes": pbytes,
                          "achieved_GBs": round(path_gbs, 1),
                          "frac": round(path_gbs / HBM_PEAK_GBS, 4)},
        # the dominant (slowest single-launch) kernel against the same peak
        "roofline": {
            "scope": "dominant kernel",
            "bound": "hbm",
            "kernel": dominant,
            "symbol": stage_kernel(dominant, w, S),
            "launch_ms": round(avg_stage[dominant], 4),
            "achieved": round(ach, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic(w.name, stage_kernel(dominant, w, S)),
            "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of this kernel from an earlier "
                              "profiler run (profiles/), carried while the kernel's sources "
                              "hash the same; null once they change",
        },
        "ms_per_step_profiled": round(ms_profiled, 4),
        "host_enqueue_ms_per_step": round(host_ms, 4),
        "stages_ms": {k: round(v, 4) for k, v in avg_stage.items()},
        "stages_GBs": {k: round(sbytes[k] / (avg_stage[k] * 1e-3) / 1e9, 1) for k in avg_stage
                       if avg_stage[k] > 0},
        "structure": {"expert_union_rows_per_head": union,
                      "bucket_size_min_med_max": [int(sizes.min()), float(np.median(sizes)),
                                                  int(sizes.max())]},
    }
    if warm is not None:
        line["device_warmup"] = warm
    if dense is not None:
        dense["speedup"] = round(dense["ms_per_step"] / ms_per_step, 2)
        log(f"MiTA speedup over dense attention: {dense['speedup']:.1f}x")
        line["dense_baseline"] = dense
    if args.backward == "on" and S == 1:
        bw = backward_bench(w, Qt, Kt, Vt, idx, route)
        bw["vs_forward"] = round(bw["ms_per_call"] / ms_per_step, 2)
        line["backward"] = bw
    if args.copy_probe:
        line["copy_probe"] = copy_probe()
    if not args.no_cpu_baseline and S == 1:
        line["cpu_baseline"] = cpu_baseline(w, Qt, Kt, Vt, out, idx, route)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

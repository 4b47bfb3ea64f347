"""GPU parity of the dense-attention baseline (through the C ABI) against the
fp64 oracle's dense attention.

Bar: the kernel rounds each softmax weight to bf16 once before the P.V
product (relative error <= 2^-9 per weight) and normalises by the fp32 sum
of the unrounded weights, so |out - exact| <= 2^-9 * max|V| plus fp32
accumulation error; the test allows 2^-9 * max|V| + 1e-4.

Every test prints the case it is about to run before touching the GPU."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from mixture_top_sparse_amd.inputs import WORKLOADS, generate, to_torch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-dense] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_top_sparse_amd as mts

    mts.lib()  # fail loudly if the library is missing


CASES = {
    # name: (workload the inputs are drawn from, B, H, N, queries checked or None = all, d)
    "one_key": ("long1d_16k", 1, 1, 1, None, 64),
    "ragged_300": ("seg_40x40", 1, 2, 300, None, 64),
    "mixture_4096": ("long1d_16k", 1, 2, 4096, None, 64),
    "iid_196_batch": ("deit_s_14x14", 2, 3, 196, None, 64),
    "len_64k_sampled": ("len_64k", 1, 1, 65536, 256, 64),
    # head dimension 128 (the pages' long-sequence throughput model width)
    "d128_one_key": ("long1d_16k", 1, 1, 1, None, 128),
    "d128_ragged_300": ("seg_40x40", 1, 2, 300, None, 128),
    "d128_mixture_4096": ("long1d_16k", 1, 2, 4096, None, 128),
    "d128_len_64k_sampled": ("len_64k", 1, 1, 65536, 256, 128),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_dense_matches_oracle(name):
    import oracle as O

    import mixture_top_sparse_amd as mts

    wname, B, H, N, nsample, d = CASES[name]
    w = WORKLOADS[wname].with_(B=B, H=H, N=N, d=d, grid=(1, N, 1, 1), k=1)
    _say(f"case {name}: inputs of {wname}, B={B} H={H} N={N} d={d} bf16")
    Q, K, V = generate(w)
    Qt, Kt, Vt = to_torch((Q, K, V), "bf16", "cuda")
    out = mts.mita_dense_attention(Qt, Kt, Vt, scale=w.scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    Qd, Kd, Vd = (t.to("cpu").to(torch.float64).numpy() for t in (Qt, Kt, Vt))
    rng = np.random.default_rng(5)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            qsel = None if nsample is None else np.sort(rng.choice(N, nsample, replace=False))
            ref = O.dense(Qd[b, h], Kd[b, h], Vd[b, h], w.scale, qsel=qsel)
            g = got[b, h] if qsel is None else got[b, h][qsel]
            tol = 2.0**-9 * np.abs(Vd[b, h]).max() + 1e-4
            err = float(np.max(np.abs(g - ref)))
            worst = max(worst, err / tol)
            assert err <= tol, f"{name} (b={b}, h={h}): max err {err:.3e} > {tol:.3e}"
    _say(f"{name}: worst error {worst:.3f} of the bound")

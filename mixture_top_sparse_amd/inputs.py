"""Seeded synthetic inputs for the MiTA forward pass.

This module only draws random numbers and converts their storage type; it
holds none of the method's arithmetic, and both the GPU path's tests and the
CPU oracle's tests take their inputs from here.

Shapes follow the workloads the pages evaluate on (their datasets are not
used; synthetic values of the same shape stand in for them):

* 14x14 patch grids with m = k = 25 (ImageNet-1K / DeiT-S in the pages'
  image-classification section);
* 32x32 and 40x40 grids with m = k = 49 (the ADE20K segmentation section);
* 1D sequences of 16K-64K tokens (the long-document and Long Range Arena
  sections) and 64K-1M tokens (the throughput figure), m = k = 64.

Value recipes:

* ``iid``: every element of Q, K, V drawn i.i.d. N(0, 1), whole tensors in the
  order Q, K, V.
* ``mixture``: per (batch, head), in batch-major then head order: centres
  C [n_c, d] ~ N(0, 1), one centre assignment per token a [N] ~ U{0..n_c-1}
  shared by Q, K and V, then Q = C[a] + s*N(0,1), K = C[a] + s*N(0,1),
  V = C[a] + s*N(0,1) (noise drawn in that order).  This gives clustered
  tokens, so that top-k selection and routing are not decided by pure noise.

Draws are fp32 from numpy's PCG64; bf16 workloads are rounded to bf16 with
torch's round-to-nearest-even conversion.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    grid: tuple[int, int, int, int]  # (gh, gw, mh, mw): token grid and landmark grid
    k: int
    values: str  # "iid" or "mixture"
    centres: int = 0
    noise: float = 0.0
    seed: int = 0

    @property
    def m(self) -> int:
        return self.grid[2] * self.grid[3]

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _line(name, B, H, N, seed, centres):
    return Workload(name, B, H, N, 64, "bf16", (1, N, 1, 64), 64, "mixture", centres, 0.5, seed)


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32_14x14", 1, 1, 196, 64, "f32", (14, 14, 5, 5), 25, "iid", seed=0),
        Workload("deit_s_14x14", 64, 6, 196, 64, "bf16", (14, 14, 5, 5), 25, "iid", seed=1),
        Workload("seg_40x40", 16, 6, 1600, 64, "bf16", (40, 40, 7, 7), 49, "mixture", 64, 0.5, 2),
        Workload("seg_32x32", 16, 6, 1024, 64, "bf16", (32, 32, 7, 7), 49, "mixture", 64, 0.5, 3),
        _line("long1d_16k", 4, 8, 16384, 4, 256),
        _line("long1d_32k", 4, 8, 32768, 5, 256),
        _line("long1d_64k", 4, 8, 65536, 6, 256),
        _line("len_64k", 1, 4, 65536, 7, 1024),
        _line("len_256k", 1, 4, 262144, 8, 1024),
        _line("len_1m", 1, 4, 1048576, 9, 1024),
    ]
}


def generate(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Draw Q, K, V as fp32 numpy arrays of shape [B, H, N, d]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.B, w.H, w.N, w.d)
    if w.values == "iid":
        Q = rng.standard_normal(shape, dtype=np.float32)
        K = rng.standard_normal(shape, dtype=np.float32)
        V = rng.standard_normal(shape, dtype=np.float32)
        return Q, K, V
    if w.values != "mixture":
        raise ValueError(f"unknown value recipe {w.values!r}")
    Q = np.empty(shape, np.float32)
    K = np.empty(shape, np.float32)
    V = np.empty(shape, np.float32)
    s = np.float32(w.noise)
    for b in range(w.B):
        for h in range(w.H):
            C = rng.standard_normal((w.centres, w.d), dtype=np.float32)
            a = rng.integers(0, w.centres, size=w.N)
            Ca = C[a]
            Q[b, h] = Ca + s * rng.standard_normal((w.N, w.d), dtype=np.float32)
            K[b, h] = Ca + s * rng.standard_normal((w.N, w.d), dtype=np.float32)
            V[b, h] = Ca + s * rng.standard_normal((w.N, w.d), dtype=np.float32)
    return Q, K, V


def generate_dout(w: Workload) -> np.ndarray:
    """The gradient of a loss with respect to the output, for the backward
    pass: [B, H, N, d] fp32, i.i.d. N(0, 1) from seed 1000 + w.seed."""
    rng = np.random.Generator(np.random.PCG64(1000 + w.seed))
    return rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)


def generate_selection(w: Workload, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Arbitrary experts and routes (not the ones the method would select):
    idx [B, H, m, k] with keys drawn uniformly, repeats across experts
    allowed, and routes [B, H, N] drawn so that a few experts get most of the
    queries and some none.  For the backward pass, which takes both as
    given."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = rng.integers(0, w.N, size=(w.B, w.H, w.m, w.k)).astype(np.int32)
    p = rng.dirichlet(np.full(w.m, 0.3), size=(w.B, w.H))
    routes = np.empty((w.B, w.H, w.N), np.int32)
    for b in range(w.B):
        for h in range(w.H):
            routes[b, h] = rng.choice(w.m, size=w.N, p=p[b, h])
    return idx, routes


def to_torch(arrs, dtype: str, device: str = "cpu"):
    """Convert fp32 numpy arrays to torch tensors of the workload's storage
    type (bf16 by round-to-nearest-even)."""
    import torch

    td = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return tuple(torch.from_numpy(a).to(td).to(device).contiguous() for a in arrs)


def exact_f64(t) -> np.ndarray:
    """The exact fp64 values of a (CPU or device) torch tensor."""
    import torch

    return t.detach().to("cpu").to(torch.float64).numpy()

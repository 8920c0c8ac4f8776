"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random matrices; it holds none of the method's
arithmetic. Both the GPU path and the oracle receive the same bytes.

Seed rule: matrix j (0-based) of workload c draws from
``numpy.random.default_rng(numpy.random.SeedSequence([c, j]))``. Normals are
drawn in fp64, scaled, then rounded once to the storage dtype (fp32 with
``astype``; bf16 through torch, round to nearest even).

The workloads stand in for Llama-3-8B gradients (no real gradients or weights
are used):

1. one 256 x 1024 fp32 N(0, 1) matrix; Polar Express table, restart at 2;
2. sixteen 1024 x 4096 fp32 N(0, 0.02^2) matrices (k/v projection shaped);
3. one Llama-3-8B layer's seven projections in bf16, N(0, 1) / sqrt(fan_in)
   with fan_in the number of input features (columns);
4. one owner rank's share of a 32-layer model over 8 owner slots: the seven
   shapes four times each (layer-major), bf16 N(0, 1), 28 matrices;
5. eight 2048 x 8192 fp32 matrices U diag(s) V^T with U, V orthonormal from
   the QR of Gaussian matrices (column signs fixed by sign(diag R)) and s
   log-uniform on [1e-6, 1]; You table, restarts at 1 and 3.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

LLAMA8B_LAYER_SHAPES: Tuple[Tuple[str, int, int], ...] = (
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 14336, 4096),
    ("up_proj", 14336, 4096),
    ("down_proj", 4096, 14336),
)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    shapes: Tuple[Tuple[int, int], ...]
    dtype: str                      # "f32" or "bf16"
    coefficients: str               # "polar_express" or "you"
    restarts: Tuple[int, ...]
    backends: Tuple[str, ...]
    labels: Tuple[str, ...] = field(default=())


WORKLOADS = {
    1: Workload(1, "single 256x1024 fp32 N(0,1)", ((256, 1024),), "f32",
                "polar_express", (2,), ("direct", "gram")),
    2: Workload(2, "16 x 1024x4096 fp32 N(0,0.02^2)", ((1024, 4096),) * 16,
                "f32", "polar_express", (2,), ("gram",)),
    3: Workload(3, "Llama-3-8B layer (7 projections) bf16",
                tuple((m, n) for _, m, n in LLAMA8B_LAYER_SHAPES), "bf16",
                "polar_express", (2,), ("gram",),
                tuple(name for name, _, _ in LLAMA8B_LAYER_SHAPES)),
    4: Workload(4, "Llama-3-8B owner share: 28 projections bf16 N(0,1)",
                tuple((m, n) for _ in range(4)
                      for _, m, n in LLAMA8B_LAYER_SHAPES), "bf16",
                "polar_express", (2,), ("gram", "direct"),
                tuple(f"layer{i}.{name}" for i in range(4)
                      for name, _, _ in LLAMA8B_LAYER_SHAPES)),
    5: Workload(5, "8 x 2048x8192 fp32 controlled spectrum", ((2048, 8192),) * 8,
                "f32", "you", (1, 3), ("gram",)),
}


def rng_for(workload: int, j: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload, j]))


def _to_storage(x64: np.ndarray, dtype: str):
    """Round once to the storage dtype. Returns a CPU torch tensor."""
    import torch
    x32 = x64.astype(np.float32)
    t = torch.from_numpy(x32)
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f16":
        return t.to(torch.float16)
    raise ValueError(dtype)


def gaussian(workload: int, j: int, m: int, n: int, scale: float = 1.0,
             dtype: str = "f32"):
    x = rng_for(workload, j).standard_normal((m, n)) * scale
    return _to_storage(x, dtype)


def controlled_spectrum(workload: int, j: int, m: int, n: int,
                        smin: float = 1e-6, smax: float = 1.0,
                        dtype: str = "f32"):
    """U diag(s) V^T with Haar-like orthonormal factors; draw order U, V, s."""
    assert m <= n
    rng = rng_for(workload, j)
    U, Ru = np.linalg.qr(rng.standard_normal((m, m)))
    U = U * np.sign(np.diag(Ru))
    V, Rv = np.linalg.qr(rng.standard_normal((n, m)))
    V = V * np.sign(np.diag(Rv))
    s = np.exp(rng.uniform(np.log(smin), np.log(smax), size=m))
    return _to_storage((U * s) @ V.T, dtype)


def matrix(workload: int, j: int):
    """Matrix j of the numbered workload, as a CPU torch tensor."""
    w = WORKLOADS[workload]
    m, n = w.shapes[j]
    if workload == 1:
        return gaussian(1, j, m, n, 1.0, w.dtype)
    if workload == 2:
        return gaussian(2, j, m, n, 0.02, w.dtype)
    if workload == 3:
        return gaussian(3, j, m, n, 1.0 / np.sqrt(n), w.dtype)
    if workload == 4:
        return gaussian(4, j, m, n, 1.0, w.dtype)
    if workload == 5:
        return controlled_spectrum(5, j, m, n, dtype=w.dtype)
    raise KeyError(workload)


def matrices(workload: int) -> List:
    return [matrix(workload, j) for j in range(len(WORKLOADS[workload].shapes))]


def small_gaussian(seed: int, m: int, n: int, dtype: str = "f32",
                   scale: float = 1.0):
    """Ad-hoc test matrix (seed stream 100 + seed, so it never collides)."""
    return gaussian(100 + seed, 0, m, n, scale, dtype)

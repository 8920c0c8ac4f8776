"""Shared helpers for the GPU tests (comparisons against fp64 references)."""

import numpy as np
import pytest
import torch

import newton_schulz_matrix_amd as nsmi


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    nsmi.library()  # raises if the HIP library is missing: no silent fallback


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def fp16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of fp16 at |x| (subnormal spacing near zero)."""
    h = np.abs(np.asarray(x, dtype=np.float64)).astype(np.float16)
    return np.spacing(h).astype(np.float64)


def assert_close_product(got, want, bound, what=""):
    """|got - want| <= one fp16 ulp of want + an accumulation bound."""
    got = np.asarray(got, np.float64)
    tol = fp16_ulp(want) + bound
    bad = np.abs(got - want) > tol
    assert not bad.any(), (
        f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; worst excess "
        f"{np.max(np.abs(got - want) - tol):.3e}")

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


def tile_errors(got, ref, tile: int = 256) -> np.ndarray:
    """Relative Frobenius error of every tile x tile block (ragged edges
    included), in the output's own orientation. The GEMM kernels write
    256 x 256 tiles of the short-side-first product; for a tall output the
    same grid is transposed, so every kernel tile is one block here."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m, n = ref.shape
    errs = []
    for i in range(0, m, tile):
        for j in range(0, n, tile):
            r = ref[i:i + tile, j:j + tile]
            g = got[i:i + tile, j:j + tile]
            nr = np.linalg.norm(r)
            errs.append(np.linalg.norm(g - r) / (nr if nr > 0 else 1.0))
    return np.array(errs)


def assert_tiles_uniform(got, ref, factor: float = 2.0, tile: int = 256, what: str = ""):
    """No tile's relative error may exceed `factor` times the whole matrix's.

    A correct fp16 implementation spreads its rounding error evenly: on every
    workload the fp16 rounding model's worst 256 x 256 tile is within 1.06x of
    its whole-matrix error. A single wrong tile (one of up to ~900) would
    barely move the whole-matrix figure but fails here."""
    e = rel_fro(got, ref)
    te = tile_errors(got, ref, tile)
    worst = int(np.argmax(te))
    assert te[worst] <= factor * e + 1e-7, (
        f"{what}: tile {worst} of {te.size} has relative error {te[worst]:.3e}, "
        f"{te[worst] / max(e, 1e-300):.2f}x the matrix's {e:.3e}")
    return e, float(te.max())

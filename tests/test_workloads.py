"""The synthetic workloads: shapes, dtypes, determinism and distributions."""

import numpy as np
import pytest
import torch

import workloads as W


def test_shapes_and_dtypes():
    assert W.WORKLOADS[1].shapes == ((256, 1024),)
    assert len(W.WORKLOADS[2].shapes) == 16
    assert [s for s in W.WORKLOADS[3].shapes] == [
        (4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
        (14336, 4096), (14336, 4096), (4096, 14336)]
    w4 = W.WORKLOADS[4]
    assert len(w4.shapes) == 28 and w4.shapes[:7] == W.WORKLOADS[3].shapes
    assert w4.dtype == "bf16" and w4.coefficients == "polar_express"
    assert W.WORKLOADS[5].restarts == (1, 3) and W.WORKLOADS[5].coefficients == "you"


def test_deterministic_and_distinct():
    a = W.matrix(1, 0)
    b = W.matrix(1, 0)
    assert a.dtype == torch.float32 and a.shape == (256, 1024)
    assert torch.equal(a, b)
    x = W.gaussian(2, 0, 64, 64, 0.02)
    y = W.gaussian(2, 1, 64, 64, 0.02)
    assert not torch.equal(x, y)
    assert abs(float(x.std()) - 0.02) < 0.002


def test_bf16_rounding():
    t = W.gaussian(3, 0, 32, 64, 1.0 / 8.0, "bf16")
    assert t.dtype == torch.bfloat16
    x32 = (np.random.default_rng(np.random.SeedSequence([3, 0]))
           .standard_normal((32, 64)) / 8.0).astype(np.float32)
    assert torch.equal(t, torch.from_numpy(x32).to(torch.bfloat16))


def test_controlled_spectrum_small():
    G = W.controlled_spectrum(99, 0, 32, 96).numpy().astype(np.float64)
    s = np.linalg.svd(G, compute_uv=False)
    assert s.max() <= 1.0 + 1e-5 and s.min() >= 1e-6 * (1 - 1e-3) - 1e-6
    assert np.all(np.diff(np.sort(s)) >= 0)

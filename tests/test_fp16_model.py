"""The fp16 rounding model is a diagnostic; these checks keep it honest.

With its rounding switched off it must reproduce the fp64 oracle up to fp32
accumulation error, and with rounding on it must stay within the error
range that fp16 storage allows on small, well-conditioned inputs.
"""

import numpy as np

from oracle import (POLAR_EXPRESS_COEFFICIENTS, YOU_COEFFICIENTS,
                    direct_newton_schulz, gram_newton_schulz)
from oracle import fp16_model


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_model_without_rounding_matches_oracle(monkeypatch):
    monkeypatch.setattr(fp16_model, "_h", lambda x: np.asarray(x, np.float32))
    G = np.random.default_rng(0).standard_normal((48, 80))
    for co in (POLAR_EXPRESS_COEFFICIENTS, YOU_COEFFICIENTS):
        for S in ((2,), (1, 3)):
            ref = gram_newton_schulz(G, co, S)
            for sym in (False, True):
                assert rel(fp16_model.gram_fp16(G, co, S, symmetric=sym), ref) < 1e-4
            assert rel(fp16_model.gram_fp16(G, co, S, literal=True), ref) < 1e-4
        ref = direct_newton_schulz(G, co)
        assert rel(fp16_model.direct_fp16(G, co), ref) < 1e-4
        assert rel(fp16_model.gram_fp16(G.T, co, (2,)), gram_newton_schulz(G.T, co)) < 1e-4


def test_model_with_rounding_is_near_oracle():
    G = np.random.default_rng(1).standard_normal((64, 192))
    ref = gram_newton_schulz(G, YOU_COEFFICIENTS, (1, 3))
    err = rel(fp16_model.gram_fp16(G, YOU_COEFFICIENTS, (1, 3)), ref)
    assert 1e-5 < err < 1e-2


def test_normalize_fp16_rounds_once():
    G = np.random.default_rng(2).standard_normal((8, 16)).astype(np.float32)
    X, nrm = fp16_model.normalize_fp16(G)
    want = (G / (np.float32(nrm) + np.float32(1e-7))).astype(np.float16)
    np.testing.assert_array_equal(X.astype(np.float16), want)


def test_literal_order_model_is_a_different_rounding_of_the_same_iteration():
    """The literal-order model evolves R through (a I + Z) R (a I + Z) with
    full products; with rounding it lands near the oracle but not on the
    mirrored model's bits, and it refuses to mirror."""
    G = np.random.default_rng(3).standard_normal((64, 192))
    ref = gram_newton_schulz(G, YOU_COEFFICIENTS, (2,))
    lit = fp16_model.gram_fp16(G, YOU_COEFFICIENTS, (2,), literal=True)
    sym = fp16_model.gram_fp16(G, YOU_COEFFICIENTS, (2,), symmetric=True)
    assert 1e-5 < rel(lit, ref) < 1e-2
    assert not np.array_equal(lit, sym)
    import pytest
    with pytest.raises(ValueError):
        fp16_model.gram_fp16(G, YOU_COEFFICIENTS, (2,), literal=True, symmetric=True)


def test_literal_order_model_catches_a_dropped_factor(monkeypatch):
    """With rounding off, a recurrence that forgets one (a I + Z) factor is
    far from the oracle: the model's R update is really exercised."""
    monkeypatch.setattr(fp16_model, "_h", lambda x: np.asarray(x, np.float32))
    G = np.random.default_rng(4).standard_normal((40, 90))
    ref = gram_newton_schulz(G, YOU_COEFFICIENTS, ())
    assert rel(fp16_model.gram_fp16(G, YOU_COEFFICIENTS, (), literal=True), ref) < 1e-4
    real_eye = np.eye
    monkeypatch.setattr(fp16_model.np, "eye", lambda n, dtype=None: 0.0 * real_eye(n))
    bad = fp16_model.gram_fp16(G, YOU_COEFFICIENTS, (), literal=True)
    monkeypatch.setattr(fp16_model.np, "eye", real_eye)
    assert rel(bad, ref) > 1e-2

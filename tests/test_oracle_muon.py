"""Pins for the oracle's Muon step (a stated reading; the pages' formula is
missing, so parity against the pages is unpinned). Pinned here is the
composition the reading defines:

* the momentum recursion M_t = beta M_{t-1} + G against its geometric closed
  form beta^t M_0 + (1 - beta^t) / (1 - beta) G;
* the update W' - W against -lr * scale times the SVD closed form of M'
  (the Gram iteration is pinned to the closed form elsewhere);
* linearity in lr * scale, beta = 0 (M' = G) and lr = 0 (W' = W);
* planted mistakes (momentum from the old M, sign of the update, update
  from G instead of M') fail one of these.
"""

import numpy as np
import pytest

from oracle import YOU_COEFFICIENTS, closed_form, muon_step


def gauss(m, n, seed, s=1.0):
    return s * np.random.default_rng(seed).standard_normal((m, n))


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_momentum_geometric_closed_form():
    G, M0, W = gauss(10, 16, 1), gauss(10, 16, 2), gauss(10, 16, 3, 0.02)
    beta, M = 0.9, M0
    for t in range(1, 6):
        M, W = muon_step(G, M, W, beta, 0.02, 1.0, YOU_COEFFICIENTS)
        want = beta ** t * M0 + (1 - beta ** t) / (1 - beta) * G
        assert rel(M, want) < 1e-13


@pytest.mark.parametrize("shape", [(12, 20), (20, 12)])
def test_update_is_the_closed_form_of_the_new_momentum(shape):
    G, M, W = gauss(*shape, 4), gauss(*shape, 5), gauss(*shape, 6, 0.02)
    M1, W1 = muon_step(G, M, W, 0.95, 0.02, 1.5, YOU_COEFFICIENTS, (2,))
    assert rel(M1, 0.95 * M + G) < 1e-15
    upd = (W1 - W) / (-0.02 * 1.5)
    assert rel(upd, closed_form(M1, YOU_COEFFICIENTS)) < 1e-9


def test_linearity_and_degenerate_cases():
    G, M, W = gauss(8, 14, 7), gauss(8, 14, 8), gauss(8, 14, 9, 0.02)
    _, W1 = muon_step(G, M, W, 0.5, 0.01, 1.0, YOU_COEFFICIENTS)
    _, W2 = muon_step(G, M, W, 0.5, 0.02, 1.5, YOU_COEFFICIENTS)
    assert rel(W2 - W, 3.0 * (W1 - W)) < 1e-12
    M0, _ = muon_step(G, M, W, 0.0, 0.02, 1.0, YOU_COEFFICIENTS)
    assert np.array_equal(M0, G)
    _, Wz = muon_step(G, M, W, 0.9, 0.0, 1.0, YOU_COEFFICIENTS)
    assert np.array_equal(Wz, W)


def _mut(G, M, W, beta, lr, scale, co, old_m=False, plus=False, from_g=False):
    M1 = beta * M + G
    src = G if from_g else (M if old_m else M1)
    O = closed_form(src, co)
    return M1, (W + lr * scale * O) if plus else (W - lr * scale * O)


@pytest.mark.parametrize("kw", [dict(old_m=True), dict(plus=True), dict(from_g=True)])
def test_pins_catch_planted_muon_mistakes(kw):
    G, M, W = gauss(12, 20, 10), gauss(12, 20, 11), gauss(12, 20, 12, 0.02)
    _, W1 = _mut(G, M, W, 0.9, 0.02, 1.0, YOU_COEFFICIENTS, **kw)
    M1 = 0.9 * M + G
    upd = (W1 - W) / (-0.02)
    assert rel(upd, closed_form(M1, YOU_COEFFICIENTS)) > 1e-3

"""Pins for the tensor-parallel route of the oracle (gram_newton_schulz_sharded).

The route follows the Newton-Schulz reference page, section "Gram 空间 NS"
(R is a sum of local Gram matrices: exact TP through one all-reduce) and the
article page, section "6. 与TP的结合" (distributed mode). It is pinned
against what the mathematics fixes, not against a retyped copy of itself:

* the SVD closed form of the whole matrix (singular values mapped by the
  composed polynomial, singular vectors kept), for every shard count from 1
  to l, tall and wide, several restart patterns;
* the unsharded oracle (itself pinned to the closed form elsewhere);
* partition properties of the column split;
* planted mistakes a sharded implementation could plausibly make (Gram of
  one shard only, a shard left out of a restart, the norm of one shard, the
  output columns out of order) each fail one of these pins.
"""

import numpy as np
import pytest

from oracle import (POLAR_EXPRESS_COEFFICIENTS, YOU_COEFFICIENTS, closed_form,
                    gram_newton_schulz, gram_newton_schulz_sharded, shard_bounds)


def gauss(m, n, seed):
    return np.random.default_rng(seed).standard_normal((m, n))


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("l,shards", [(7, 1), (7, 2), (7, 3), (7, 7), (20, 6), (64, 64), (65, 8)])
def test_shard_bounds_partition(l, shards):
    b = shard_bounds(l, shards)
    assert len(b) == shards and b[0][0] == 0 and b[-1][1] == l
    assert all(b[i][1] == b[i + 1][0] for i in range(shards - 1))
    sizes = [e - s for s, e in b]
    assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1
    assert sizes == sorted(sizes, reverse=True)      # the larger shards come first
    assert sum(1 for x in sizes if x == max(sizes)) == (l % shards or shards)


@pytest.mark.parametrize("bad", [0, 8])
def test_shard_bounds_rejects(bad):
    with pytest.raises(ValueError):
        shard_bounds(7, bad)


@pytest.mark.parametrize("shape", [(12, 20), (20, 12), (9, 9)])
@pytest.mark.parametrize("restarts", [(), (2,), (1, 3), (1, 2, 3, 4)])
def test_sharded_equals_closed_form(shape, restarts):
    G = gauss(*shape, seed=sum(shape) + len(restarts))
    l = max(shape)
    for co in (YOU_COEFFICIENTS, POLAR_EXPRESS_COEFFICIENTS):
        want = closed_form(G, co)
        for shards in (1, 2, 3, 5, l):
            got = gram_newton_schulz_sharded(G, co, restarts, shards)
            assert got.shape == G.shape
            assert rel(got, want) < 1e-9, (shards, co is YOU_COEFFICIENTS)


def test_sharded_equals_unsharded_oracle():
    for shape, shards in (((64, 200), 4), ((200, 64), 7), ((33, 100), 10)):
        G = gauss(*shape, seed=shards)
        a = gram_newton_schulz_sharded(G, YOU_COEFFICIENTS, (2,), shards)
        b = gram_newton_schulz(G, YOU_COEFFICIENTS, (2,))
        assert rel(a, b) < 1e-12


def test_one_shard_is_the_unsharded_iteration():
    G = gauss(16, 40, seed=3)
    a = gram_newton_schulz_sharded(G, YOU_COEFFICIENTS, (1, 3), 1)
    b = gram_newton_schulz(G, YOU_COEFFICIENTS, (1, 3))
    assert rel(a, b) < 1e-14


# ---------------------------------------------------------- planted mistakes

def _sharded_mut(G, co, S, shards, eps=1e-7, one_gram=False, skip_restart=False,
                 local_norm=False, reversed_out=False):
    """A copy of the sharded route with one planted mistake."""
    G = np.asarray(G, np.float64)
    t = G.shape[0] > G.shape[1]
    Xf = G.T if t else G
    parts = [Xf[:, a:b] for a, b in shard_bounds(Xf.shape[1], shards)]
    nrm = np.sqrt(np.sum(parts[0] ** 2)) if local_norm else np.sqrt(sum(np.sum(P * P) for P in parts))
    Xs = [P / (nrm + eps) for P in parts]
    I = np.eye(Xf.shape[0])
    gram = (lambda Xs: Xs[0] @ Xs[0].T) if one_gram else (lambda Xs: sum(X @ X.T for X in Xs))
    R, Q, K = gram(Xs), None, len(co)
    for k, (a, b, c) in enumerate(co):
        if k in S and Q is not None:
            Xs = [Xs[0]] + [Q @ X for X in Xs[1:]] if skip_restart else [Q @ X for X in Xs]
            R, Q = gram(Xs), None
        Z = b * R + c * R @ R
        Q = Z + a * I if Q is None else Z @ Q + a * Q
        if k + 1 < K and (k + 1) not in S:
            M = a * I + Z
            R = M @ R @ M
    outs = [Q @ X for X in Xs]
    out = np.concatenate(outs[::-1] if reversed_out else outs, axis=1)
    return out.T if t else out


@pytest.mark.parametrize("kw", [dict(one_gram=True), dict(skip_restart=True),
                                dict(local_norm=True), dict(reversed_out=True)])
def test_pins_catch_planted_sharding_mistakes(kw):
    caught = False
    for G in (gauss(12, 20, seed=5), gauss(20, 12, seed=6)):
        for co in (YOU_COEFFICIENTS, POLAR_EXPRESS_COEFFICIENTS):
            with np.errstate(all="ignore"):
                out = _sharded_mut(G, co, (2,), 3, **kw)
            if not np.all(np.isfinite(out)) or rel(out, closed_form(G, co)) > 1e-6:
                caught = True
    assert caught, kw

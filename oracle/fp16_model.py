"""fp16 rounding model of Newton-Schulz (DIAGNOSTIC, not a parity oracle).

TEST INFRASTRUCTURE ONLY. This module estimates how far *any* correct fp16
implementation of the method must sit from the fp64 oracle, so that a GPU
error can be read against the method's own rounding floor.

It follows the "Newton-Schulz 变体" page, section "精度流水线" (precision
pipeline): normalise in fp32, cast to fp16, iterate in fp16. Products are
formed in fp32 (numpy float32 matmul) and every stored matrix (X, R, Z, Q, T)
is rounded to fp16 once; scalar epilogues (b R + c R^2, + a Q, + a I) are
evaluated in fp32 before that rounding.

``symmetric=True`` models an implementation that computes only the lower
triangle of each Gram-space product (all of them are symmetric in exact
arithmetic) and mirrors it.

``literal=True`` (Gram space only) models the plainest library rendering of
the page's equations instead: every product is a full matrix product in the
shape of a general multiply or multiply-add (Z = b R + c R R, Q <- a Q + Z Q),
nothing is mirrored, and R is evolved in the form the recurrence follows
from, R <- (a I + Z) R (a I + Z), with the factor (a I + Z) stored in fp16 and
each of the two products rounded to fp16.
"""

from __future__ import annotations

import numpy as np


def _h(x: np.ndarray) -> np.ndarray:
    """Round to fp16 (round to nearest even, subnormals kept), back to fp32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def _mirror(P: np.ndarray) -> np.ndarray:
    return np.tril(P) + np.tril(P, -1).T


def normalize_fp16(G, eps: float = 1e-7):
    """fp32 Frobenius normalisation followed by the fp16 cast."""
    G32 = np.asarray(G, dtype=np.float32)
    norm = np.float32(np.sqrt(np.sum(G32.astype(np.float64) ** 2)))
    return _h(G32 / (norm + np.float32(eps))), float(norm)


def direct_fp16(G, coefficients, eps: float = 1e-7, symmetric: bool = False,
                out_fp32: bool = False) -> np.ndarray:
    X, _ = normalize_fp16(G, eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.copy()
    f = _mirror if symmetric else (lambda P: P)
    K = len(coefficients)
    for k, (a, b, c) in enumerate(coefficients):
        A = _h(f(X @ X.T))
        B = _h(f(np.float32(b) * A + np.float32(c) * (A @ A)))
        Xn = np.float32(a) * X + B @ X
        X = Xn if (out_fp32 and k == K - 1) else _h(Xn)
    return X.T.copy() if tall else X


def gram_fp16(G, coefficients, restart_iterations=(2,), eps: float = 1e-7,
              symmetric: bool = False, out_fp32: bool = False,
              literal: bool = False) -> np.ndarray:
    if literal:
        if symmetric:
            raise ValueError("the literal-order model mirrors nothing")
        return _gram_fp16_literal(G, coefficients, restart_iterations, eps, out_fp32)
    X, _ = normalize_fp16(G, eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.copy()
    f = _mirror if symmetric else (lambda P: P)
    K = len(coefficients)
    S = set(int(i) for i in restart_iterations)
    eye = np.eye(X.shape[0], dtype=np.float32)
    R = _h(f(X @ X.T))
    Q = None
    for k, (a, b, c) in enumerate(coefficients):
        a, b, c = np.float32(a), np.float32(b), np.float32(c)
        if k in S and Q is not None:
            X = _h(Q @ X)
            R = _h(f(X @ X.T))
            Q = None
        z = f(b * R + c * (R @ R))
        Z = _h(z)
        if Q is None:
            Q = _h(z + a * eye)
        else:
            Q = _h(f(Z @ Q + a * Q))
        if k + 1 < K and (k + 1) not in S:
            T = _h(f(Z @ R + a * R))
            R = _h(f(T @ Z + a * T))
    out = Q @ X
    if not out_fp32:
        out = _h(out)
    return out.T.copy() if tall else out


def _gram_fp16_literal(G, coefficients, restart_iterations, eps, out_fp32):
    """Gram-space iteration in the order the page writes it (see module doc)."""
    X, _ = normalize_fp16(G, eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T.copy()
    K = len(coefficients)
    S = set(int(i) for i in restart_iterations)
    eye = np.eye(X.shape[0], dtype=np.float32)
    R = _h(X @ X.T)
    Q = None
    for k, (a, b, c) in enumerate(coefficients):
        a, b, c = np.float32(a), np.float32(b), np.float32(c)
        if k in S and Q is not None:
            X = _h(Q @ X)
            R = _h(X @ X.T)
            Q = None
        Z = _h(b * R + c * (R @ R))
        Q = _h(Z + a * eye) if Q is None else _h(a * Q + Z @ Q)
        if k + 1 < K and (k + 1) not in S:
            M = _h(a * eye + Z)
            R = _h(_h(M @ R) @ M)
    out = Q @ X
    if not out_fp32:
        out = _h(out)
    return out.T.copy() if tall else out

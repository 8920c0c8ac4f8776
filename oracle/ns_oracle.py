"""fp64 reference implementation of Newton-Schulz orthogonalisation.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark; never by the GPU library.

Everything here is plain numpy in float64, written from the DMuon
documentation page "Newton-Schulz 变体" (Newton-Schulz variants):

* section "精度流水线" (precision pipeline), step 1: the input is divided by
  its norm plus eps before iterating (``normalize``). Step 2 (the fp16 cast)
  is *not* applied here: the oracle iterates in fp64 so that it gives the
  exact-arithmetic result the fp16 implementation approximates.
* section "直接空间 NS（经典）" (direct space): the update
  X_{k+1} = a_k X_k + b_k (X_k X_k^T) X_k + c_k (X_k X_k^T)^2 X_k on the full
  matrix (``direct_newton_schulz``). The same update is the equation in
  section 1 ("Dedicated Ownership") of the "Core Concepts" page.
* section "Gram 空间 NS（Dao-AILab）", equations Z_k and Q_{k+1}: iterate on
  R = X X^T, with Z_k = b_k R_k + c_k R_k^2 and the accumulated product
  Q_{k+1} = Z_k Q_k + a_k Q_k, R evolved from R_k and Z_k, output Q X
  (``gram_newton_schulz``).
* section "重启机制" (restart mechanism): at the listed step indices Q is
  applied to X and R is recomputed from X.
* section "系数集" (coefficient sets): the two 5-step tables.

Readings taken where the page is silent (each is listed in the design notes):

* the norm is the Frobenius norm of the whole matrix, eps is added to the
  norm (not to its square), default eps = 1e-7;
* a matrix with more rows than columns is transposed first so the Gram
  matrix is formed on the short side, for both backends, and the result is
  transposed back;
* step k uses row k of the table (row 0 first);
* a restart before step i sets X <- Q X, R <- X X^T and Q <- I; a restart at
  step 0 is a no-op; restart indices are ignored by the direct backend;
* the R recurrence is R_{k+1} = (a_k I + Z_k) R_k (a_k I + Z_k), which follows
  from X_{k+1} = (a_k I + Z_k) X_k; it is skipped when R_{k+1} is not used
  (after the last step, or when step k+1 restarts).

``gram_newton_schulz_sharded`` takes the tensor-parallel route of the same
iteration (X split by columns, R as the sum of per-shard Gram matrices,
per-shard restarts and outputs): the pages' exact-TP statement in section
"Gram 空间 NS", and section "6. 与TP的结合" of the distributed-Muon article.

``muon_step`` composes the momentum update, the Gram iteration and the
parameter update along a stated reading of the article page's description
(its formula is missing from the pages): parity unpinned as to the pages.

Parity pins (tests/test_oracle_pins.py): gram == direct in fp64, the SVD
closed form ``closed_form`` (singular values mapped by the composed scalar
polynomial, singular vectors kept), restart invariance, and special cases
with known answers (diagonal, scaled identity, rank one, zero).
"""

from __future__ import annotations

import numpy as np

# Section "系数集": the Polar Express table as the page prints it (rounded to
# three decimals, with the page's 1.05 safety factor already applied). The
# numbers are used exactly as printed.
POLAR_EXPRESS_COEFFICIENTS = (
    (7.893, -20.381, 14.939),
    (3.912, -2.544, 0.470),
    (3.761, -2.512, 0.476),
    (3.160, -2.148, 0.440),
    (2.191, -1.441, 0.361),
)

# Section "系数集": the table credited to @YouJiacheng, as printed.
YOU_COEFFICIENTS = (
    (4.0848, -6.8946, 2.9270),
    (3.9505, -6.3029, 2.6377),
    (3.7418, -5.5913, 2.3037),
    (2.8769, -3.1427, 1.2046),
    (2.8366, -3.0525, 1.2012),
)

COEFFICIENT_SETS = {
    "polar_express": POLAR_EXPRESS_COEFFICIENTS,
    "you": YOU_COEFFICIENTS,
}

DEFAULT_EPS = 1e-7
DEFAULT_RESTARTS = (2,)


def _as_f64(G) -> np.ndarray:
    G = np.asarray(G, dtype=np.float64)
    if G.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    return G


def normalize(G, eps: float = DEFAULT_EPS):
    """Precision pipeline, step 1: X = G / (||G||_F + eps), in fp64.

    Returns ``(X, norm)`` with ``norm`` the Frobenius norm of G.
    """
    G = _as_f64(G)
    norm = float(np.sqrt(np.sum(G * G)))
    return G / (norm + eps), norm


def _short_side(X: np.ndarray):
    """Put the short side first (transposing a tall matrix)."""
    if X.shape[0] > X.shape[1]:
        return X.T.copy(), True
    return X, False


def direct_newton_schulz(G, coefficients=POLAR_EXPRESS_COEFFICIENTS,
                         eps: float = DEFAULT_EPS) -> np.ndarray:
    """Direct-space NS: X <- a X + b (X X^T) X + c (X X^T)^2 X per step."""
    X, _ = normalize(G, eps)
    X, transposed = _short_side(X)
    for a, b, c in coefficients:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T.copy() if transposed else X


def gram_newton_schulz(G, coefficients=POLAR_EXPRESS_COEFFICIENTS,
                       restart_iterations=DEFAULT_RESTARTS,
                       eps: float = DEFAULT_EPS) -> np.ndarray:
    """Gram-space NS with accumulated product Q and restarts; output Q X."""
    X, _ = normalize(G, eps)
    X, transposed = _short_side(X)
    K = len(coefficients)
    restarts = set(int(i) for i in restart_iterations)
    if any(i < 0 or i >= K for i in restarts):
        raise ValueError("restart index out of range")
    eye = np.eye(X.shape[0])

    R = X @ X.T
    Q = None  # None stands for the identity: nothing accumulated yet
    for k, (a, b, c) in enumerate(coefficients):
        if k in restarts and Q is not None:
            # restart: apply the accumulated product, rebuild R from X
            X = Q @ X
            R = X @ X.T
            Q = None
        Z = b * R + c * (R @ R)
        # Q_{k+1} = Z_k Q_k + a_k Q_k; with Q_k = I this is Z_k + a_k I
        Q = Z + a * eye if Q is None else Z @ Q + a * Q
        if k + 1 < K and (k + 1) not in restarts:
            M = a * eye + Z
            R = M @ R @ M
    out = Q @ X
    return out.T.copy() if transposed else out


def shard_bounds(l: int, shards: int):
    """Column blocks of the short-side-first X for `shards` shards.

    Shard i holds l // shards columns, one more for i < l % shards (the
    plainest balanced split; the pages fix no split).
    """
    if shards < 1 or shards > l:
        raise ValueError("need 1 <= shards <= l")
    bounds, c0 = [], 0
    for i in range(shards):
        lc = l // shards + (1 if i < l % shards else 0)
        bounds.append((c0, c0 + lc))
        c0 += lc
    return bounds


def gram_newton_schulz_sharded(G, coefficients=POLAR_EXPRESS_COEFFICIENTS,
                               restart_iterations=DEFAULT_RESTARTS, shards: int = 2,
                               eps: float = DEFAULT_EPS) -> np.ndarray:
    """Gram-space NS along the tensor-parallel route, shard by shard.

    Follows the Newton-Schulz reference page, section "Gram 空间 NS" (R is a
    sum of local Gram matrices, so TP is exact through one all-reduce), and
    the article page, section "6. 与TP的结合" (distributed mode: the norm
    from a scalar all-reduce of per-shard sums of squares; one Gram
    all-reduce whenever X changes). X is split by columns into X_1..X_T;
    every "all-reduce" is a plain sum over shards; the s x s iteration is
    the unsharded one; each shard applies Q to its own columns.
    """
    G = _as_f64(G)
    transposed = G.shape[0] > G.shape[1]
    Xfull = G.T if transposed else G
    blocks = shard_bounds(Xfull.shape[1], shards)
    parts = [Xfull[:, a:b] for a, b in blocks]
    # scalar all-reduce of the per-shard sums of squares
    norm = float(np.sqrt(sum(float(np.sum(P * P)) for P in parts)))
    Xs = [P / (norm + eps) for P in parts]
    K = len(coefficients)
    restarts = set(int(i) for i in restart_iterations)
    if any(i < 0 or i >= K for i in restarts):
        raise ValueError("restart index out of range")
    eye = np.eye(Xfull.shape[0])

    def gram(Xs):   # all-reduce of the local Gram matrices
        return sum(Xi @ Xi.T for Xi in Xs)

    R = gram(Xs)
    Q = None
    for k, (a, b, c) in enumerate(coefficients):
        if k in restarts and Q is not None:
            Xs = [Q @ Xi for Xi in Xs]
            R = gram(Xs)
            Q = None
        Z = b * R + c * (R @ R)
        Q = Z + a * eye if Q is None else Z @ Q + a * Q
        if k + 1 < K and (k + 1) not in restarts:
            M = a * eye + Z
            R = M @ R @ M
    out = np.concatenate([Q @ Xi for Xi in Xs], axis=1)
    return out.T.copy() if transposed else out


def muon_step(G, M, W, beta: float, lr: float, scale: float = 1.0,
              coefficients=POLAR_EXPRESS_COEFFICIENTS,
              restart_iterations=DEFAULT_RESTARTS, eps: float = DEFAULT_EPS):
    """One Muon step around the Gram iteration, in fp64: returns (M', W').

    PARITY UNPINNED against the pages: the article page (sections
    "1. Introduction" and "2. Muon执行过程") says only that a Muon step keeps
    a momentum M of the gradient, orthogonalises M and uses the result as
    the update direction; the formula itself is missing from the extracted
    text and no beta or update scale is given (lr = 0.02 appears in an
    example). This function is the plainest reading of that description:

        M' = beta M + G,    W' = W - lr * scale * gram_newton_schulz(M').

    What is pinned (tests/test_oracle_muon.py) is this composition: the
    momentum recursion against its geometric closed form, the update
    against the SVD closed form of M', and linearity in lr * scale.
    """
    G, M, W = _as_f64(G), _as_f64(M), _as_f64(W)
    M_new = beta * M + G
    O = gram_newton_schulz(M_new, coefficients, restart_iterations, eps)
    return M_new, W - (lr * scale) * O


def step_maps(coefficients):
    """The per-step scalar polynomials p_k(s) = a_k s + b_k s^3 + c_k s^5."""
    return [(lambda s, a=a, b=b, c=c: a * s + b * s ** 3 + c * s ** 5)
            for a, b, c in coefficients]


def scalar_map(coefficients, s):
    """Composed map p = p_{K-1} o ... o p_0 applied to singular values s."""
    s = np.asarray(s, dtype=np.float64)
    for p in step_maps(coefficients):
        s = p(s)
    return s


def closed_form(G, coefficients=POLAR_EXPRESS_COEFFICIENTS,
                eps: float = DEFAULT_EPS) -> np.ndarray:
    """U diag(p(sigma / (||G||_F + eps))) V^T from the thin SVD of G.

    Each NS step maps X = U S V^T to U p_k(S) V^T because
    X X^T X = U S^3 V^T, so the whole iteration acts on singular values
    through the composed polynomial and keeps the singular vectors.
    """
    G = _as_f64(G)
    norm = float(np.sqrt(np.sum(G * G)))
    U, sig, Vt = np.linalg.svd(G, full_matrices=False)
    return (U * scalar_map(coefficients, sig / (norm + eps))) @ Vt

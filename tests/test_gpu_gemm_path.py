"""The grouped GEMM kernel on the paths the iteration's stages take,
elementwise against fp64 products of the same fp16 operands.

ns_gemm_grouped exposes every descriptor option the stage planner uses: the
row-pair layout of internal buffers, beta * C folded from the B slices
(C == B^T), the second output D2 = D + delta I of the first Z product after a
start or restart, the transposed second output DT of the restart product,
symmetric (lower-tile + mirror) mode, the clipped, typed epilogue that
writes a caller's buffer, and K-major operands (X read as the right operand
of Q X, or as the left operand of X^T Q, from its own row-pair buffer). Each
launch holds more than 256 tiles, so the dealing of tiles to the XCDs and
the banded tile walks (several bands of tile rows, lower-triangle bands for
symmetric products) are all exercised; the launches of 896 tiles and more
also have a claimed tail pool, and the K-major launch two K classes (two
deal segments). Shapes
are the Llama-3-8B owner batch's: SYRK 4096 x 14336, symmetric 4096^3 Gram-
space products, Q X with Q 4096^2 and X 4096 x 14336, plus a ragged
caller-buffer tail.

Bound per element (products accumulate in fp32, rounded once):
|got - want| <= ulp(want) + (K + 4) 2^-24 (|alpha| |A||B|^T + |beta| |C| + |gamma|).
"""

import numpy as np
import pytest
import torch

import newton_schulz_matrix_amd as nsmi
from gpu_helpers import fp16_ulp, require_gpu, to64

pytestmark = pytest.mark.gpu


def to_pairs(X: torch.Tensor) -> torch.Tensor:
    """Row-pair layout: element (i, j) at (i/2) 2C + (j/32) 64 + (i%2) 32 + j%32."""
    R, C = X.shape
    return X.reshape(R // 2, 2, C // 32, 32).permute(0, 2, 1, 3).contiguous().reshape(R, C)


def from_pairs(Y: torch.Tensor) -> torch.Tensor:
    R, C = Y.shape
    return Y.reshape(R // 2, C // 32, 2, 32).permute(0, 2, 1, 3).contiguous().reshape(R, C)


def rand16(shape, scale, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).half()


def sym16(n, seed):
    """A symmetric fp16 matrix with entries ~ 1/sqrt(n) (a Gram-like R)."""
    A = torch.randn((n, n), generator=torch.Generator(device="cuda").manual_seed(seed),
                    device="cuda") / np.sqrt(2.0 * n)
    return (A + A.T).half()


def ulp_of(want, dtype):
    if dtype == torch.float16:
        return fp16_ulp(want)
    a = np.abs(want)
    if dtype == torch.bfloat16:
        return np.maximum(a, 2.0 ** -133) * 2.0 ** -7
    return np.maximum(a, 2.0 ** -149) * 2.0 ** -23


def assert_bound(got, want, bound, dtype, what):
    tol = ulp_of(want, dtype) + bound
    excess = np.abs(got - want) - tol
    bad = excess > 0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements out of bound; "
                           f"worst excess {excess.max():.3e} at "
                           f"{np.unravel_index(int(np.argmax(excess)), excess.shape)}")


def acc_bound(K, alpha, A64, B64, beta=0.0, C64=None, gamma=0.0):
    b = abs(alpha) * (np.abs(A64) @ np.abs(B64).T)
    if C64 is not None:
        b = b + abs(beta) * np.abs(C64)
    return (K + 4) * 2.0 ** -24 * (b + abs(gamma))


def test_syrk_pairs_two_problems():
    """R = X X^T for two 4096 x 14336 matrices in one launch (272 tiles)."""
    require_gpu()
    print("syrk 2 x 4096x14336 pairs", flush=True)
    Xs = [rand16((4096, 14336), 1.0 / np.sqrt(14336), s) for s in (1, 2)]
    Ds = [torch.empty((4096, 4096), dtype=torch.float16, device="cuda") for _ in Xs]
    Ps = [to_pairs(X) for X in Xs]   # A and B the same buffer, as in the plan
    nsmi.ns_gemm_grouped([dict(a=P, b=P, d=D, M=4096, N=4096, K=14336, symmetric=1,
                               a_pairs=1, b_pairs=1, d_pairs=1) for P, D in zip(Ps, Ds)])
    torch.cuda.synchronize()
    for X, D in zip(Xs, Ds):
        R = from_pairs(D)
        assert torch.equal(R, R.T)
        X64 = to64(X)
        want = X64 @ X64.T
        assert_bound(to64(R), want, acc_bound(14336, 1.0, X64, X64), torch.float16, "syrk")


def test_symmetric_z_products_fold_d2_gamma():
    """Z = c R R + b R (b R folded from the B slices) with D2 = Z + a I on the
    real diagonal (diag_n < 4096), and a second product R2 R2 + 0.5 R2 + 0.3 I,
    in one launch (272 tiles)."""
    require_gpu()
    print("symmetric 4096^3 fold + D2", flush=True)
    R1, R2 = sym16(4096, 3), sym16(4096, 4)
    P1, P2 = to_pairs(R1), to_pairs(R2)
    Z = torch.empty_like(R1)
    Q = torch.empty_like(R1)
    Z2 = torch.empty_like(R1)
    a, b, c, diag_n = 3.912, -2.544, 0.470, 4000
    nsmi.ns_gemm_grouped([
        dict(a=P1, b=P1, c=P1, d=Z, d2=Q, M=4096, N=4096, K=4096, symmetric=1, c_is_bt=1,
             a_pairs=1, b_pairs=1, c_pairs=1, d_pairs=1, alpha=c, beta=b, delta=a,
             diag_n=diag_n),
        dict(a=P2, b=P2, c=P2, d=Z2, M=4096, N=4096, K=4096, symmetric=1, c_is_bt=1,
             a_pairs=1, b_pairs=1, c_pairs=1, d_pairs=1, alpha=1.0, beta=0.5, gamma=0.3,
             diag_n=4096),
    ])
    torch.cuda.synchronize()
    R64 = to64(R1)
    want = c * (R64 @ R64) + b * R64
    bound = acc_bound(4096, c, R64, R64, b, R64)
    z = from_pairs(Z)
    q = from_pairs(Q)
    assert torch.equal(z, z.T) and torch.equal(q, q.T)
    assert_bound(to64(z), want, bound, torch.float16, "Z")
    eye = np.zeros((4096, 4096))
    eye[np.arange(diag_n), np.arange(diag_n)] = 1.0
    assert_bound(to64(q), want + a * eye, bound + 2.0 ** -24 * abs(a), torch.float16, "Z + aI")
    # off the real diagonal the two outputs are the same bits
    off = torch.ones((4096, 4096), dtype=torch.bool, device="cuda")
    off[torch.arange(diag_n), torch.arange(diag_n)] = False
    assert torch.equal(z[off], q[off])
    S64 = to64(R2)
    want2 = S64 @ S64 + 0.5 * S64 + 0.3 * np.eye(4096)
    z2 = from_pairs(Z2)
    assert torch.equal(z2, z2.T)
    assert_bound(to64(z2), want2, acc_bound(4096, 1.0, S64, S64, 0.5, S64, 0.3),
                 torch.float16, "R2 R2 + 0.5 R2 + 0.3 I")


def test_symmetric_with_c_read_in_the_epilogue():
    """R <- T Z + a T: C = T read in the epilogue (not folded), all symmetric,
    grouped with a SYRK of a different K so the launch mixes problem sizes."""
    require_gpu()
    Tm, Zm = sym16(2048, 5), sym16(2048, 6)
    X = rand16((2048, 8192), 1.0 / np.sqrt(8192), 7)
    D = torch.empty_like(Tm)
    R = torch.empty_like(Tm)
    a = 2.191
    Xp = to_pairs(X)
    nsmi.ns_gemm_grouped([
        dict(a=to_pairs(Tm), b=to_pairs(Zm), c=to_pairs(Tm), d=D, M=2048, N=2048, K=2048,
             symmetric=1, a_pairs=1, b_pairs=1, c_pairs=1, d_pairs=1, alpha=1.0, beta=a),
        dict(a=Xp, b=Xp, d=R, M=2048, N=2048, K=8192, symmetric=1, a_pairs=1, b_pairs=1,
             d_pairs=1),
    ])
    torch.cuda.synchronize()
    T64, Z64 = to64(Tm), to64(Zm)
    d = from_pairs(D)
    assert torch.equal(d, d.T)
    # symmetric mode computes the lower triangle of T Z + a T and mirrors it:
    # compare the lower triangle with the product, the upper with its mirror
    want = T64 @ Z64 + a * T64
    low = np.tril(want) + np.tril(want, -1).T
    lowb = acc_bound(2048, 1.0, T64, Z64, a, T64)
    lowb = np.tril(lowb) + np.tril(lowb, -1).T
    assert_bound(to64(d), low, lowb, torch.float16, "T Z + a T")
    X64 = to64(X)
    r = from_pairs(R)
    assert_bound(to64(r), X64 @ X64.T, acc_bound(8192, 1.0, X64, X64), torch.float16, "syrk")


def test_qx_with_transposed_output_and_fold():
    """X' = B X + a X (the direct step, C = X = (X^T)^T folded) with the
    transposed second output, Q 4096^2 and X 4096 x 14336 (896 tiles)."""
    require_gpu()
    print("QX 4096 x 4096 x 14336 + DT", flush=True)
    Qm = rand16((4096, 4096), 1.0 / np.sqrt(4096), 8)
    X = rand16((4096, 14336), 1.0 / np.sqrt(14336), 9)
    XT = X.T.contiguous()
    D = torch.empty((4096, 14336), dtype=torch.float16, device="cuda")
    DT = torch.empty((14336, 4096), dtype=torch.float16, device="cuda")
    a = 2.8366
    nsmi.ns_gemm_grouped([dict(a=to_pairs(Qm), b=to_pairs(XT), c=to_pairs(X), d=D, dt=DT,
                               M=4096, N=14336, K=4096, c_is_bt=1, a_pairs=1, b_pairs=1,
                               c_pairs=1, d_pairs=1, alpha=1.0, beta=a)])
    torch.cuda.synchronize()
    d = from_pairs(D)
    assert torch.equal(from_pairs(DT), d.T)
    Q64, X64 = to64(Qm), to64(X)
    want = Q64 @ X64 + a * X64
    assert_bound(to64(d), want, acc_bound(4096, 1.0, Q64, X64.T, a, X64), torch.float16,
                 "Q X + a X")


def test_kmajor_operands():
    """The Gram iteration's products by X without X^T: Q X with X read as a
    K-major right operand (Q 4096^2, X 4096 x 14336, fp16 row-pair output,
    896 tiles), and in the same launch X2^T Q2 with X2 (1024 x 8192) read as
    a K-major left operand into a caller's bf16 buffer, clipped, with an fp32
    C read in the epilogue and a negative alpha (the Muon update's form)."""
    require_gpu()
    print("K-major QX 4096 x 4096 x 14336 + X^T Q 8192 x 1024 x 1024", flush=True)
    Qm = rand16((4096, 4096), 1.0 / np.sqrt(4096), 30)
    X = rand16((4096, 14336), 1.0, 31)
    D = torch.empty((4096, 14336), dtype=torch.float16, device="cuda")
    Q2 = rand16((1024, 1024), 1.0 / np.sqrt(1024), 32)
    X2 = rand16((1024, 8192), 1.0, 33)
    vm, vn, ldd = 8000, 1000, 1001
    W = torch.randn((vm, ldd), device="cuda")
    Dt = torch.full((vm, ldd), 7.0, dtype=torch.bfloat16, device="cuda")
    alpha = -0.02
    nsmi.ns_gemm_grouped([
        dict(a=to_pairs(Qm), b=to_pairs(X), d=D, M=4096, N=14336, K=4096, a_pairs=1, b_pairs=1,
             d_pairs=1, b_kmajor=1),
        dict(a=to_pairs(X2), b=to_pairs(Q2), c=W, d=Dt, M=8192, N=1024, K=1024, ldc=ldd,
             ldd=ldd, valid_m=vm, valid_n=vn, a_pairs=1, b_pairs=1, a_kmajor=1, alpha=alpha,
             beta=1.0),
    ])
    torch.cuda.synchronize()
    Q64, X64 = to64(Qm), to64(X)
    assert_bound(to64(from_pairs(D)), Q64 @ X64, acc_bound(4096, 1.0, Q64, X64.T),
                 torch.float16, "Q X, X K-major")
    A64, B64 = to64(X2).T[:vm], to64(Q2)[:vn]
    C64 = to64(W)[:, :vn]
    got = to64(Dt)
    assert_bound(got[:, :vn], alpha * (A64 @ B64.T) + C64,
                 acc_bound(1024, alpha, A64, B64, 1.0, C64), torch.bfloat16,
                 "X^T Q, X K-major, clipped")
    assert np.all(got[:, vn:] == 7.0)


@pytest.mark.parametrize("d_dtype,c_dtype", [(torch.bfloat16, torch.float32),
                                             (torch.float32, torch.bfloat16),
                                             (torch.float16, torch.float16)])
def test_clipped_caller_buffers(d_dtype, c_dtype):
    """The final product's epilogue writing a caller's row-major buffer:
    ragged valid block, leading dimensions above the width, C of any type
    read only inside the block, stores outside the block never happen. Two
    problems (wide and tall) and a 4096-square SYRK share the launch."""
    require_gpu()
    A = rand16((512, 384), 1.0 / np.sqrt(384), 10)
    B = rand16((768, 384), 1.0, 11)
    A2 = rand16((768, 384), 1.0 / np.sqrt(384), 12)
    B2 = rand16((512, 384), 1.0, 13)
    X = rand16((4096, 1024), 1.0 / np.sqrt(1024), 14)
    ldc, ldd = 701, 703
    Cbig = (torch.randn((300, ldc), device="cuda")).to(c_dtype)
    Dbig = torch.full((300, ldd), 7.0, dtype=d_dtype, device="cuda")
    C2 = (torch.randn((700, 300), device="cuda")).to(c_dtype)
    D2big = torch.full((700, 300), 7.0, dtype=d_dtype, device="cuda")
    R = torch.empty((4096, 4096), dtype=torch.float16, device="cuda")
    alpha, beta, gamma = 0.7, -1.3, 0.25
    Xp = to_pairs(X)
    nsmi.ns_gemm_grouped([
        dict(a=A, b=B, c=Cbig, d=Dbig, M=512, N=768, K=384, ldc=ldc, ldd=ldd, valid_m=300,
             valid_n=700, diag_n=300, alpha=alpha, beta=beta, gamma=gamma),
        dict(a=A2, b=B2, c=C2, d=D2big, M=768, N=512, K=384, ldc=300, ldd=300, valid_m=700,
             valid_n=300, diag_n=300, alpha=alpha, beta=beta, gamma=gamma),
        dict(a=Xp, b=Xp, d=R, M=4096, N=4096, K=1024, symmetric=1, a_pairs=1, b_pairs=1,
             d_pairs=1),
    ])
    torch.cuda.synchronize()
    for (Am, Bm, C, D, m, n) in ((A, B, Cbig, Dbig, 300, 700), (A2, B2, C2, D2big, 700, 300)):
        A64, B64 = to64(Am)[:m], to64(Bm)[:n]
        C64 = to64(C)[:m, :n]
        eye = np.zeros((m, n))
        k = min(m, n, 300)
        eye[np.arange(k), np.arange(k)] = 1.0
        want = alpha * (A64 @ B64.T) + beta * C64 + gamma * eye
        got = to64(D)
        assert_bound(got[:m, :n], want, acc_bound(384, alpha, A64, B64, beta, C64, gamma),
                     d_dtype, f"clipped {m}x{n}")
        assert np.all(got[:, n:] == 7.0)      # columns past the block untouched
    X64 = to64(X)
    assert_bound(to64(from_pairs(R)), X64 @ X64.T, acc_bound(1024, 1.0, X64, X64),
                 torch.float16, "syrk 4096x1024")


def _path_problems(seed):
    """One problem per epilogue path, at sizes both kernels tile: symmetric
    with fold and D2, symmetric with C read in the epilogue, SYRK, full with
    fold and the transposed output, clipped caller buffers of each type
    combination, and both K-major operand forms (Q X into a row-pair buffer,
    X^T Q into a clipped caller buffer with C)."""
    S = sym16(512, seed)
    T = sym16(512, seed + 1)
    X = rand16((512, 1024), 1.0 / 32, seed + 2)
    Q = rand16((512, 512), 1.0 / 22, seed + 3)
    A = rand16((512, 384), 1.0 / 20, seed + 4)
    Bm = rand16((768, 384), 1.0, seed + 5)
    C32 = torch.randn((300, 701), device="cuda")
    Cbf = torch.randn((300, 701), device="cuda").to(torch.bfloat16)
    Sp, Tp, Xp = to_pairs(S), to_pairs(T), to_pairs(X)

    def outs():
        e = lambda *sh, dt=torch.float16: torch.full(sh, 5.0, dtype=dt, device="cuda")
        return dict(z=e(512, 512), q=e(512, 512), r=e(512, 512), syrk=e(512, 512),
                    x=e(512, 1024), xt=e(1024, 512), cl1=e(300, 703, dt=torch.bfloat16),
                    cl2=e(300, 703, dt=torch.float32), cl3=e(300, 703),
                    kx=e(512, 1024), kt=e(1000, 703, dt=torch.bfloat16))
    def probs(o):
        return [
            dict(a=Sp, b=Sp, c=Sp, d=o["z"], d2=o["q"], M=512, N=512, K=512, symmetric=1,
                 c_is_bt=1, a_pairs=1, b_pairs=1, c_pairs=1, d_pairs=1, alpha=0.47, beta=-2.5,
                 delta=3.9, diag_n=500),
            dict(a=Tp, b=Sp, c=Tp, d=o["r"], M=512, N=512, K=512, symmetric=1, a_pairs=1,
                 b_pairs=1, c_pairs=1, d_pairs=1, alpha=1.0, beta=2.19, gamma=0.5,
                 diag_n=511),
            dict(a=Xp, b=Xp, d=o["syrk"], M=512, N=512, K=1024, symmetric=1, a_pairs=1,
                 b_pairs=1, d_pairs=1),
            dict(a=to_pairs(Q), b=to_pairs(X.T.contiguous()), c=Xp, d=o["x"], dt=o["xt"],
                 M=512, N=1024, K=512, c_is_bt=1, a_pairs=1, b_pairs=1, c_pairs=1, d_pairs=1,
                 alpha=1.0, beta=2.87),
            dict(a=A, b=Bm, c=C32, d=o["cl1"], M=512, N=768, K=384, ldc=701, ldd=703,
                 valid_m=300, valid_n=700, diag_n=300, alpha=0.7, beta=-1.3, gamma=0.25),
            dict(a=A, b=Bm, c=Cbf, d=o["cl2"], M=512, N=768, K=384, ldc=701, ldd=703,
                 valid_m=300, valid_n=700, diag_n=300, alpha=-0.02, beta=1.0),
            dict(a=A, b=Bm, d=o["cl3"], M=512, N=768, K=384, ldd=703, valid_m=300,
                 valid_n=700, diag_n=0, alpha=1.0),
            dict(a=to_pairs(Q), b=Xp, d=o["kx"], M=512, N=1024, K=512, a_pairs=1, b_pairs=1,
                 d_pairs=1, b_kmajor=1),
            dict(a=Xp, b=to_pairs(Q), c=C32, d=o["kt"], M=1024, N=512, K=512, ldc=701, ldd=703,
                 valid_m=300, valid_n=500, a_pairs=1, b_pairs=1, a_kmajor=1, alpha=-0.02,
                 beta=1.0),
        ]
    return outs, probs


@pytest.mark.parametrize("seed", [21, 22])
def test_small_tile_kernel_gives_the_same_bits(seed):
    """The 64 x 64 tile kernel (used for stages with few 256-tiles, e.g. a
    single small matrix) against the 256 x 256 tile kernel on every epilogue
    path: the same MFMA over the same k steps, the same fold point and the
    same epilogue arithmetic, so every output must be bitwise equal, and
    untouched where neither may write."""
    require_gpu()
    outs, probs = _path_problems(seed)
    big, small = outs(), outs()
    nsmi.ns_gemm_grouped(probs(big), tile_edge=256)
    nsmi.ns_gemm_grouped(probs(small), tile_edge=64)
    torch.cuda.synchronize()
    for k in big:
        assert torch.equal(big[k], small[k]), k
    for k in ("cl1", "cl2", "cl3"):
        assert torch.all(big[k][:, 700:].float() == 5.0), k
    assert torch.all(big["kt"][300:].float() == 5.0) and torch.all(big["kt"][:, 500:].float() == 5.0)
    # the K-major products are the products (not only the same in both kernels)
    pk = probs(big)
    Q64, X64 = to64(from_pairs(pk[7]["a"])), to64(from_pairs(pk[7]["b"]))
    assert_bound(to64(from_pairs(big["kx"])), Q64 @ X64, acc_bound(512, 1.0, Q64, X64.T),
                 torch.float16, "Q X, X K-major")
    A64, B64, C64 = X64.T[:300], Q64[:500], to64(pk[8]["c"])[:300, :500]
    assert_bound(to64(big["kt"])[:300, :500], -0.02 * (A64 @ B64.T) + C64,
                 acc_bound(512, -0.02, A64, B64, 1.0, C64), torch.bfloat16,
                 "X^T Q, X K-major, clipped")

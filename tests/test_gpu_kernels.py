"""Kernel-level GPU checks against fp64 products of the same fp16 operands.

* normalisation + cast (precision pipeline, steps 1-2): against
  fp16(G / (||G||_F + eps)) computed on the host in fp64;
* SYRK R = X X^T (Gram-space section): against the fp64 product of the same
  fp16 X, plus exact symmetry;
* the NT GEMM with its epilogue (alpha A B^T + beta C + gamma I), in full
  and in symmetric (lower tiles + mirror) mode.

Products accumulate in fp32 and are rounded once to fp16, so each element
must lie within one fp16 ulp of the exact value plus the fp32 accumulation
bound K * 2^-24 * sum |a_ik b_jk|.
"""

import numpy as np
import pytest
import torch

import newton_schulz_matrix_amd as nsmi
from gpu_helpers import assert_close_product, fp16_ulp, require_gpu, to64

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _host_normalize(G64, eps=1e-7):
    nu = np.sqrt(np.sum(G64 * G64))
    return (G64 / (nu + eps)).astype(np.float16), nu


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1), (7, 13), (13, 7), (64, 64), (300, 200),
                                   (256, 1024), (1000, 37), (33, 4100)])
def test_normalize_matches_host(dtype, shape):
    require_gpu()
    print(f"normalize {dtype} {shape}", flush=True)
    g = torch.Generator().manual_seed(hash(shape) % 1000)
    G = torch.randn(shape, generator=g).to(DT[dtype])
    G64 = to64(G)
    want, nu = _host_normalize(G64)
    x, norm = nsmi.ns_normalize(G.cuda(), transpose_tall=True, return_norm=True)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    if shape[0] > shape[1]:
        want = want.T
    assert got.shape == want.shape
    assert abs(float(norm.item()) - nu) <= 1e-5 * nu
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert np.all(diff <= fp16_ulp(want))
    assert np.mean(got == want) >= 0.999 or got.size < 1000


def test_normalize_strided_and_unaligned_input():
    require_gpu()
    base = torch.randn(70, 131, dtype=torch.float32)
    view = base[3:, 1:100]           # ldg = 131, base pointer not 16-byte aligned
    want, _ = _host_normalize(to64(view))
    x = nsmi.ns_normalize(base.cuda()[3:, 1:100], transpose_tall=False)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    assert np.all(np.abs(got.astype(np.float64) - want.astype(np.float64)) <= fp16_ulp(want))


def test_normalize_zero_and_no_transpose():
    require_gpu()
    z = nsmi.ns_normalize(torch.zeros(40, 9, device="cuda"), transpose_tall=False)
    assert z.shape == (40, 9) and not torch.any(z)


def _rand16(shape, scale, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).half()


@pytest.mark.parametrize("s,l", [(256, 128), (256, 1024), (512, 384), (768, 2048)])
def test_syrk(s, l):
    require_gpu()
    print(f"syrk {s}x{l}", flush=True)
    X = _rand16((s, l), 1.0 / np.sqrt(l), s + l)
    R = nsmi.ns_syrk(X.cuda())
    torch.cuda.synchronize()
    X64 = to64(X)
    want = X64 @ X64.T
    bound = l * 2.0 ** -24 * (np.abs(X64) @ np.abs(X64).T)
    got = to64(R)
    assert_close_product(got, want, bound, f"syrk {s}x{l}")
    assert torch.equal(R, R.T)


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (512, 768, 384), (1024, 256, 1024), (256, 512, 640)])
def test_gemm_nt_full(M, N, K):
    require_gpu()
    print(f"gemm {M}x{N}x{K}", flush=True)
    A = _rand16((M, K), 1.0 / np.sqrt(K), 1)
    B = _rand16((N, K), 1.0, 2)
    C = _rand16((M, N), 1.0, 3)
    alpha, beta, gamma = 0.7, -1.3, 0.25
    D = nsmi.ns_gemm_nt(A.cuda(), B.cuda(), C.cuda(), alpha, beta, gamma)
    torch.cuda.synchronize()
    A64, B64, C64 = to64(A), to64(B), to64(C)
    want = alpha * (A64 @ B64.T) + beta * C64 + gamma * np.eye(M, N)
    bound = (K + 2) * 2.0 ** -24 * (abs(alpha) * (np.abs(A64) @ np.abs(B64).T)
                                   + abs(beta) * np.abs(C64) + gamma)
    assert_close_product(to64(D), want, bound, f"gemm {M}x{N}x{K}")


@pytest.mark.parametrize("n", [256, 768])
def test_gemm_nt_symmetric(n):
    require_gpu()
    R = nsmi.ns_syrk(_rand16((n, 512), 1.0 / np.sqrt(512), n).cuda())
    # R R^T with beta R + gamma I: symmetric in exact arithmetic
    D = nsmi.ns_gemm_nt(R, R, R, 2.0, -0.5, 1.5, symmetric=True)
    torch.cuda.synchronize()
    assert torch.equal(D, D.T)
    R64 = to64(R)
    want = 2.0 * R64 @ R64 + -0.5 * R64 + 1.5 * np.eye(n)
    bound = (n + 2) * 2.0 ** -24 * (2.0 * np.abs(R64) @ np.abs(R64) + 0.5 * np.abs(R64) + 1.5)
    assert_close_product(to64(D), want, bound, f"sym gemm {n}")

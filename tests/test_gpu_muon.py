"""GPU checks of the fused Muon step (ns_muon_step) against the oracle's
reading of it (oracle.muon_step; its formula is a reading, the pages' is
missing, so parity against the pages is unpinned, and the composition is
pinned in tests/test_oracle_muon.py).

* momentum: M' = fp(beta M + G) from one fp32 fma per element: within one
  ulp of the fp64 value rounded to M's type (bitwise in >= 99.9% of
  elements for fp32);
* parameter: the applied update (W' - W) / (-lr scale) against the oracle
  NS of M' at the 1e-2 bar (fp32 parameters, so W's rounding is far below
  the update); bf16 buffers within their rounding;
* a batch of mixed shapes equals per-matrix calls bitwise, lr = 0 leaves W
  bitwise unchanged, beta = 0 gives M' = G, several steps accumulate.
"""

import numpy as np
import pytest
import torch

import newton_schulz_matrix_amd as nsmi
import workloads as W
from gpu_helpers import assert_tiles_uniform, rel_fro, require_gpu, to64
from oracle import YOU_COEFFICIENTS, muon_step

pytestmark = pytest.mark.gpu


def _case(shape, seed, dt=torch.float32):
    G = W.small_gaussian(seed, *shape)
    M = W.small_gaussian(seed + 100, *shape)
    P = W.small_gaussian(seed + 200, *shape) * 0.02
    return G.to(dt), M.to(dt), P.to(dt)


def _ulps32(a, b):
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


@pytest.mark.parametrize("shape", [(300, 1000), (1000, 300), (256, 256), (7, 13)])
def test_muon_step_fp32(shape):
    require_gpu()
    G, M, P = _case(shape, sum(shape))
    beta, lr, scale = 0.95, 0.02, 1.5
    g, m, p = G.cuda(), M.cuda(), P.cuda()
    nsmi.ns_muon_step([g], [m], [p], beta, lr, [scale], nsmi.YOU_COEFFICIENTS, (2,))
    torch.cuda.synchronize()
    M1, P1 = muon_step(to64(G), to64(M), to64(P), np.float64(np.float32(beta)), lr, scale,
                       YOU_COEFFICIENTS, (2,))
    u = _ulps32(m.cpu().numpy(), M1)
    assert u.max() <= 1 and np.mean(u == 0) >= 0.999
    upd = (to64(p) - to64(P)) / (-np.float64(np.float32(lr)) * np.float64(np.float32(scale)))
    want = (P1 - to64(P)) / (-lr * scale)
    err = rel_fro(upd, want)
    print(f"muon {shape}: update rel err {err:.3e}", flush=True)
    assert err <= 1e-2


def test_muon_step_bf16_buffers():
    require_gpu()
    G, M, P = _case((384, 1000), 5, torch.bfloat16)
    beta, lr = 0.9, 0.02
    g, m, p = G.cuda(), M.cuda(), P.cuda()
    nsmi.ns_muon_step([g], [m], [p], beta, lr, None, nsmi.YOU_COEFFICIENTS, (2,))
    torch.cuda.synchronize()
    M1, P1 = muon_step(to64(G), to64(M), to64(P), np.float64(np.float32(beta)), lr, 1.0,
                       YOU_COEFFICIENTS, (2,))
    # momentum: one bf16 rounding of the fp32 fma
    want_m = torch.from_numpy(M1).float().to(torch.bfloat16).double().numpy()
    ulp_m = np.maximum(np.abs(want_m), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(to64(m) - want_m) <= ulp_m)
    # parameter: W' = bf16(W - lr * U) with U the GPU's NS(M'). Per element,
    # |W'_i - P1_i| <= ulp_i + lr |U_i - U_ref,i| (one bf16 rounding, ulp_i the
    # bf16 spacing at P1_i, generous for round-to-nearest). So the excess over
    # one ulp is bounded elementwise by lr |U - U_ref|, whose Frobenius norm
    # the 1e-2 bar bounds by lr * 1e-2 * ||U_ref||.
    ulp_p = np.maximum(np.abs(P1), 2.0 ** -133) * 2.0 ** -7
    excess = np.maximum(np.abs(to64(p) - P1) - ulp_p, 0.0)
    u_ref = (P1 - to64(P)) / (-lr)
    bound = lr * 1e-2 * np.linalg.norm(u_ref)
    print(f"bf16 muon: rounding excess {np.linalg.norm(excess):.3e} vs bar {bound:.3e}",
          flush=True)
    assert np.linalg.norm(excess) <= bound


def test_muon_batched_equals_single_calls_and_edge_cases():
    require_gpu()
    shapes = [(300, 1000), (1000, 300), (256, 700), (64, 64)]
    cases = [_case(s, 40 + i) for i, s in enumerate(shapes)]
    scales = [1.0, 0.5, 2.0, 1.25]
    gs = [c[0].cuda() for c in cases]
    ms = [c[1].cuda() for c in cases]
    ps = [c[2].cuda() for c in cases]
    nsmi.ns_muon_step(gs, ms, ps, 0.9, 0.02, scales, nsmi.YOU_COEFFICIENTS, (2,))
    for i, c in enumerate(cases):
        m1, p1 = c[1].cuda(), c[2].cuda()
        nsmi.ns_muon_step([gs[i]], [m1], [p1], 0.9, 0.02, [scales[i]], nsmi.YOU_COEFFICIENTS,
                          (2,))
        torch.cuda.synchronize()
        assert torch.equal(m1, ms[i]) and torch.equal(p1, ps[i])
    # lr = 0: parameters untouched; beta = 0: momentum becomes the gradient
    G, M, P = _case((300, 700), 77)
    g, m, p = G.cuda(), M.cuda(), P.cuda()
    nsmi.ns_muon_step([g], [m], [p], 0.0, 0.0, None, nsmi.YOU_COEFFICIENTS, (2,))
    torch.cuda.synchronize()
    assert torch.equal(p.cpu(), P) and torch.equal(m.cpu(), G)


def test_muon_three_steps():
    require_gpu()
    G, M, P = _case((512, 1500), 9)
    g, m, p = G.cuda(), M.cuda(), P.cuda()
    M64, P64 = to64(M), to64(P)
    for _ in range(3):
        nsmi.ns_muon_step([g], [m], [p], 0.9, 0.02, None, nsmi.YOU_COEFFICIENTS, (2,))
        M64, P64 = muon_step(to64(G), M64, P64, np.float64(np.float32(0.9)), 0.02, 1.0,
                             YOU_COEFFICIENTS, (2,))
    torch.cuda.synchronize()
    assert rel_fro(to64(m), M64) < 1e-6
    err = rel_fro(to64(p) - to64(P), P64 - to64(P))
    print(f"three steps: accumulated update rel err {err:.3e}", flush=True)
    assert err <= 1e-2


def test_muon_step_owner_batch_full_size():
    """The fused Muon step on the 28-matrix owner batch in the benchmark's
    configuration (bf16 gradients, fp32 momentum and parameters, Polar
    Express, restart [2], beta 0.95, lr 0.02): one matrix of each Gram shape
    class against the oracle (momentum within one fp32 ulp, update at the
    1e-2 bar). Momentum and parameters are drawn on the device from a seeded
    generator."""
    require_gpu()
    from oracle import COEFFICIENT_SETS
    w = W.WORKLOADS[4]
    Gs = [W.matrix(4, j).cuda() for j in range(len(w.shapes))]
    gen = torch.Generator(device="cuda").manual_seed(404)
    Ms = [torch.randn(G.shape, generator=gen, device="cuda") for G in Gs]
    Ps = [torch.randn(G.shape, generator=gen, device="cuda") * 0.02 for G in Gs]
    M0 = {j: Ms[j].cpu() for j in (0, 1, 4)}          # q 4096^2, k 1024x4096, gate 14336x4096
    P0 = {j: Ps[j].cpu() for j in (0, 1, 4)}
    beta, lr = 0.95, 0.02
    nsmi.ns_muon_step(Gs, Ms, Ps, beta, lr, None, nsmi.COEFFICIENT_SETS[w.coefficients],
                      w.restarts)
    torch.cuda.synchronize()
    for j in (0, 1, 4):
        M1, P1 = muon_step(to64(Gs[j].cpu()), to64(M0[j]), to64(P0[j]),
                           np.float64(np.float32(beta)), lr, 1.0,
                           COEFFICIENT_SETS[w.coefficients], w.restarts)
        u = _ulps32(Ms[j].cpu().numpy(), M1)
        assert u.max() <= 1
        upd = (to64(Ps[j]) - to64(P0[j])) / (-np.float64(np.float32(lr)))
        err, worst = assert_tiles_uniform(upd, (P1 - to64(P0[j])) / (-lr),
                                          what=f"muon owner batch #{j}")
        print(f"muon owner batch #{j} {tuple(Gs[j].shape)}: update rel err {err:.3e} "
              f"(worst tile {worst:.3e})", flush=True)
        assert err <= 1e-2

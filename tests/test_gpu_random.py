"""Randomised GPU parity: seeded mixed batches through one grouped call.

Each case draws 1-5 matrices of random shape (1 to 700 per side, ragged and
degenerate widths included), a random input dtype (fp32 / bf16 / fp16), a
random output dtype, one of the two coefficient tables, a random restart set
and a backend, runs them through one ns_batched call and compares every
output with the fp64 oracle. The bar is the parity tests' one: relative
Frobenius error <= 1e-2, or <= 1.5x the fp16 rounding model's own error where
the method itself cannot reach 1e-2 in fp16 (the model shares no code with
the GPU path). Inputs are Gaussian with a random scale, so the normalisation
is exercised over many orders of magnitude. Where the printed Polar Express
table would overflow fp16 on a case's inputs (see pe_in_fp16_range) the
case runs the You table instead.
"""

import numpy as np
import pytest
import torch

import newton_schulz_matrix_amd as nsmi
from gpu_helpers import rel_fro, require_gpu, to64
from oracle import (POLAR_EXPRESS_COEFFICIENTS, YOU_COEFFICIENTS,
                    direct_newton_schulz, gram_newton_schulz, scalar_map)
from oracle import fp16_model

pytestmark = pytest.mark.gpu

TABLES = [("pe", POLAR_EXPRESS_COEFFICIENTS, nsmi.POLAR_EXPRESS_COEFFICIENTS),
          ("you", YOU_COEFFICIENTS, nsmi.YOU_COEFFICIENTS)]
RESTARTS = [(), (2,), (1, 3), (1, 2, 3, 4), (4,)]
IN_DTYPES = [torch.float32, torch.bfloat16, torch.float16]
OUT_DTYPES = [torch.float16, torch.float32, torch.bfloat16]
# output rounding on top of the fp16 iterate (bf16 keeps 8 bits)
OUT_SLACK = {torch.float16: 0.0, torch.float32: 0.0, torch.bfloat16: 4e-3}


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    count = int(rng.integers(1, 6))
    dims = [1, 2, 3, 7, 31, 64, 100, 129, 256, 300, 511, 700]
    shapes = []
    for _ in range(count):
        if rng.random() < 0.5:
            shapes.append((int(rng.choice(dims)), int(rng.choice(dims))))
        else:
            shapes.append((int(rng.integers(1, 701)), int(rng.integers(1, 701))))
    table = TABLES[int(rng.integers(len(TABLES)))]
    restarts = RESTARTS[int(rng.integers(len(RESTARTS)))]
    backend = "gram" if rng.random() < 0.7 else "direct"
    in_dtype = IN_DTYPES[int(rng.integers(len(IN_DTYPES)))]
    out_dtype = OUT_DTYPES[int(rng.integers(len(OUT_DTYPES)))]
    Gs = []
    for (m, n) in shapes:
        scale = float(10.0 ** rng.uniform(-3, 3))
        x = rng.standard_normal((m, n)) * scale
        Gs.append(torch.from_numpy(x.astype(np.float32)).to(in_dtype))
    if table[0] == "pe" and not all(pe_in_fp16_range(G) for G in Gs):
        table = TABLES[1]
    return Gs, table, restarts, backend, out_dtype


def pe_in_fp16_range(G):
    """The printed Polar Express table is not a convergent polar iteration:
    its composed map reaches 1e4-1e30 on parts of [0, 1] (and overflows fp16
    there, as the method itself does). Random cases use it only where the
    map stays below 1e3 on the input's own normalised singular values."""
    G64 = to64(G)
    s = np.linalg.svd(G64, compute_uv=False) / np.linalg.norm(G64)
    return bool(np.max(np.abs(scalar_map(POLAR_EXPRESS_COEFFICIENTS, s))) <= 1e3)


@pytest.mark.parametrize("seed", range(24))
def test_random_batch(seed):
    require_gpu()
    Gs, (tname, co64, co), restarts, backend, out_dtype = draw_case(seed)
    desc = (f"seed {seed}: {backend} {tname} restarts {restarts} in {Gs[0].dtype} "
            f"out {out_dtype} shapes {[tuple(G.shape) for G in Gs]}")
    print(desc, flush=True)
    outs = nsmi.ns_batched([G.cuda() for G in Gs], backend, co, restarts,
                           out_dtype=out_dtype)
    torch.cuda.synchronize()
    for G, out in zip(Gs, outs):
        assert out.shape == G.shape and out.dtype == out_dtype
        G64 = to64(G)
        if backend == "gram":
            ref = gram_newton_schulz(G64, co64, restarts)
            emu = fp16_model.gram_fp16(G64, co64, restarts, symmetric=True)
        else:
            ref = direct_newton_schulz(G64, co64)
            emu = fp16_model.direct_fp16(G64, co64, symmetric=True)
        err = rel_fro(to64(out), ref)
        floor = rel_fro(emu, ref)
        bar = max(1e-2, 1.5 * floor) + OUT_SLACK[out_dtype]
        print(f"  {tuple(G.shape)}: rel err {err:.3e} (fp16 model {floor:.3e}, bar {bar:.3e})",
              flush=True)
        assert err <= bar, desc

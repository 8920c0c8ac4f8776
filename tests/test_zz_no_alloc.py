"""The workspace-free entry point ns_batched_noalloc (static device scratch)
against ns_batched, through the C ABI.

Two calls in a row, the second on a smaller batch, so stale scratch
contents from the first call cannot leak into the second; each output must
equal ns_batched's bitwise (the same kernels on the same plan). A batch
whose workspace exceeds the scratch is refused before any device work.
"""

import pytest
import torch

import newton_schulz_matrix_amd as nsmi
import workloads as W
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

BATCHES = [[(300, 700), (1000, 300), (256, 1024), (513, 257)], [(100, 200), (64, 64), (7, 13)]]


@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_noalloc_equals_batched_two_calls(backend):
    require_gpu()
    table = nsmi.YOU_COEFFICIENTS
    rs = (2,) if backend == "gram" else ()
    for k, shapes in enumerate(BATCHES):
        print(f"{backend} call {k}: {shapes}", flush=True)
        assert nsmi.ns_workspace_size(shapes, backend, table, rs) <= nsmi.NS_NOALLOC_SCRATCH_BYTES
        Gs = [W.small_gaussian(90 + 10 * k + i, *sh).cuda() for i, sh in enumerate(shapes)]
        outs = [torch.full(G.shape, 9.0, dtype=torch.float16, device="cuda") for G in Gs]
        nsmi.ns_batched_noalloc(Gs, outs, backend, table, rs)
        want = nsmi.ns_batched(Gs, backend, table, rs)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, want)):
            assert torch.equal(a, b), (backend, k, i, shapes[i])


def test_noalloc_refuses_a_batch_larger_than_the_scratch():
    require_gpu()
    G = W.small_gaussian(5, 4096, 4096).cuda()
    assert nsmi.ns_workspace_size([(4096, 4096)]) > nsmi.NS_NOALLOC_SCRATCH_BYTES
    out = torch.full(G.shape, 9.0, dtype=torch.float16, device="cuda")
    with pytest.raises(nsmi.NsError) as e:
        nsmi.ns_batched_noalloc([G], [out])
    assert e.value.status == nsmi.NS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 9.0)

"""Calls captured into a HIP graph and replayed.

A call enqueues kernel launches only (its descriptor tables travel as
kernel arguments of small fill launches), so torch.cuda.graph can capture
it. Each replay must equal an eager call on the same inputs, bitwise: the
graph is replayed several times with eager work and synchronisations
between the replays, and the inputs are overwritten in place between
replays so that every replay has to read them again.
"""

import pytest
import torch

import newton_schulz_matrix_amd as nsmi
import workloads as W
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_batched_call_replays_bitwise(backend):
    require_gpu()
    shapes = [(256, 1024), (300, 700), (700, 300), (64, 64)]
    Gs = [W.small_gaussian(60 + i, *sh).cuda() for i, sh in enumerate(shapes)]
    outs = [torch.empty(G.shape, dtype=torch.float16, device="cuda") for G in Gs]
    table = nsmi.YOU_COEFFICIENTS
    rs = (2,) if backend == "gram" else ()
    ws = torch.empty(nsmi.ns_workspace_size(shapes, backend, table, rs), dtype=torch.uint8,
                     device="cuda")
    g = _capture(lambda: nsmi.ns_batched(Gs, backend, table, rs, outs=outs, workspace=ws))
    for rep in range(4):
        new = [W.small_gaussian(70 + 10 * rep + i, *sh).cuda() for i, sh in enumerate(shapes)]
        for G, N in zip(Gs, new):
            G.copy_(N)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        # eager reference on the same inputs, separate outputs and workspace
        want = nsmi.ns_batched(Gs, backend, table, rs)
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        del junk
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), (rep, i, shapes[i])


def test_large_launches_with_a_claimed_pool_replay_bitwise():
    """Six 1024 x 4096 matrices and one 2048 x 8192: the restart and output
    products run on the 256 x 256 kernel with 640 tiles each, so their
    last tiles are claimed through a counter in the workspace, which every
    replay must reset (a stale counter would leave those tiles unwritten)."""
    require_gpu()
    shapes = [(1024, 4096)] * 6 + [(2048, 8192)]
    print(f"graph replay, claimed pool: {shapes}", flush=True)
    Gs = [W.small_gaussian(120 + i, *sh).cuda() for i, sh in enumerate(shapes)]
    outs = [torch.empty(G.shape, dtype=torch.float16, device="cuda") for G in Gs]
    table = nsmi.POLAR_EXPRESS_COEFFICIENTS
    ws = torch.empty(nsmi.ns_workspace_size(shapes, "gram", table, (2,)), dtype=torch.uint8,
                     device="cuda")
    g = _capture(lambda: nsmi.ns_batched(Gs, "gram", table, (2,), outs=outs, workspace=ws))
    for rep in range(3):
        for i, (G, sh) in enumerate(zip(Gs, shapes)):
            G.copy_(W.small_gaussian(130 + 10 * rep + i, *sh).cuda())
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = nsmi.ns_batched(Gs, "gram", table, (2,))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), (rep, i, shapes[i])


def test_single_matrix_workload_replays_bitwise():
    """The 256 x 1024 workload (Polar Express, restart [2]), both backends
    captured in one graph."""
    require_gpu()
    G = W.matrix(1, 0).cuda()
    og = torch.empty(G.shape, dtype=torch.float16, device="cuda")
    od = torch.empty(G.shape, dtype=torch.float16, device="cuda")
    co = nsmi.POLAR_EXPRESS_COEFFICIENTS
    wg = torch.empty(nsmi.ns_workspace_size([tuple(G.shape)], "gram", co, (2,)),
                     dtype=torch.uint8, device="cuda")
    wd = torch.empty(nsmi.ns_workspace_size([tuple(G.shape)], "direct", co, ()),
                     dtype=torch.uint8, device="cuda")

    def call():
        nsmi.ns_gram(G, co, (2,), out=og, workspace=wg)
        nsmi.ns_direct(G, co, out=od, workspace=wd)

    g = _capture(call)
    eg = nsmi.ns_gram(G, co, (2,))
    ed = nsmi.ns_direct(G, co)
    torch.cuda.synchronize()
    for _ in range(3):
        og.zero_()
        od.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(og, eg) and torch.equal(od, ed)


def test_sharded_call_replays_bitwise():
    """The column-sharded route (4 virtual shards, shard reduction kernel)
    captured; its output and workspace come from the graph's memory pool."""
    require_gpu()
    G = W.small_gaussian(90, 384, 1536).cuda()
    co = nsmi.POLAR_EXPRESS_COEFFICIENTS
    holder = {}

    def call():
        holder["out"] = nsmi.ns_gram_sharded(G, 4, co, (2,))

    g = _capture(call)
    out = holder["out"]
    for rep in range(3):
        G.copy_(W.small_gaussian(91 + rep, 384, 1536).cuda())
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = nsmi.ns_gram_sharded(G, 4, co, (2,))
        torch.cuda.synchronize()
        assert torch.equal(got, want), rep


def test_muon_step_replays_bitwise():
    """ns_muon_step updates momentum and parameters in place; before each
    replay the state is restored, and the replayed state must equal an eager
    step from the same state."""
    require_gpu()
    shapes = [(256, 1024), (1024, 256), (300, 500)]
    grads = [W.small_gaussian(100 + i, *sh).cuda().to(torch.bfloat16)
             for i, sh in enumerate(shapes)]
    m0 = [W.small_gaussian(110 + i, *sh).cuda().float() for i, sh in enumerate(shapes)]
    w0 = [W.small_gaussian(120 + i, *sh).cuda().float() for i, sh in enumerate(shapes)]
    mom = [m.clone() for m in m0]
    par = [w.clone() for w in w0]
    co = nsmi.POLAR_EXPRESS_COEFFICIENTS
    ws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")

    def call():
        nsmi.ns_muon_step(grads, mom, par, 0.95, 0.02, coefficients=co,
                          restart_iterations=(2,), workspace=ws)

    g = _capture(call)
    for rep in range(3):
        for a, b in zip(mom + par, m0 + w0):
            a.copy_(b)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in mom + par]
        em = [m.clone() for m in m0]
        ew = [w.clone() for w in w0]
        nsmi.ns_muon_step(grads, em, ew, 0.95, 0.02, coefficients=co, restart_iterations=(2,))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, em + ew)):
            assert torch.equal(a, b), (rep, i)

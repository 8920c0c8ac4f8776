"""Calls on several streams and from several host threads.

Each call copies its descriptor tables through a ring of pinned host slots
that all calls on a device share (a slot is reused only after the copy
recorded on it has completed). Calls with their own workspaces on
different streams, interleaved, and calls from two host threads at once,
must each equal the same call made alone on the default stream, bitwise.
"""

import threading

import pytest
import torch

import newton_schulz_matrix_amd as nsmi
import workloads as W
from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

SHAPES = [(256, 1024), (700, 300), (1024, 1024)]


def _inputs(seed):
    return [W.small_gaussian(seed + i, *s).cuda() for i, s in enumerate(SHAPES)]


def _ws(Gs, backend):
    rs = (2,) if backend == "gram" else ()
    n = nsmi.ns_workspace_size([tuple(G.shape) for G in Gs], backend,
                               nsmi.POLAR_EXPRESS_COEFFICIENTS, rs)
    return torch.empty(n, dtype=torch.uint8, device="cuda"), rs


@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_interleaved_streams(backend):
    require_gpu()
    co = nsmi.POLAR_EXPRESS_COEFFICIENTS
    inputs = [_inputs(200 + 10 * k) for k in range(4)]
    want = []
    for Gs in inputs:
        _, rs = _ws(Gs, backend)
        want.append(nsmi.ns_batched(Gs, backend, co, rs))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ws = [_ws(Gs, backend)[0] for Gs in inputs]
    outs = [[torch.empty(G.shape, dtype=torch.float16, device="cuda") for G in Gs]
            for Gs in inputs]
    torch.cuda.synchronize()
    # 3 rounds x 4 calls: more calls than slots in the staging ring
    for _ in range(3):
        for k, Gs in enumerate(inputs):
            with torch.cuda.stream(streams[k % 2]):
                nsmi.ns_batched(Gs, backend, co, _ws(Gs, backend)[1], outs=outs[k],
                                workspace=ws[k])
    torch.cuda.synchronize()
    for k in range(len(inputs)):
        for a, b in zip(outs[k], want[k]):
            assert torch.equal(a, b), (backend, k)


def test_two_host_threads():
    require_gpu()
    co = nsmi.POLAR_EXPRESS_COEFFICIENTS
    inputs = [_inputs(300), _inputs(320)]
    want = [nsmi.ns_batched(Gs, "gram", co, (2,)) for Gs in inputs]
    torch.cuda.synchronize()
    results = [None, None]
    errors = []

    def run(k):
        try:
            s = torch.cuda.Stream()
            ws, rs = _ws(inputs[k], "gram")
            outs = [torch.empty(G.shape, dtype=torch.float16, device="cuda")
                    for G in inputs[k]]
            with torch.cuda.stream(s):
                for _ in range(6):
                    nsmi.ns_batched(inputs[k], "gram", co, rs, outs=outs, workspace=ws)
            s.synchronize()
            results[k] = outs
        except Exception as e:   # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for k in range(2):
        assert results[k] is not None
        for a, b in zip(results[k], want[k]):
            assert torch.equal(a, b), k

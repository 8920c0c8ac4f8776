"""Diagnostics surface: ns_backend_status / get_backend_status /
get_ns_backend and the NewtonSchulz configuration object (the page's
"查询当前后端" and "强制指定内核" sections).

Host checks run everywhere; the device checks are marked gpu.
"""

import ctypes
import os

import pytest

import newton_schulz_matrix_amd as nsmi

needs_lib = pytest.mark.skipif(not os.path.exists(nsmi.LIB_PATH), reason="libnsmi.so not built")


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@needs_lib
def test_status_rejects_null():
    assert nsmi.library().ns_backend_status(None) == nsmi.NS_ERR_INVALID_ARG


@needs_lib
def test_status_fields_are_well_formed():
    st = nsmi.get_backend_status()
    assert st["deterministic"] is True
    assert st["gemm_tile"] == 256
    assert st["version"] >= 1
    assert "hip-mfma-f16" in st["kernel"]
    assert st["auto_choice"] in (None, "hip-mfma-f16")
    assert (st["auto_choice"] is None) == (not st["gfx950_available"])
    assert isinstance(nsmi.get_ns_backend(), str)


@needs_lib
@pytest.mark.skipif(not _no_gpu(), reason="only meaningful where no GPU is visible")
def test_status_without_device():
    st = nsmi.get_backend_status()
    assert st["gfx950_available"] is False
    assert st["device_index"] == -1 and st["compute_units"] == 0 and st["arch"] == ""
    with pytest.raises(RuntimeError, match="gfx950"):
        nsmi.NewtonSchulz(kernel="hip-mfma-f16")


@needs_lib
@pytest.mark.parametrize("kw, exc", [
    (dict(backend="svd"), ValueError),
    (dict(kernel="cublas"), ValueError),
    (dict(kernel="cute_sm80"), ValueError),
    (dict(kernel="quack"), ValueError),
    (dict(restart_iterations=(9,)), nsmi.NsError),
    (dict(coefficients=()), nsmi.NsError),
    (dict(eps=-1.0), nsmi.NsError),
])
def test_newton_schulz_object_rejects_at_construction(kw, exc):
    with pytest.raises(exc):
        nsmi.NewtonSchulz(**kw)


@needs_lib
def test_newton_schulz_object_keeps_its_configuration():
    ns = nsmi.NewtonSchulz("direct", coefficients=nsmi.YOU_COEFFICIENTS, restart_iterations=(1, 3))
    assert ns.backend == "direct" and ns.kernel == "hip-mfma-f16" and ns.deterministic
    assert ns.coefficients == tuple(tuple(float(x) for x in r) for r in nsmi.YOU_COEFFICIENTS)
    assert ns.restart_iterations == (1, 3)
    assert "direct" in repr(ns)


@pytest.mark.gpu
def test_status_on_device():
    from gpu_helpers import require_gpu
    require_gpu()
    st = nsmi.get_backend_status()
    assert st["gfx950_available"] and st["arch"].startswith("gfx950")
    assert st["compute_units"] > 0 and st["clock_mhz"] > 0 and st["device_index"] >= 0
    assert st["auto_choice"] == "hip-mfma-f16"
    assert "gfx950" in nsmi.get_ns_backend()
    nsmi.NewtonSchulz(kernel="hip-mfma-f16")   # explicit kernel constructs on gfx950


@pytest.mark.gpu
@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_newton_schulz_object_matches_entry_points(backend):
    import torch
    import workloads as W
    from gpu_helpers import require_gpu
    require_gpu()
    G = W.small_gaussian(11, 300, 700).cuda()
    ns = nsmi.NewtonSchulz(backend, coefficients=nsmi.YOU_COEFFICIENTS, restart_iterations=(2,))
    a = ns(G)
    b = (nsmi.ns_gram(G, nsmi.YOU_COEFFICIENTS, (2,)) if backend == "gram"
         else nsmi.ns_direct(G, nsmi.YOU_COEFFICIENTS))
    c = ns.batched([G, G])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c[0], a) and torch.equal(c[1], a)

"""C-ABI contract checks that need no GPU.

The library must load, export every function include/ns.h declares, and
reject bad arguments on the host before touching a device. Calls that would
launch work are only made with deliberately invalid arguments, or (for the
"no device" status) only when no GPU is visible.
"""

import ctypes
import os
import re

import pytest

import newton_schulz_matrix_amd as nsmi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ns.h")

pytestmark = pytest.mark.skipif(not os.path.exists(nsmi.LIB_PATH),
                                reason="libnsmi.so not built")


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ns_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("ns_normalize", "ns_direct", "ns_gram", "ns_batched",
                 "ns_workspace_size", "ns_status_string", "ns_backend_info"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(nsmi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert nsmi.status_string(0) == "NS_OK"
    assert nsmi.status_string(1) == "NS_ERR_INVALID_ARG"
    assert nsmi.status_string(2) == "NS_ERR_UNSUPPORTED"
    assert nsmi.status_string(3) == "NS_ERR_WORKSPACE"
    assert nsmi.status_string(4) == "NS_ERR_HIP"
    assert nsmi.status_string(99) == "NS_ERR_UNKNOWN"


def test_backend_info_is_a_string():
    info = nsmi.ns_backend_info()
    assert "NS" in info and "hip-mfma-f16" in info
    if _no_gpu():
        assert "no gfx950" in info


def _mats(shapes, g=1, out=1):
    arr = (nsmi._Matrix * len(shapes))()
    for i, (m, n) in enumerate(shapes):
        arr[i] = nsmi._Matrix(g, nsmi.NS_DT_F32, m, n, n, out, nsmi.NS_DT_F16, n)
    return arr


def _size(shapes, backend="gram", coeffs=nsmi.POLAR_EXPRESS_COEFFICIENTS, restarts=(2,),
          eps=1e-7):
    return nsmi.ns_workspace_size(shapes, backend, coeffs, restarts, eps)


def test_workspace_size_monotone_and_additive():
    a = _size([(256, 1024)])
    b = _size([(256, 2048)])
    c = _size([(512, 1024)])
    assert 0 < a < b and a < c
    both = _size([(256, 1024), (512, 1024)])
    assert both >= a + c - 4096
    # padding: any shape inside one 256 block costs the same buffers
    assert _size([(1, 1)]) == _size([(200, 250)])
    # tall and wide of the same pair use the same short-side buffers
    assert _size([(1024, 256)]) == _size([(256, 1024)])
    # buffer counts: gram keeps X twice (s x l) and R, Z, T, Q, Q' (s x s);
    # direct keeps X, X^T twice and A, B. The difference between the two
    # backends is one s x l buffer less three s x s ones, plus table bytes.
    s, l = 1024, 4096
    diff = _size([(s, l)], "direct", restarts=()) - _size([(s, l)])
    assert abs(diff - (s * l - 3 * s * s) * 2) < 64 * 1024
    # and one more column block of 256 adds two s x 256 fp16 buffers to gram
    grow = _size([(s, l + 256)]) - _size([(s, l)])
    assert abs(grow - 2 * s * 256 * 2) < 4096


def test_workspace_size_llama_owner_batch_fits():
    from workloads import WORKLOADS
    n = _size(list(WORKLOADS[4].shapes))
    assert 4e9 < n < 20e9


@pytest.mark.parametrize("bad", [
    dict(shapes=[(0, 4)]), dict(shapes=[(4, 0)]), dict(shapes=[(70000, 4)]),
    dict(coeffs=()), dict(coeffs=((1.0, float("nan"), 0.0),)),
    dict(coeffs=((1.0, 0.0, 0.0),) * 17),
    dict(restarts=(5,)), dict(restarts=(-1,)), dict(eps=-1.0), dict(eps=float("inf")),
])
def test_workspace_size_rejects(bad):
    kw = dict(shapes=[(16, 32)], coeffs=nsmi.POLAR_EXPRESS_COEFFICIENTS, restarts=(2,),
              eps=1e-7)
    kw.update(bad)
    with pytest.raises(nsmi.NsError) as e:
        nsmi.ns_workspace_size(kw["shapes"], "gram", kw["coeffs"], kw["restarts"], kw["eps"])
    assert e.value.status == nsmi.NS_ERR_INVALID_ARG


def test_direct_ignores_restart_indices():
    assert _size([(16, 32)], "direct", restarts=(9,)) > 0


def _params(coeffs=nsmi.POLAR_EXPRESS_COEFFICIENTS, restarts=(2,), eps=1e-7):
    return nsmi._params(coeffs, restarts, eps)


def test_calls_reject_bad_arguments_before_any_device_work():
    lib = nsmi.library()
    p, keep = _params()
    fake = 0x1000
    fake_out, fake_m, fake_w = 0x100000, 0x200000, 0x300000   # distinct, never touched
    good = _mats([(16, 32)], fake, fake_out)
    # null matrix pointers
    assert lib.ns_gram(_mats([(16, 32)], None, fake), ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_direct(_mats([(16, 32)], fake, None), ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    # leading dimension smaller than n
    bad_ld = _mats([(16, 32)], fake, fake_out)
    bad_ld[0].ldg = 8
    assert lib.ns_gram(bad_ld, ctypes.byref(p), fake, 1 << 30, None) == nsmi.NS_ERR_INVALID_ARG
    # bad dtype
    bad_dt = _mats([(16, 32)], fake, fake_out)
    bad_dt[0].out_dtype = 7
    assert lib.ns_gram(bad_dt, ctypes.byref(p), fake, 1 << 30, None) == nsmi.NS_ERR_INVALID_ARG
    # bad backend / negative count
    assert lib.ns_batched(good, 1, 5, ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_batched(good, -1, 0, ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    # null params
    assert lib.ns_gram(good, None, fake, 1 << 30, None) == nsmi.NS_ERR_INVALID_ARG
    # workspace missing or too small
    assert lib.ns_gram(good, ctypes.byref(p), None, 0, None) == nsmi.NS_ERR_WORKSPACE
    assert lib.ns_gram(good, ctypes.byref(p), fake, 16, None) == nsmi.NS_ERR_WORKSPACE
    # count == 0 is a no-op, even with no workspace
    assert lib.ns_batched(good, 0, 0, ctypes.byref(p), None, 0, None) == nsmi.NS_OK
    # restart index out of range (gram)
    p2, keep2 = _params(restarts=(5,))
    assert lib.ns_gram(good, ctypes.byref(p2), fake, 1 << 30, None) == nsmi.NS_ERR_INVALID_ARG


def test_normalize_and_unit_calls_reject_bad_arguments():
    lib = nsmi.library()
    fake = 0x1000
    fake_out, fake_m, fake_w = 0x100000, 0x200000, 0x300000   # distinct, never touched
    nb = ctypes.c_size_t(0)
    assert lib.ns_normalize_workspace_size(3, 5, ctypes.byref(nb)) == nsmi.NS_OK and nb.value > 0
    assert lib.ns_normalize_workspace_size(0, 5, ctypes.byref(nb)) == nsmi.NS_ERR_INVALID_ARG
    args = dict(g=fake, dt=nsmi.NS_DT_F32, m=3, n=5, ldg=5, x=fake, ldx=5, tr=1, eps=1e-7)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.ns_normalize(a["g"], a["dt"], a["m"], a["n"], a["ldg"], a["x"], a["ldx"],
                                a["tr"], a["eps"], None, fake, 1 << 20, None)

    assert call(g=None) == nsmi.NS_ERR_INVALID_ARG
    assert call(ldg=4) == nsmi.NS_ERR_INVALID_ARG
    assert call(dt=9) == nsmi.NS_ERR_INVALID_ARG
    assert call(eps=-1.0) == nsmi.NS_ERR_INVALID_ARG
    # tall input transposed: x is (n, m), needs ldx >= m
    assert call(m=9, n=5, ldx=5) == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_normalize(fake, 0, 3, 5, 5, fake, 5, 1, 1e-7, None, fake, 4, None) \
        == nsmi.NS_ERR_WORKSPACE
    # unit GEMM shape rules
    ws = 1 << 20
    assert lib.ns_gemm_nt(fake, fake, None, fake, 200, 256, 64, 1.0, 0.0, 0.0, 0, fake, ws,
                          None) == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gemm_nt(fake, fake, None, fake, 256, 512, 64, 1.0, 0.0, 0.0, 1, fake, ws,
                          None) == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gemm_nt(fake, fake, None, fake, 256, 256, 128, 1.0, 1.0, 0.0, 0, fake, ws,
                          None) == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gemm_nt(fake, fake, None, fake, 256, 256, 128, 1.0, 0.0, 0.0, 0, fake, 8,
                          None) == nsmi.NS_ERR_WORKSPACE
    assert lib.ns_syrk(fake, 256, 100, fake, fake, ws, None) == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gemm_nt(fake, fake, None, fake, 256, 256, 64, 1.0, 0.0, 0.0, 0, fake, ws,
                          None) == nsmi.NS_ERR_INVALID_ARG


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful where no GPU is visible")
def test_valid_call_without_device_reports_unsupported():
    lib = nsmi.library()
    p, keep = _params()
    fake = 0x1000
    fake_out, fake_m, fake_w = 0x100000, 0x200000, 0x300000   # distinct, never touched
    good = _mats([(16, 32)], fake, fake_out)
    assert lib.ns_gram(good, ctypes.byref(p), fake, 1 << 40, None) == nsmi.NS_ERR_UNSUPPORTED
    assert lib.ns_normalize(fake, 0, 3, 5, 5, fake, 5, 1, 1e-7, None, fake, 1 << 20, None) \
        == nsmi.NS_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(nsmi, "_lib", None)
    monkeypatch.setattr(nsmi, "LIB_PATH", "/nonexistent/libnsmi.so")
    with pytest.raises(RuntimeError, match="missing"):
        nsmi.library()


def _sharded_size(m, n, shards, restarts=(2,)):
    lib = nsmi.library()
    p, keep = _params(restarts=restarts)
    mat = nsmi._Matrix(None, nsmi.NS_DT_F32, m, n, n, None, nsmi.NS_DT_F16, n)
    nb = ctypes.c_size_t(0)
    st = lib.ns_gram_sharded_workspace_size(ctypes.byref(mat), shards, ctypes.byref(p),
                                            ctypes.byref(nb))
    return st, nb.value


def test_sharded_workspace_rules():
    st1, one = _sharded_size(256, 1024, 1)
    assert st1 == nsmi.NS_OK
    assert one == _size([(256, 1024)])             # one shard: the ns_gram layout
    st4, four = _sharded_size(256, 1024, 4)
    assert st4 == nsmi.NS_OK and four > one        # partial Grams and padded shards
    assert _sharded_size(1024, 256, 4)[1] == four  # tall and wide alike
    for bad in (0, -1, 65, 1025):                  # range and shards <= max(m, n)
        assert _sharded_size(256, 1024, bad)[0] == nsmi.NS_ERR_INVALID_ARG
    assert _sharded_size(3, 5, 5)[0] == nsmi.NS_OK
    assert _sharded_size(3, 5, 6)[0] == nsmi.NS_ERR_INVALID_ARG
    assert _sharded_size(16, 32, 2, restarts=(7,))[0] == nsmi.NS_ERR_INVALID_ARG


def test_sharded_call_rejects_bad_arguments_before_any_device_work():
    lib = nsmi.library()
    p, keep = _params()
    fake = 0x1000
    fake_out, fake_m, fake_w = 0x100000, 0x200000, 0x300000   # distinct, never touched
    good = _mats([(16, 32)], fake, fake_out)
    assert lib.ns_gram_sharded(None, 2, ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gram_sharded(good, 0, ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gram_sharded(good, 33, ctypes.byref(p), fake, 1 << 30, None) \
        == nsmi.NS_ERR_INVALID_ARG
    assert lib.ns_gram_sharded(good, 2, ctypes.byref(p), fake, 16, None) \
        == nsmi.NS_ERR_WORKSPACE
    assert lib.ns_gram_sharded(_mats([(16, 32)], None, fake), 2, ctypes.byref(p), fake,
                               1 << 30, None) == nsmi.NS_ERR_INVALID_ARG


def _muon(shapes, g=None, m=None, w=None, scale=1.0, dt=None):
    dt = nsmi.NS_DT_F32 if dt is None else dt
    arr = (nsmi._MuonMatrix * len(shapes))()
    for i, (r, c) in enumerate(shapes):
        arr[i] = nsmi._MuonMatrix(g, dt, r, c, c, m, dt, c, w, dt, c, scale)
    return arr


def test_muon_workspace_matches_the_gram_layout():
    lib = nsmi.library()
    p, keep = _params()
    shapes = [(256, 1024), (1024, 256), (300, 700)]
    nb = ctypes.c_size_t(0)
    assert lib.ns_muon_workspace_size(_muon(shapes), 3, ctypes.byref(p), ctypes.byref(nb)) \
        == nsmi.NS_OK
    assert nb.value == _size(shapes)


def test_muon_step_rejects_bad_arguments_before_any_device_work():
    lib = nsmi.library()
    p, keep = _params()
    fake = 0x1000
    fake_out, fake_m, fake_w = 0x100000, 0x200000, 0x300000   # distinct, never touched
    ok = _muon([(16, 32)], fake, fake_m, fake_w)
    call = lambda mats, beta=0.9, lr=0.02, n=1, ws=1 << 30: lib.ns_muon_step(
        mats, n, ctypes.byref(p), beta, lr, fake, ws, None)
    assert call(_muon([(16, 32)], None, fake_m, fake_w)) == nsmi.NS_ERR_INVALID_ARG
    assert call(_muon([(16, 32)], fake, None, fake_w)) == nsmi.NS_ERR_INVALID_ARG
    assert call(_muon([(16, 32)], fake, fake_m, None)) == nsmi.NS_ERR_INVALID_ARG
    assert call(_muon([(16, 32)], fake, fake_m, fake_w, dt=9)) == nsmi.NS_ERR_INVALID_ARG
    assert call(_muon([(16, 32)], fake, fake_m, fake_w, scale=float("nan"))) == nsmi.NS_ERR_INVALID_ARG
    assert call(ok, beta=float("inf")) == nsmi.NS_ERR_INVALID_ARG
    assert call(ok, lr=float("nan")) == nsmi.NS_ERR_INVALID_ARG
    assert call(ok, n=-1) == nsmi.NS_ERR_INVALID_ARG
    assert call(ok, ws=16) == nsmi.NS_ERR_WORKSPACE
    assert lib.ns_muon_step(None, 0, ctypes.byref(p), 0.9, 0.02, None, 0, None) == nsmi.NS_OK
    bad_ld = _muon([(16, 32)], fake, fake_m, fake_w)
    bad_ld[0].ld_grad = 8
    assert call(bad_ld) == nsmi.NS_ERR_INVALID_ARG


def test_binding_leading_dimension_rules():
    """Row-major views only: contiguous rows that do not overlap. An
    expanded (stride-0) or transposed view is refused before any pointer
    reaches the library; column slices keep their row stride as ld."""
    import torch
    base = torch.zeros(6, 10)
    assert nsmi._rowmajor_ld(base) == 10
    assert nsmi._rowmajor_ld(base[:, 2:7]) == 10          # column slice: ld = row stride
    assert nsmi._rowmajor_ld(base[:1]) == 10              # one row
    assert nsmi._rowmajor_ld(torch.zeros(1, 10).expand(1, 10)) == 10
    with pytest.raises(ValueError, match="overlapping rows"):
        nsmi._rowmajor_ld(torch.zeros(1, 10).expand(5, 10))
    with pytest.raises(ValueError, match="overlapping rows"):
        nsmi._rowmajor_ld(torch.zeros(40).as_strided((4, 10), (5, 1)))
    with pytest.raises(ValueError, match="contiguous"):
        nsmi._rowmajor_ld(base.t())
    with pytest.raises(ValueError, match="2-D"):
        nsmi._rowmajor_ld(torch.zeros(2, 3, 4))


def test_output_overlapping_its_input_is_refused():
    """A matrix whose output byte range overlaps its input range is refused
    on the host, before any device work (pointers are never dereferenced)."""
    lib = nsmi.library()
    p, _keep = nsmi._params(nsmi.POLAR_EXPRESS_COEFFICIENTS, (2,), 1e-7)
    base = 1 << 40                                    # a fake, never-touched address
    for out_off in (0, 8 * 2 - 2, 7 * 16 * 2):        # same start, inside row 0, last row
        m = nsmi._Matrix(base, nsmi.NS_DT_F16, 8, 16, 16, base + out_off, nsmi.NS_DT_F16, 16)
        assert lib.ns_batched(ctypes.byref(m), 1, nsmi.NS_GRAM, ctypes.byref(p), ctypes.c_void_p(1),
                              1 << 30, None) == nsmi.NS_ERR_INVALID_ARG
    # just past the input's last byte: passes argument checks (no GPU here)
    m = nsmi._Matrix(base, nsmi.NS_DT_F16, 8, 16, 16, base + 8 * 16 * 2, nsmi.NS_DT_F16, 16)
    assert lib.ns_batched(ctypes.byref(m), 1, nsmi.NS_GRAM, ctypes.byref(p), ctypes.c_void_p(1),
                          1 << 30, None) in (nsmi.NS_ERR_UNSUPPORTED, nsmi.NS_OK)


def test_binding_checks_shapes_and_types_before_device_work():
    """Shapes and dtypes the library would misread (reading past B, writing
    past a small output) are refused in the binding, on CPU tensors too."""
    import torch
    with pytest.raises(ValueError, match="output shape"):
        nsmi._matrix(torch.zeros(8, 16), torch.zeros(8, 8, dtype=torch.float16))
    h = lambda *s: torch.zeros(*s, dtype=torch.float16)
    with pytest.raises(ValueError, match="columns"):
        nsmi.ns_gemm_nt(h(256, 128), h(256, 64))
    with pytest.raises(ValueError, match="C has shape"):
        nsmi.ns_gemm_nt(h(256, 128), h(256, 128), h(256, 128))
    with pytest.raises(ValueError, match="fp16"):
        nsmi.ns_gemm_nt(torch.zeros(256, 128), h(256, 128))
    with pytest.raises(ValueError, match="fp16"):
        nsmi.ns_syrk(torch.zeros(256, 128))


def _grouped(**kw):
    """One ns_gemm_grouped problem with fake, aligned, never-dereferenced
    pointers; returns the status (arguments are checked before any device
    work, so a valid problem reaches the device check)."""
    base = dict(a=0x10000, b=0x20000, c=None, d=0x30000, d2=None, dt=None, M=256, N=512,
                K=256, ldc=512, ldd=512, valid_m=256, valid_n=512, diag_n=0,
                c_dtype=nsmi.NS_DT_F16, d_dtype=nsmi.NS_DT_F16, symmetric=0, c_is_bt=0,
                a_pairs=1, b_pairs=1, c_pairs=0, d_pairs=0, a_kmajor=0, b_kmajor=0,
                alpha=1.0, beta=0.0, gamma=0.0, delta=0.0)
    base.update(kw)
    p = nsmi._GemmProblem(**base)
    return nsmi.library().ns_gemm_grouped(ctypes.byref(p), 1, 0, ctypes.c_void_p(0x40000),
                                          ctypes.c_size_t(1 << 20), None)


def test_gemm_grouped_kmajor_rules():
    """K-major operands: at most one, in the row-pair layout, not in the
    symmetric mode and not a B whose transpose is folded in as C."""
    ok = {nsmi.NS_OK, nsmi.NS_ERR_UNSUPPORTED, nsmi.NS_ERR_HIP}
    assert _grouped(b_kmajor=1) in ok
    assert _grouped(a_kmajor=1) in ok
    bad = nsmi.NS_ERR_INVALID_ARG
    assert _grouped(a_kmajor=1, b_kmajor=1) == bad
    assert _grouped(b_kmajor=1, b_pairs=0) == bad
    assert _grouped(a_kmajor=1, a_pairs=0) == bad
    sym = dict(M=512, valid_m=512, symmetric=1)
    assert _grouped(**sym) in ok
    assert _grouped(a_kmajor=1, **sym) == bad
    assert _grouped(b_kmajor=1, **sym) == bad
    fold = dict(N=256, valid_n=256, c=0x50000, ldc=256, ldd=256, beta=1.0, c_is_bt=1)
    assert _grouped(b_kmajor=1, **fold) == bad
    # the same fold with a row-major B, or with a K-major A, is accepted
    assert _grouped(**fold) in ok
    assert _grouped(a_kmajor=1, **fold) in ok

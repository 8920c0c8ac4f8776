"""Python binding of the gfx950 Newton-Schulz library (libnsmi.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/ns.h. PyTorch supplies device
memory (outputs and workspaces) and the current stream. If the library is
not built, importing works but every call raises.

Names follow the C ABI: ``ns_normalize``, ``ns_gram``, ``ns_direct``,
``ns_batched``, ``ns_workspace_size``, plus the building blocks ``ns_syrk``
and ``ns_gemm_nt`` and the diagnostics ``ns_backend_info`` /
``ns_status_string``.

The coefficient tables are the two 5-step sets of the DMuon page
"Newton-Schulz 变体", section "系数集" (coefficient sets), as printed there;
the Polar Express set is the default and the default restart list is [2]
(section "重启机制").
"""

from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libnsmi.so")

POLAR_EXPRESS_COEFFICIENTS = (
    (7.893, -20.381, 14.939),
    (3.912, -2.544, 0.470),
    (3.761, -2.512, 0.476),
    (3.160, -2.148, 0.440),
    (2.191, -1.441, 0.361),
)
YOU_COEFFICIENTS = (
    (4.0848, -6.8946, 2.9270),
    (3.9505, -6.3029, 2.6377),
    (3.7418, -5.5913, 2.3037),
    (2.8769, -3.1427, 1.2046),
    (2.8366, -3.0525, 1.2012),
)
COEFFICIENT_SETS = {"polar_express": POLAR_EXPRESS_COEFFICIENTS,
                    "you": YOU_COEFFICIENTS}
DEFAULT_RESTARTS = (2,)
DEFAULT_EPS = 1e-7

(NS_OK, NS_ERR_INVALID_ARG, NS_ERR_UNSUPPORTED, NS_ERR_WORKSPACE, NS_ERR_HIP,
 NS_ERR_INTERNAL) = range(6)
NS_CHECK_BATCHED, NS_CHECK_SHARDED, NS_CHECK_MUON = range(3)
NS_DT_F32, NS_DT_BF16, NS_DT_F16 = 0, 1, 2
NS_GRAM, NS_DIRECT = 0, 1
NS_UNIT_WORKSPACE_BYTES = 4096
BACKENDS = {"gram": NS_GRAM, "direct": NS_DIRECT}


class NsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class _Params(ctypes.Structure):
    _fields_ = [("num_steps", ctypes.c_int),
                ("coeffs", ctypes.POINTER(ctypes.c_float)),
                ("restarts", ctypes.POINTER(ctypes.c_int)),
                ("num_restarts", ctypes.c_int),
                ("eps", ctypes.c_float)]


class TimingReport(ctypes.Structure):
    _fields_ = [("gemm_ms", ctypes.c_double), ("gemm_launches", ctypes.c_int64),
                ("gemm_flops", ctypes.c_double), ("norm_ms", ctypes.c_double),
                ("norm_launches", ctypes.c_int64), ("norm_bytes", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class _BackendStatus(ctypes.Structure):
    _fields_ = [("device_found", ctypes.c_int), ("device_index", ctypes.c_int),
                ("arch", ctypes.c_char * 64), ("compute_units", ctypes.c_int),
                ("clock_mhz", ctypes.c_int), ("deterministic", ctypes.c_int),
                ("gemm_tile", ctypes.c_int), ("version", ctypes.c_int),
                ("kernel", ctypes.c_char_p)]


class _MuonMatrix(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("grad_dtype", ctypes.c_int),
                ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("ld_grad", ctypes.c_int64),
                ("momentum", ctypes.c_void_p), ("momentum_dtype", ctypes.c_int),
                ("ld_momentum", ctypes.c_int64),
                ("param", ctypes.c_void_p), ("param_dtype", ctypes.c_int),
                ("ld_param", ctypes.c_int64), ("scale", ctypes.c_float)]


class _GemmProblem(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("c", ctypes.c_void_p),
                ("d", ctypes.c_void_p), ("d2", ctypes.c_void_p), ("dt", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("ldc", ctypes.c_int64), ("ldd", ctypes.c_int64),
                ("valid_m", ctypes.c_int64), ("valid_n", ctypes.c_int64),
                ("diag_n", ctypes.c_int64),
                ("c_dtype", ctypes.c_int), ("d_dtype", ctypes.c_int),
                ("symmetric", ctypes.c_int), ("c_is_bt", ctypes.c_int),
                ("a_pairs", ctypes.c_int), ("b_pairs", ctypes.c_int),
                ("c_pairs", ctypes.c_int), ("d_pairs", ctypes.c_int),
                ("a_kmajor", ctypes.c_int), ("b_kmajor", ctypes.c_int),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("gamma", ctypes.c_float), ("delta", ctypes.c_float)]


class _Matrix(ctypes.Structure):
    _fields_ = [("g", ctypes.c_void_p),
                ("g_dtype", ctypes.c_int),
                ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("ldg", ctypes.c_int64),
                ("out", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int),
                ("ldo", ctypes.c_int64)]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libnsmi.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m newton_schulz_matrix_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P, M = ctypes.POINTER(_Params), ctypes.POINTER(_Matrix)
        sigs = {
            "ns_workspace_size": [M, ctypes.c_int, ctypes.c_int, P, ctypes.POINTER(sz)],
            "ns_normalize_workspace_size": [i64, i64, ctypes.POINTER(sz)],
            "ns_normalize": [vp, ctypes.c_int, i64, i64, i64, vp, i64, ctypes.c_int,
                             ctypes.c_float, vp, vp, sz, vp],
            "ns_direct": [M, P, vp, sz, vp],
            "ns_gram": [M, P, vp, sz, vp],
            "ns_batched": [M, ctypes.c_int, ctypes.c_int, P, vp, sz, vp],
            "ns_batched_noalloc": [M, ctypes.c_int, ctypes.c_int, P, vp],
            "ns_gram_sharded_workspace_size": [M, ctypes.c_int, P, ctypes.POINTER(sz)],
            "ns_gram_sharded": [M, ctypes.c_int, P, vp, sz, vp],
            "ns_muon_workspace_size": [ctypes.POINTER(_MuonMatrix), ctypes.c_int, P,
                                       ctypes.POINTER(sz)],
            "ns_muon_step": [ctypes.POINTER(_MuonMatrix), ctypes.c_int, P, ctypes.c_float,
                             ctypes.c_float, vp, sz, vp],
            "ns_syrk": [vp, i64, i64, vp, vp, sz, vp],
            "ns_gemm_nt": [vp, vp, vp, vp, i64, i64, i64, ctypes.c_float, ctypes.c_float,
                           ctypes.c_float, ctypes.c_int, vp, sz, vp],
            "ns_gemm_grouped_workspace_size": [ctypes.c_int, ctypes.POINTER(sz)],
            "ns_gemm_grouped": [ctypes.POINTER(_GemmProblem), ctypes.c_int, ctypes.c_int, vp, sz,
                                vp],
            "ns_plan_check": [ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, P,
                              vp, sz, ctypes.c_int, ctypes.c_char_p, sz],
        }
        for name, args in sigs.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.ns_timing_enable.argtypes = [ctypes.c_int]
        lib.ns_timing_enable.restype = ctypes.c_int
        lib.ns_timing_read.argtypes = [ctypes.POINTER(TimingReport)]
        lib.ns_timing_read.restype = ctypes.c_int
        lib.ns_status_string.argtypes = [ctypes.c_int]
        lib.ns_status_string.restype = ctypes.c_char_p
        lib.ns_backend_info.argtypes = []
        lib.ns_backend_info.restype = ctypes.c_char_p
        lib.ns_backend_status.argtypes = [ctypes.POINTER(_BackendStatus)]
        lib.ns_backend_status.restype = ctypes.c_int
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().ns_status_string(status).decode()


def ns_backend_info() -> str:
    return library().ns_backend_info().decode()


def get_ns_backend() -> str:
    """One-line summary for start-up logs (the page's get_ns_backend())."""
    return ns_backend_info()


def get_backend_status() -> dict:
    """Diagnostics dictionary (the page's get_backend_status()).

    ``auto_choice`` is the kernel set every call runs ("hip-mfma-f16") or
    None when no gfx950 device is visible; ``deterministic`` is always True.
    """
    st = _BackendStatus()
    _check(library().ns_backend_status(ctypes.byref(st)), "ns_backend_status")
    found = bool(st.device_found)
    return {
        "arch": st.arch.decode(),
        "device_index": st.device_index,
        "compute_units": st.compute_units,
        "clock_mhz": st.clock_mhz,
        "gfx950_available": found,
        "auto_choice": "hip-mfma-f16" if found else None,
        "kernel": st.kernel.decode(),
        "deterministic": bool(st.deterministic),
        "gemm_tile": st.gemm_tile,
        "version": st.version,
    }


def ns_timing_enable(enable: bool = True) -> None:
    """Bracket every library launch with HIP events (see ns_timing_read)."""
    _check(library().ns_timing_enable(1 if enable else 0), "ns_timing_enable")


def ns_timing_read() -> dict:
    """Kernel time and algorithmic work recorded since the last read."""
    r = TimingReport()
    _check(library().ns_timing_read(ctypes.byref(r)), "ns_timing_read")
    return r.as_dict()


def _check(status: int, where: str) -> None:
    if status != NS_OK:
        raise NsError(status, where)


# ------------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _dtype_code(dtype) -> int:
    torch = _torch()
    codes = {torch.float32: NS_DT_F32, torch.bfloat16: NS_DT_BF16,
             torch.float16: NS_DT_F16}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}")
    return codes[dtype]


def _rowmajor_ld(t) -> int:
    """Leading dimension of a row-major 2-D view. Rows must be contiguous and
    must not overlap (an expanded or otherwise aliased view would make the
    library read or write past the storage it covers)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"row stride {t.stride(0)} is smaller than the row length "
                         f"{t.shape[1]} (overlapping rows, e.g. an expanded view)")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _device_tensor(t, name: str):
    """A tensor on the current HIP device (where the library launches)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    cur = _torch().cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{name} is on {t.device} but the current device is cuda:{cur}; "
                         f"the library runs on the current device")
    return t


def _stream_ptr(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _params(coefficients, restart_iterations, eps):
    coeffs = [float(x) for row in coefficients for x in row]
    if len(coeffs) % 3:
        raise ValueError("coefficients must be rows of (a, b, c)")
    rs = [int(i) for i in restart_iterations]
    carr = (ctypes.c_float * max(1, len(coeffs)))(*coeffs)
    rarr = (ctypes.c_int * max(1, len(rs)))(*rs)
    p = _Params(len(coeffs) // 3, carr, rarr, len(rs), float(eps))
    return p, (carr, rarr)  # keep the arrays alive


def _matrix(G, out) -> _Matrix:
    if tuple(out.shape) != tuple(G.shape):
        raise ValueError(f"output shape {tuple(out.shape)} differs from input shape "
                         f"{tuple(G.shape)}")
    return _Matrix(G.data_ptr(), _dtype_code(G.dtype), G.shape[0], G.shape[1],
                   _rowmajor_ld(G), out.data_ptr(), _dtype_code(out.dtype),
                   _rowmajor_ld(out))


def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def ns_workspace_size(shapes: Sequence[Sequence[int]], backend: str = "gram",
                      coefficients=POLAR_EXPRESS_COEFFICIENTS,
                      restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                      eps: float = DEFAULT_EPS) -> int:
    """Workspace bytes for matrices of the given (m, n) shapes."""
    mats = (_Matrix * len(shapes))()
    for i, (m, n) in enumerate(shapes):
        mats[i] = _Matrix(None, NS_DT_F32, m, n, n, None, NS_DT_F16, n)
    p, keep = _params(coefficients, restart_iterations, eps)
    nbytes = ctypes.c_size_t(0)
    _check(library().ns_workspace_size(mats, len(shapes), BACKENDS[backend],
                                       ctypes.byref(p), ctypes.byref(nbytes)),
           "ns_workspace_size")
    return nbytes.value


def ns_batched(Gs: List, backend: str = "gram",
               coefficients=POLAR_EXPRESS_COEFFICIENTS,
               restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
               eps: float = DEFAULT_EPS, out_dtype=None, outs: Optional[List] = None,
               workspace=None) -> List:
    """NS on a list of GPU matrices in one grouped call; returns the outputs."""
    torch = _torch()
    if len(Gs) == 0:
        return []
    dev = Gs[0].device
    out_dtype = out_dtype or torch.float16
    for G in Gs:
        _device_tensor(G, "G")
    if outs is None:
        outs = [torch.empty(G.shape, dtype=out_dtype, device=dev) for G in Gs]
    mats = (_Matrix * len(Gs))()
    for i, (G, O) in enumerate(zip(Gs, outs)):
        mats[i] = _matrix(G, _device_tensor(O, "out"))
    p, keep = _params(coefficients, restart_iterations, eps)
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_workspace_size(mats, len(Gs), BACKENDS[backend], ctypes.byref(p),
                                 ctypes.byref(nbytes)), "ns_workspace_size")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = _workspace(nbytes.value, dev)
    _check(lib.ns_batched(mats, len(Gs), BACKENDS[backend], ctypes.byref(p),
                          workspace.data_ptr(), workspace.numel(), _stream_ptr(Gs[0])),
           "ns_batched")
    return outs


NS_NOALLOC_SCRATCH_BYTES = 128 << 20


def ns_batched_noalloc(Gs: List, outs: List, backend: str = "gram",
                       coefficients=POLAR_EXPRESS_COEFFICIENTS,
                       restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                       eps: float = DEFAULT_EPS) -> List:
    """ns_batched with the library's static device scratch as the workspace
    (nothing is allocated; the caller passes the outputs). Calls that
    overlap on one device race; see ns_batched_noalloc in ns.h."""
    if len(Gs) != len(outs):
        raise ValueError("one output per input")
    if len(Gs) == 0:
        return outs
    mats = (_Matrix * len(Gs))()
    for i, (G, O) in enumerate(zip(Gs, outs)):
        mats[i] = _matrix(_device_tensor(G, "G"), _device_tensor(O, "out"))
    p, keep = _params(coefficients, restart_iterations, eps)
    _check(library().ns_batched_noalloc(mats, len(Gs), BACKENDS[backend], ctypes.byref(p),
                                        _stream_ptr(Gs[0])), "ns_batched_noalloc")
    return outs


def ns_gram(G, coefficients=POLAR_EXPRESS_COEFFICIENTS,
            restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
            eps: float = DEFAULT_EPS, out_dtype=None, out=None, workspace=None):
    """Gram-space NS of one GPU matrix (the page's newton_schulz)."""
    torch = _torch()
    _device_tensor(G, "G")
    out = out if out is not None else torch.empty(
        G.shape, dtype=out_dtype or torch.float16, device=G.device)
    mat = _matrix(G, _device_tensor(out, "out"))
    p, keep = _params(coefficients, restart_iterations, eps)
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_workspace_size(ctypes.byref(mat), 1, NS_GRAM, ctypes.byref(p),
                                 ctypes.byref(nbytes)), "ns_workspace_size")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = _workspace(nbytes.value, G.device)
    _check(lib.ns_gram(ctypes.byref(mat), ctypes.byref(p), workspace.data_ptr(),
                       workspace.numel(), _stream_ptr(G)), "ns_gram")
    return out


def ns_gram_sharded(G, shards: int, coefficients=POLAR_EXPRESS_COEFFICIENTS,
                    restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                    eps: float = DEFAULT_EPS, out_dtype=None):
    """Gram NS of one matrix along the column-sharded (tensor-parallel) route,
    with `shards` virtual shards on this device (see ns_gram_sharded in ns.h)."""
    torch = _torch()
    _device_tensor(G, "G")
    out = torch.empty(G.shape, dtype=out_dtype or torch.float16, device=G.device)
    mat = _matrix(G, out)
    p, keep = _params(coefficients, restart_iterations, eps)
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_gram_sharded_workspace_size(ctypes.byref(mat), int(shards), ctypes.byref(p),
                                              ctypes.byref(nbytes)),
           "ns_gram_sharded_workspace_size")
    ws = _workspace(nbytes.value, G.device)
    _check(lib.ns_gram_sharded(ctypes.byref(mat), int(shards), ctypes.byref(p), ws.data_ptr(),
                               ws.numel(), _stream_ptr(G)), "ns_gram_sharded")
    return out


def ns_muon_step(grads: List, momenta: List, params: List, beta: float, lr: float,
                 scales: Optional[List[float]] = None,
                 coefficients=POLAR_EXPRESS_COEFFICIENTS,
                 restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                 eps: float = DEFAULT_EPS, workspace=None) -> None:
    """One Muon step, in place: M <- beta M + G, W <- W - lr * scale * NS(M)
    (Gram backend; see ns_muon_step in ns.h for the reading and the fusion)."""
    if not (len(grads) == len(momenta) == len(params)):
        raise ValueError("grads, momenta and params must have the same length")
    if len(grads) == 0:
        return
    scales = [1.0] * len(grads) if scales is None else list(scales)
    if len(scales) != len(grads):
        raise ValueError("one scale per matrix")
    mats = (_MuonMatrix * len(grads))()
    for i, (G, M, W) in enumerate(zip(grads, momenta, params)):
        for t, name in ((G, "grad"), (M, "momentum"), (W, "param")):
            _device_tensor(t, name)
            if tuple(t.shape) != tuple(G.shape):
                raise ValueError(f"{name} {i} has shape {tuple(t.shape)}, grad {tuple(G.shape)}")
        m, n = G.shape
        mats[i] = _MuonMatrix(G.data_ptr(), _dtype_code(G.dtype), m, n, _rowmajor_ld(G),
                              M.data_ptr(), _dtype_code(M.dtype), _rowmajor_ld(M),
                              W.data_ptr(), _dtype_code(W.dtype), _rowmajor_ld(W),
                              float(scales[i]))
    p, keep = _params(coefficients, restart_iterations, eps)
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_muon_workspace_size(mats, len(grads), ctypes.byref(p), ctypes.byref(nbytes)),
           "ns_muon_workspace_size")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = _workspace(nbytes.value, grads[0].device)
    _check(lib.ns_muon_step(mats, len(grads), ctypes.byref(p), float(beta), float(lr),
                            workspace.data_ptr(), workspace.numel(), _stream_ptr(grads[0])),
           "ns_muon_step")


def ns_direct(G, coefficients=POLAR_EXPRESS_COEFFICIENTS, eps: float = DEFAULT_EPS,
              out_dtype=None, out=None, workspace=None):
    """Direct-space NS of one GPU matrix (the page's direct_newton_schulz)."""
    torch = _torch()
    _device_tensor(G, "G")
    out = out if out is not None else torch.empty(
        G.shape, dtype=out_dtype or torch.float16, device=G.device)
    mat = _matrix(G, _device_tensor(out, "out"))
    p, keep = _params(coefficients, (), eps)
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_workspace_size(ctypes.byref(mat), 1, NS_DIRECT, ctypes.byref(p),
                                 ctypes.byref(nbytes)), "ns_workspace_size")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = _workspace(nbytes.value, G.device)
    _check(lib.ns_direct(ctypes.byref(mat), ctypes.byref(p), workspace.data_ptr(),
                         workspace.numel(), _stream_ptr(G)), "ns_direct")
    return out


def ns_normalize(G, eps: float = DEFAULT_EPS, transpose_tall: bool = True,
                 return_norm: bool = False):
    """fp16(G / (||G||_F + eps)); tall inputs come back transposed."""
    torch = _torch()
    _device_tensor(G, "G")
    m, n = G.shape
    tr = transpose_tall and m > n
    x = torch.empty((n, m) if tr else (m, n), dtype=torch.float16, device=G.device)
    norm = torch.empty(1, dtype=torch.float32, device=G.device)
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_normalize_workspace_size(m, n, ctypes.byref(nbytes)),
           "ns_normalize_workspace_size")
    ws = _workspace(nbytes.value, G.device)
    _check(lib.ns_normalize(G.data_ptr(), _dtype_code(G.dtype), m, n, _rowmajor_ld(G),
                            x.data_ptr(), x.shape[1], 1 if transpose_tall else 0,
                            float(eps), norm.data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream_ptr(G)), "ns_normalize")
    return (x, norm) if return_norm else x


def ns_syrk(X):
    """R = X X^T for an fp16 (s, l) GPU matrix (s % 256 == 0, l % 64 == 0)."""
    torch = _torch()
    if X.dim() != 2 or X.dtype != torch.float16:
        raise ValueError("X must be a 2-D fp16 tensor")
    _device_tensor(X, "X")
    X = X.contiguous()
    s, l = X.shape
    R = torch.empty((s, s), dtype=torch.float16, device=X.device)
    ws = _workspace(NS_UNIT_WORKSPACE_BYTES, X.device)
    _check(library().ns_syrk(X.data_ptr(), s, l, R.data_ptr(), ws.data_ptr(), ws.numel(),
                             _stream_ptr(X)), "ns_syrk")
    return R


def ns_gemm_nt(A, B, C=None, alpha: float = 1.0, beta: float = 0.0,
               gamma: float = 0.0, symmetric: bool = False):
    """alpha A B^T + beta C + gamma I on fp16 GPU matrices."""
    torch = _torch()
    for name, t in (("A", A), ("B", B), ("C", C)):
        if t is not None and (t.dim() != 2 or t.dtype != torch.float16):
            raise ValueError(f"{name} must be a 2-D fp16 tensor")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"B has {B.shape[1]} columns, A has {K}")
    if C is not None and tuple(C.shape) != (M, N):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(M, N)}")
    A, B = _device_tensor(A, "A").contiguous(), _device_tensor(B, "B").contiguous()
    if C is not None:
        C = _device_tensor(C, "C").contiguous()
    D = torch.empty((M, N), dtype=torch.float16, device=A.device)
    cptr = C.data_ptr() if C is not None else None
    ws = _workspace(NS_UNIT_WORKSPACE_BYTES, A.device)
    _check(library().ns_gemm_nt(A.data_ptr(), B.data_ptr(), cptr, D.data_ptr(), M, N, K,
                                alpha, beta, gamma, 1 if symmetric else 0, ws.data_ptr(),
                                ws.numel(), _stream_ptr(A)), "ns_gemm_nt")
    return D


def ns_gemm_grouped(problems: List[dict], tile_edge: int = 0) -> None:
    """Products of the grouped GEMM kernel with every descriptor option, in
    one launch (kernel-level testing; see ns_gemm_problem in ns.h).

    Each problem is a dict: "a", "b", "d" (GPU tensors; a and b fp16 holding
    M*K and N*K elements in the layout their *_pairs flag names, a as
    (K, M) and b as (K, N) if "a_kmajor" / "b_kmajor"), optional "c", "d2",
    "dt", the sizes "M", "N", "K", and optionally "ldc", "ldd" (default N),
    "valid_m", "valid_n" (default M, N), "diag_n" (default 0), "symmetric",
    "c_is_bt", "a_pairs", "b_pairs", "c_pairs", "d_pairs", "a_kmajor",
    "b_kmajor" (default 0), "alpha" (1), "beta", "gamma", "delta" (0).
    tile_edge: 256 or 64 forces that kernel, 0 picks as the iteration's
    stages do."""
    if not problems:
        return
    arr = (_GemmProblem * len(problems))()
    dev = problems[0]["a"].device
    for i, q in enumerate(problems):
        for key in ("a", "b", "c", "d", "d2", "dt"):
            if q.get(key) is not None:
                _device_tensor(q[key], key)
        M, N = int(q["M"]), int(q["N"])
        c = q.get("c")
        arr[i] = _GemmProblem(
            q["a"].data_ptr(), q["b"].data_ptr(), c.data_ptr() if c is not None else None,
            q["d"].data_ptr(),
            q["d2"].data_ptr() if q.get("d2") is not None else None,
            q["dt"].data_ptr() if q.get("dt") is not None else None,
            M, N, int(q["K"]), int(q.get("ldc", N)), int(q.get("ldd", N)),
            int(q.get("valid_m", M)), int(q.get("valid_n", N)), int(q.get("diag_n", 0)),
            _dtype_code(c.dtype) if c is not None else NS_DT_F16, _dtype_code(q["d"].dtype),
            int(q.get("symmetric", 0)), int(q.get("c_is_bt", 0)),
            int(q.get("a_pairs", 0)), int(q.get("b_pairs", 0)),
            int(q.get("c_pairs", 0)), int(q.get("d_pairs", 0)),
            int(q.get("a_kmajor", 0)), int(q.get("b_kmajor", 0)),
            float(q.get("alpha", 1.0)), float(q.get("beta", 0.0)),
            float(q.get("gamma", 0.0)), float(q.get("delta", 0.0)))
    lib = library()
    nbytes = ctypes.c_size_t(0)
    _check(lib.ns_gemm_grouped_workspace_size(len(problems), ctypes.byref(nbytes)),
           "ns_gemm_grouped_workspace_size")
    ws = _workspace(nbytes.value, dev)
    _check(lib.ns_gemm_grouped(arr, len(problems), int(tile_edge), ws.data_ptr(), ws.numel(),
                               _stream_ptr(problems[0]["a"])), "ns_gemm_grouped")


def ns_plan_check(entry: int, mats, backend: str = "gram", shards: int = 1,
                  coefficients=POLAR_EXPRESS_COEFFICIENTS,
                  restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                  eps: float = DEFAULT_EPS, ws: int = 1 << 40, ws_bytes: int = 0,
                  plant: int = 0):
    """Host-side bounds check of a call's launch plan (no device needed).

    mats: a list of _Matrix (NS_CHECK_BATCHED, NS_CHECK_SHARDED) or
    _MuonMatrix (NS_CHECK_MUON) records whose pointers are plain addresses
    (never dereferenced). Returns (status, message)."""
    typ = _MuonMatrix if entry == NS_CHECK_MUON else _Matrix
    arr = (typ * len(mats))(*mats)
    p, keep = _params(coefficients, restart_iterations, eps)
    msg = ctypes.create_string_buffer(512)
    st = library().ns_plan_check(entry, ctypes.cast(arr, ctypes.c_void_p), len(mats),
                                 BACKENDS[backend], int(shards), ctypes.byref(p), ws,
                                 ws_bytes, int(plant), msg, 512)
    return st, msg.value.decode()


def newton_schulz(G, backend: str = "gram", coefficients=POLAR_EXPRESS_COEFFICIENTS,
                  restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                  eps: float = DEFAULT_EPS, out_dtype=None):
    """Dispatch on the page's algorithm axis ("gram" or "direct")."""
    if backend == "gram":
        return ns_gram(G, coefficients, restart_iterations, eps, out_dtype)
    if backend == "direct":
        return ns_direct(G, coefficients, eps, out_dtype)
    raise ValueError(f"unknown backend {backend!r}")


KERNELS = ("auto", "hip-mfma-f16")


class NewtonSchulz:
    """Configured NS operator (the page's NewtonSchulz(...) object).

    backend: "gram" or "direct" (the algorithm axis). kernel: "auto" or
    "hip-mfma-f16"; this library has one kernel set, so any other explicit
    kernel name (the page's CUDA kernels among them) raises at construction,
    as the page specifies for an unavailable explicit kernel, and so does an
    explicit "hip-mfma-f16" when no gfx950 device is visible. deterministic:
    accepted for interface parity; every call is bitwise reproducible anyway.
    """

    def __init__(self, backend: str = "gram", kernel: str = "auto",
                 coefficients=POLAR_EXPRESS_COEFFICIENTS,
                 restart_iterations: Iterable[int] = DEFAULT_RESTARTS,
                 eps: float = DEFAULT_EPS, deterministic: bool = True):
        if backend not in ("gram", "direct"):
            raise ValueError(f"unknown backend {backend!r} (expected 'gram' or 'direct')")
        if kernel not in KERNELS:
            raise ValueError(f"kernel {kernel!r} is not available in this library "
                             f"(available: {', '.join(KERNELS)})")
        library()   # fails loudly when the library has not been built
        if kernel != "auto" and not get_backend_status()["gfx950_available"]:
            raise RuntimeError(f"kernel {kernel!r} needs a gfx950 device")
        self.backend = backend
        self.kernel = "hip-mfma-f16"
        self.coefficients = tuple(tuple(float(x) for x in row) for row in coefficients)
        self.restart_iterations = tuple(int(i) for i in restart_iterations)
        self.eps = float(eps)
        self.deterministic = True
        # validate the table and restart indices once, on the host
        ns_workspace_size([(1, 1)], backend, self.coefficients, self.restart_iterations,
                          self.eps)

    def __call__(self, G, out_dtype=None):
        return newton_schulz(G, self.backend, self.coefficients, self.restart_iterations,
                             self.eps, out_dtype)

    def batched(self, Gs, outs=None, workspace=None, out_dtype=None):
        return ns_batched(Gs, self.backend, self.coefficients, self.restart_iterations,
                          self.eps, outs=outs, workspace=workspace, out_dtype=out_dtype)

    def __repr__(self):
        return (f"NewtonSchulz(backend={self.backend!r}, kernel={self.kernel!r}, "
                f"steps={len(self.coefficients)}, restarts={self.restart_iterations})")

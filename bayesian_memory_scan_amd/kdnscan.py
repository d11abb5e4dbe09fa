"""Python binding of libkdnscan: precision-tracking memory scans on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libkdnscan.so; torch supplies device memory and the current
stream.  The functions carry the C names and follow include/kdnscan.h.

If the library has not been built this module raises at import: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "lib", "LIB_PATH", "KDN_OK", "KDN_EINVAL", "KDN_EUNSUPPORTED", "KDN_EWORKSPACE", "KDN_EHIP",
    "KDN_F32", "KDN_BF16", "KdnError",
    "kdn_diag_scan_fwd", "kdn_diag_scan_bwd", "kdn_diag_noise_scan_fwd", "kdn_diag_scan_varlen_fwd",
    "kdn_mobius_precision_scan", "kdn_decode_step",
    "kdn_diag_plan", "kdn_set_diag_segments", "kdn_status_string", "kdn_last_hip_error",
    "header_functions",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdnscan.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "kdnscan.h")

KDN_OK, KDN_EINVAL, KDN_EUNSUPPORTED, KDN_EWORKSPACE, KDN_EHIP = 0, -1, -2, -3, -4
KDN_F32, KDN_BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python -m bayesian_memory_scan_amd._build). There is no CPU fallback.")

# torch ships its own HIP runtime (same SONAME as the system one).  Load torch
# first so that libkdnscan binds to that single runtime instance: streams and
# device pointers from torch are then valid in the library.
try:
    import torch as _torch_mod  # noqa: F401
except ImportError:  # pragma: no cover - CPU-only validation use
    _torch_mod = None

lib = ctypes.CDLL(LIB_PATH)

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_f = ctypes.c_float
_szp = ctypes.POINTER(ctypes.c_size_t)

lib.kdn_diag_scan_fwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _szp, _vp]
lib.kdn_diag_scan_fwd.restype = ctypes.c_int
lib.kdn_diag_scan_varlen_fwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                         _vp, _vp, _vp, _vp, _szp, _vp]
lib.kdn_diag_scan_varlen_fwd.restype = ctypes.c_int
lib.kdn_diag_noise_scan_fwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.kdn_diag_noise_scan_fwd.restype = ctypes.c_int
lib.kdn_diag_scan_bwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                  _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _szp, _vp]
lib.kdn_diag_scan_bwd.restype = ctypes.c_int
lib.kdn_mobius_precision_scan.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                          _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _szp, _vp]
lib.kdn_mobius_precision_scan.restype = ctypes.c_int
lib.kdn_decode_step.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                _vp, _f, _vp, _vp, _vp, _vp]
lib.kdn_decode_step.restype = ctypes.c_int
lib.kdn_diag_plan.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_i32),
                              ctypes.POINTER(_i32), ctypes.POINTER(_i64), _i32]
lib.kdn_diag_plan.restype = ctypes.c_int
lib.kdn_set_diag_segments.argtypes = [_i32]
lib.kdn_set_diag_segments.restype = _i32
lib.kdn_status_string.argtypes = [ctypes.c_int]
lib.kdn_status_string.restype = ctypes.c_char_p
lib.kdn_last_hip_error.argtypes = []
lib.kdn_last_hip_error.restype = ctypes.c_char_p


class KdnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        extra = f"; HIP: {lib.kdn_last_hip_error().decode()}" if code == KDN_EHIP else ""
        super().__init__(f"{fn} failed: {code} ({kdn_status_string(code)}){extra}")
        self.code = code


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions include/kdnscan.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(kdn_\w+)\s*\(", text, re.M)))


def kdn_last_hip_error() -> str:
    return lib.kdn_last_hip_error().decode()


def kdn_status_string(code: int) -> str:
    return lib.kdn_status_string(int(code)).decode()


def kdn_set_diag_segments(segments: int) -> int:
    return int(lib.kdn_set_diag_segments(int(segments)))


def kdn_diag_plan(B: int, H: int, T: int, d_k: int, d_v: int):
    """(chunk, segments, segment token bounds) the library uses for this shape."""
    chunk, segs = _i32(), _i32()
    rc = lib.kdn_diag_plan(B, H, T, d_k, d_v, ctypes.byref(chunk), ctypes.byref(segs), None, 0)
    if rc != KDN_OK:
        raise KdnError("kdn_diag_plan", rc)
    bounds = (_i64 * (segs.value + 1))()
    rc = lib.kdn_diag_plan(B, H, T, d_k, d_v, None, None, bounds, segs.value)
    if rc != KDN_OK:
        raise KdnError("kdn_diag_plan", rc)
    return chunk.value, segs.value, list(bounds)


# ---------------------------------------------------------------------------
# torch-tensor front ends (device memory and stream plumbing only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtypes, device):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(fn, args, device):
    """Query the workspace size, allocate it with torch, return (tensor, size)."""
    torch = _torch()
    need = ctypes.c_size_t(0)
    rc = fn(*args(None, ctypes.byref(need)))
    if rc != KDN_OK:
        raise KdnError(fn.__name__, rc)
    if need.value == 0:
        return None, need
    ws = torch.empty(need.value, dtype=torch.uint8, device=device)
    return ws, need


def _nbytes(ws, need):
    """Size argument of a run call: NULL when no workspace is passed (a NULL
    workspace with a non-NULL size pointer would be a size query)."""
    return None if ws is None else ctypes.byref(need)


def _in_dtype(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return KDN_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return KDN_BF16  # int16/uint16 tensors are read as raw bf16 bits
    raise TypeError(f"unsupported input dtype {t.dtype}")


def kdn_diag_scan_fwd(q, k, v, beta, d, A, I_prior, I0=None, mu0=None,
                      o=None, I_T=None, mu_T=None, want_state=True, stream=None):
    """Diagonal-precision scan forward on [B,H,T,.] CUDA tensors.

    q, k [B,H,T,d_k]; v, beta [B,H,T,d_v]; d [B,H,T] (all float32, or all
    bfloat16 / raw-bf16 int16); A [H] float32; I_prior float; optional I0, mu0
    [B,H,d_k,d_v] float32.  beta None selects Palimpsa-M gating (beta_t = d_t).
    Returns (o, I_T, mu_T) (states None when want_state is False).
    """
    torch = _torch()
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)
    for n, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)):
        _check(t, n, dts, dev)
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, k, v, beta, d must share one dtype")
    f32 = (torch.float32,)
    _check(A, "A", f32, dev)
    _check(I0, "I0", f32, dev)
    _check(mu0, "mu0", f32, dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    if want_state:
        I_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if I_T is None else I_T
        mu_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if mu_T is None else mu_T
    st = _stream(stream)

    def args(ws, nbytes):
        return (B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(o), _ptr(I_T), _ptr(mu_T),
                ws, nbytes, st)

    ws, need = _workspace(lib.kdn_diag_scan_fwd, args, dev)
    rc = lib.kdn_diag_scan_fwd(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_fwd", rc)
    return o, I_T, mu_T


def kdn_diag_scan_varlen_fwd(q, k, v, beta, d, A, I_prior, cu_seqlens, I0=None, mu0=None,
                             want_state=True, stream=None):
    """Diagonal scan over a packed variable-length batch.

    q, k [H,total_T,d_k]; v, beta [H,total_T,d_v]; d [H,total_T] (float32 or
    bf16; beta None = Palimpsa-M gating); cu_seqlens int64 [N+1] on the device;
    I0, mu0 [N,H,d_k,d_v] float32 or None.  Returns (o [H,total_T,d_v], I_T,
    mu_T [N,H,d_k,d_v]).
    """
    torch = _torch()
    dev = q.device
    H, T, dk = q.shape
    dv = v.shape[-1]
    dts = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)
    for n, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)):
        _check(t, n, dts, dev)
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, k, v, beta, d must share one dtype")
    _check(cu_seqlens, "cu_seqlens", (torch.int64,), dev)
    for n, t in (("A", A), ("I0", I0), ("mu0", mu0)):
        _check(t, n, (torch.float32,), dev)
    N = cu_seqlens.numel() - 1
    o = torch.empty((H, T, dv), dtype=torch.float32, device=dev)
    I_T = mu_T = None
    if want_state:
        I_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        mu_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    st = _stream(stream)

    def args(ws, nbytes):
        return (N, H, T, dk, dv, _in_dtype(q), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                _ptr(beta), _ptr(d), _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(o),
                _ptr(I_T), _ptr(mu_T), ws, nbytes, st)

    ws, need = _workspace(lib.kdn_diag_scan_varlen_fwd, args, dev)
    rc = lib.kdn_diag_scan_varlen_fwd(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_varlen_fwd", rc)
    return o, I_T, mu_T


def kdn_diag_noise_scan_fwd(q, k, v, beta, a, p, lambda0=None, mu0=None, want_state=True,
                            stream=None):
    """Diagonal KDN with process noise on [B,H,T,.] CUDA tensors.

    q, k [B,H,T,d_k]; v, beta [B,H,T,d_v] (float32 or bf16); a, p [B,H,T]
    float32; optional lambda0, mu0 [B,H,d_k,d_v] float32.  Returns
    (o, lambda_T, mu_T) (states None when want_state is False).
    """
    torch = _torch()
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)
    for n, t in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        _check(t, n, dts, dev)
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, beta must share one dtype")
    for n, t in (("a", a), ("p", p), ("lambda0", lambda0), ("mu0", mu0)):
        _check(t, n, (torch.float32,), dev)
    o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    lam_T = mu_T = None
    if want_state:
        lam_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        mu_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    rc = lib.kdn_diag_noise_scan_fwd(B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(beta), _ptr(a), _ptr(p), _ptr(lambda0), _ptr(mu0),
                                     _ptr(o), _ptr(lam_T), _ptr(mu_T), _stream(stream))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_noise_scan_fwd", rc)
    return o, lam_T, mu_T


def kdn_diag_scan_bwd(q, k, v, beta, d, A, I_prior, d_o, I0=None, mu0=None, d_I_T=None,
                      d_mu_T=None, want_prior=True, stream=None):
    """Gradient of kdn_diag_scan_fwd for L = sum(d_o o) + sum(d_I_T I_T) + sum(d_mu_T mu_T).

    Inputs as for the forward call plus d_o [B,H,T,d_v] and optional d_I_T,
    d_mu_T [B,H,d_k,d_v] (all float32).  Returns a dict of float32 tensors:
    dq, dk [B,H,T,d_k]; dv, dbeta [B,H,T,d_v]; dd [B,H,T]; dA [H];
    dI_prior [1] (when want_prior); dI0 / dmu0 [B,H,d_k,d_v] when I0 / mu0
    are given.
    """
    torch = _torch()
    dev = q.device
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)
    for n, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)):
        _check(t, n, dts, dev)
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, k, v, beta, d must share one dtype")
    f32 = (torch.float32,)
    for n, t in (("A", A), ("d_o", d_o), ("I0", I0), ("mu0", mu0), ("d_I_T", d_I_T),
                 ("d_mu_T", d_mu_T)):
        _check(t, n, f32, dev)
    new = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    g = {"dq": new(B, H, T, dk), "dk": new(B, H, T, dk), "dv": new(B, H, T, dv),
         "dd": new(B, H, T), "dA": new(H)}
    if beta is not None:   # beta None: Palimpsa-M gating, whose beta share is in dd
        g["dbeta"] = new(B, H, T, dv)
    if want_prior:
        g["dI_prior"] = new(1)
    if I0 is not None:
        g["dI0"] = new(B, H, dk, dv)
    if mu0 is not None:
        g["dmu0"] = new(B, H, dk, dv)
    st = _stream(stream)
    o = lambda n: _ptr(g.get(n))

    def args(ws, nbytes):
        return (B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(d_o), _ptr(d_I_T),
                _ptr(d_mu_T), o("dq"), o("dk"), o("dv"), o("dbeta"), o("dd"), o("dA"),
                o("dI_prior"), o("dI0"), o("dmu0"), ws, nbytes, st)

    ws, need = _workspace(lib.kdn_diag_scan_bwd, args, dev)
    rc = lib.kdn_diag_scan_bwd(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_bwd", rc)
    return g


def kdn_mobius_precision_scan(a, p, Lam, lambda0=None, q=None, k=None, v=None, mu0=None,
                              want_lambda=True, want_state=True, stream=None):
    """Isotropic filter: Mobius precision scan, then (if q, k, v given) the gated mean scan.

    a, p, Lam [B,H,T] float32; lambda0 [B,H] or None (-> 1); q, k [B,H,T,d_k],
    v [B,H,T,d_v], mu0 [B,H,d_k,d_v] float32.  Returns (lambda, o, mu_T).
    """
    torch = _torch()
    dev = a.device
    B, H, T = a.shape
    f32 = (torch.float32,)
    for n, t in (("a", a), ("p", p), ("Lambda", Lam), ("lambda0", lambda0), ("q", q), ("k", k),
                 ("v", v), ("mu0", mu0)):
        _check(t, n, f32, dev)
    lam = torch.empty((B, H, T), dtype=torch.float32, device=dev) if want_lambda else None
    dk = dv = 0
    o = mu_T = None
    if q is not None:
        dk, dv = q.shape[-1], v.shape[-1]
        o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
        if want_state:
            mu_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    st = _stream(stream)

    def args(ws, nbytes):
        return (B, H, T, _ptr(a), _ptr(p), _ptr(Lam), _ptr(lambda0), _ptr(lam), dk, dv,
                _ptr(q), _ptr(k), _ptr(v), _ptr(mu0), _ptr(o), _ptr(mu_T), ws, nbytes, st)

    ws, need = _workspace(lib.kdn_mobius_precision_scan, args, dev)
    rc = lib.kdn_mobius_precision_scan(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_mobius_precision_scan", rc)
    return lam, o, mu_T


def kdn_decode_step(q, k, v, beta, d, A, I_prior, I, mu, o=None, stream=None):
    """One decode token: q, k [B,H,d_k]; v, beta [B,H,d_v]; d [B,H]; I, mu
    [B,H,d_k,d_v] float32 updated in place.  Returns o [B,H,d_v]."""
    torch = _torch()
    dev = q.device
    B, H, dk = q.shape
    dv = v.shape[-1]
    dts = (torch.float32, torch.bfloat16, torch.int16, torch.uint16)
    for n, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)):
        _check(t, n, dts, dev)
    f32 = (torch.float32,)
    for n, t in (("A", A), ("I", I), ("mu", mu)):
        _check(t, n, f32, dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    rc = lib.kdn_decode_step(B, H, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                             _ptr(d), _ptr(A), float(I_prior), _ptr(I), _ptr(mu), _ptr(o),
                             _stream(stream))
    if rc != KDN_OK:
        raise KdnError("kdn_decode_step", rc)
    return o

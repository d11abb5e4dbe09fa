"""Python binding of libkdnscan: precision-tracking memory scans on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libkdnscan.so; torch supplies device memory and streams.  The
functions carry the C names and follow include/kdnscan.h.

Before any call reaches the library, the tensor front ends check every
tensor's shape against the sizes taken from q and v (or from a, p, Lambda),
its dtype and its device, and raise ValueError / TypeError: the C ABI takes
bare pointers and cannot detect an undersized buffer.  Outputs and workspace
are allocated on the stream the kernels are enqueued on, so the caching
allocator never hands them to other work while the kernels run.

If the library has not been built this module raises at import: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "lib", "LIB_PATH", "KDN_OK", "KDN_EINVAL", "KDN_EUNSUPPORTED", "KDN_EWORKSPACE", "KDN_EHIP",
    "KDN_ESCRATCH", "KDN_F32", "KDN_BF16", "KDN_ECHO_WORDS", "KdnError", "ScanOpts",
    "kdn_diag_scan_fwd", "kdn_diag_scan_fwd_noalloc", "kdn_diag_scan_bwd", "kdn_diag_noise_scan_fwd",
    "kdn_diag_scan_varlen_fwd", "kdn_diag_scan_varlen_bwd",
    "kdn_mobius_precision_scan", "kdn_decode_step",
    "kdn_diag_plan", "kdn_diag_varlen_plan", "kdn_status_string", "kdn_last_hip_error",
    "header_functions",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdnscan.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "kdnscan.h")

KDN_OK, KDN_EINVAL, KDN_EUNSUPPORTED, KDN_EWORKSPACE, KDN_EHIP, KDN_ESCRATCH = 0, -1, -2, -3, -4, -5
KDN_F32, KDN_BF16 = 0, 1
KDN_ECHO_WORDS = 8

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


class ScanOpts(ctypes.Structure):
    """kdn_scan_opts: per-call segment request, bounds echo and main-pass events."""
    _fields_ = [("segments", _i32), ("reserved", _i32), ("bounds_echo", _vp),
                ("echo_capacity", _i64), ("echo_words", _i64), ("main_begin", _vp),
                ("main_end", _vp)]


_optp = ctypes.POINTER(ScanOpts)

_DIAG_ARGS = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
              _vp, _vp, _vp]
_VARLEN_ARGS = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f,
                _vp, _vp, _vp, _vp, _vp]
_MOB_ARGS = [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_WS = [_vp, _szp, _vp]

lib.kdn_diag_scan_fwd.argtypes = _DIAG_ARGS + _WS
lib.kdn_diag_scan_fwd_ex.argtypes = _DIAG_ARGS + [_optp] + _WS
lib.kdn_diag_scan_fwd_noalloc.argtypes = _DIAG_ARGS + [_vp]
lib.kdn_diag_scan_varlen_fwd.argtypes = _VARLEN_ARGS + _WS
lib.kdn_diag_scan_varlen_fwd_ex.argtypes = _VARLEN_ARGS + [_optp] + _WS
lib.kdn_mobius_precision_scan.argtypes = _MOB_ARGS + _WS
lib.kdn_mobius_precision_scan_ex.argtypes = _MOB_ARGS + [_optp] + _WS
lib.kdn_diag_noise_scan_fwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.kdn_diag_scan_bwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                  _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp] + _WS
lib.kdn_diag_scan_bwd_ex.argtypes = lib.kdn_diag_scan_bwd.argtypes[:-3] + [_optp] + _WS
lib.kdn_diag_scan_varlen_bwd.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp,
                                         _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp] + _WS
lib.kdn_decode_step.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                _vp, _f, _vp, _vp, _vp, _vp]
lib.kdn_diag_plan.argtypes = [_i64, _i64, _i64, _i64, _i64, _i32, ctypes.POINTER(_i32),
                              ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i64), _i32]
lib.kdn_diag_varlen_plan.argtypes = [_i64, _i64, _i64, _i64, _i64, _i32, ctypes.POINTER(_i64),
                                     ctypes.POINTER(_i32), ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
for _fn in (lib.kdn_diag_scan_fwd, lib.kdn_diag_scan_fwd_ex, lib.kdn_diag_scan_fwd_noalloc, lib.kdn_diag_scan_varlen_fwd,
            lib.kdn_diag_scan_varlen_fwd_ex, lib.kdn_mobius_precision_scan,
            lib.kdn_mobius_precision_scan_ex, lib.kdn_diag_noise_scan_fwd, lib.kdn_diag_scan_bwd,
            lib.kdn_diag_scan_bwd_ex, lib.kdn_diag_scan_varlen_bwd, lib.kdn_decode_step, lib.kdn_diag_plan,
            lib.kdn_diag_varlen_plan):
    _fn.restype = ctypes.c_int
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


def kdn_diag_plan(B: int, H: int, T: int, d_k: int, d_v: int, segments: int = 0):
    """(chunk, segments, sub-segments, segment token bounds) of a diagonal
    scan of this shape; `segments` as in the scan call (0: automatic)."""
    chunk, segs, subs = _i32(), _i32(), _i32()
    rc = lib.kdn_diag_plan(B, H, T, d_k, d_v, segments, ctypes.byref(chunk), ctypes.byref(segs),
                           ctypes.byref(subs), None, 0)
    if rc != KDN_OK:
        raise KdnError("kdn_diag_plan", rc)
    bounds = (_i64 * (segs.value + 1))()
    rc = lib.kdn_diag_plan(B, H, T, d_k, d_v, segments, None, None, None, bounds, segs.value)
    if rc != KDN_OK:
        raise KdnError("kdn_diag_plan", rc)
    return chunk.value, segs.value, subs.value, list(bounds)


def kdn_diag_varlen_plan(N: int, H: int, total_T: int, d_k: int, d_v: int, segments: int = 0):
    """(seg_tokens, sub-segments, item capacity, composite capacity) of a
    packed batch's forward scan; `segments` 0 (automatic) or 1 (no split)."""
    seg, subs, items, comps = _i64(), _i32(), _i64(), _i64()
    rc = lib.kdn_diag_varlen_plan(N, H, total_T, d_k, d_v, segments, ctypes.byref(seg),
                                  ctypes.byref(subs), ctypes.byref(items), ctypes.byref(comps))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_varlen_plan", rc)
    return seg.value, subs.value, items.value, comps.value


# ---------------------------------------------------------------------------
# torch-tensor front ends (device memory and stream plumbing only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _in_dtypes():
    torch = _torch()
    return (torch.float32, torch.bfloat16, torch.int16, torch.uint16)


def _check(t, name, dtypes, shape=None):
    """Type, dtype, contiguity and shape of one tensor argument (None passes)."""
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_dtype(named):
    ts = [(n, t) for n, t in named if t is not None]
    for n, t in ts[1:]:
        if t.dtype != ts[0][1].dtype:
            raise TypeError(f"{n} has dtype {t.dtype} but {ts[0][0]} has {ts[0][1].dtype}: "
                            "the token inputs must share one dtype")


def _on_gpu(named):
    """Every tensor on the same GPU device; returns it."""
    ts = [(n, t) for n, t in named if t is not None]
    dev = ts[0][1].device
    if dev.type != "cuda":
        raise ValueError(f"{ts[0][0]} is on {dev}: the scans run on the GPU only")
    for n, t in ts:
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, expected {dev}")
    return dev


def _rank(t, name, n):
    if t is None or not hasattr(t, "dim") or t.dim() != n:
        raise ValueError(f"{name} must be a {n}-d tensor")


def _stream(stream):
    """The torch stream to enqueue on: the current one, a torch stream, or a
    raw hipStream_t handle (int) wrapped as an external stream."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _opts(segments, echo, timing=None, stream=None):
    """The options struct of one call.  timing: None or a pair of
    torch.cuda.Event(enable_timing=True) that the library records right before
    and right after the call's main pass (events not yet recorded are recorded
    once on `stream` first, which creates them)."""
    torch = _torch()
    if int(segments) < 0:
        raise ValueError("segments must be >= 0")
    o = ScanOpts()
    o.segments = int(segments)
    if echo is not None:
        _check(echo, "echo", (torch.int64,))
        o.bounds_echo = echo.data_ptr()
        o.echo_capacity = echo.numel()
    if timing is not None:
        ev = tuple(timing)
        if len(ev) != 2 or not all(isinstance(e, torch.cuda.Event) for e in ev):
            raise TypeError("timing must be a pair of torch.cuda.Event")
        for e in ev:
            if not e.cuda_event:
                e.record(stream)
        o.main_begin, o.main_end = ev[0].cuda_event, ev[1].cuda_event
    return o


def _workspace(fn, name, args, device):
    """Query the workspace size and allocate it with torch (on the current
    stream, which the caller has set to the launch stream); returns
    (tensor or None, size)."""
    torch = _torch()
    need = ctypes.c_size_t(0)
    rc = fn(*args(None, ctypes.byref(need)))
    if rc != KDN_OK:
        raise KdnError(name, rc)
    if need.value == 0:
        return None, need
    return torch.empty(need.value, dtype=torch.uint8, device=device), need


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
                      o=None, I_T=None, mu_T=None, want_state=True, segments=0, echo=None,
                      info=None, timing=None, stream=None):
    """Diagonal-precision scan forward on [B,H,T,.] GPU tensors.

    q, k [B,H,T,d_k]; v, beta [B,H,T,d_v]; d [B,H,T] (all float32, or all
    bfloat16 / raw-bf16 int16); A [H] float32; I_prior float; optional I0, mu0
    [B,H,d_k,d_v] float32.  beta None selects Palimpsa-M gating (beta_t = d_t).
    segments: 0 = automatic plan, n = n segments.  echo: optional int64 GPU
    tensor that receives the bounds echo (kdn_scan_opts); info: optional dict
    that receives "echo_words"; timing: optional pair of timing-enabled
    torch.cuda.Event recorded around the main pass.  Returns (o, I_T, mu_T)
    (states None when want_state is False).
    """
    torch = _torch()
    _rank(q, "q", 4)
    _rank(v, "v", 4)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                      ("beta", beta, (B, H, T, dv)), ("d", d, (B, H, T))):
        if t is None and n != "beta":
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)))
    state = (B, H, dk, dv)
    for n, t, shp in (("A", A, (H,)), ("I0", I0, state), ("mu0", mu0, state),
                      ("o", o, (B, H, T, dv)), ("I_T", I_T, state), ("mu_T", mu_T, state)):
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d), ("A", A), ("I0", I0),
                   ("mu0", mu0), ("o", o), ("I_T", I_T), ("mu_T", mu_T), ("echo", echo)))
    s = _stream(stream)
    opts = _opts(segments, echo, timing, s)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
        if want_state:
            I_T = torch.empty(state, dtype=torch.float32, device=dev) if I_T is None else I_T
            mu_T = torch.empty(state, dtype=torch.float32, device=dev) if mu_T is None else mu_T

        def args(ws, nbytes):
            return (B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                    _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(o), _ptr(I_T), _ptr(mu_T),
                    ctypes.byref(opts), ws, nbytes, s.cuda_stream)

        ws, need = _workspace(lib.kdn_diag_scan_fwd_ex, "kdn_diag_scan_fwd", args, dev)
        rc = lib.kdn_diag_scan_fwd_ex(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_fwd", rc)
    if info is not None:
        info["echo_words"] = opts.echo_words
    return o, I_T, mu_T


def kdn_diag_scan_fwd_noalloc(q, k, v, beta, d, A, I_prior, I0=None, mu0=None,
                              o=None, I_T=None, mu_T=None, want_state=True, stream=None):
    """kdn_diag_scan_fwd through the no-allocation entry point: the library
    uses its fixed per-GPU scratch instead of a workspace.  Arguments and
    results as for kdn_diag_scan_fwd.  Pass o (and I_T, mu_T, or
    want_state=False) to keep the call itself free of allocations."""
    torch = _torch()
    _rank(q, "q", 4)
    _rank(v, "v", 4)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                      ("beta", beta, (B, H, T, dv)), ("d", d, (B, H, T))):
        if t is None and n != "beta":
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)))
    state = (B, H, dk, dv)
    for n, t, shp in (("A", A, (H,)), ("I0", I0, state), ("mu0", mu0, state),
                      ("o", o, (B, H, T, dv)), ("I_T", I_T, state), ("mu_T", mu_T, state)):
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d), ("A", A), ("I0", I0),
                   ("mu0", mu0), ("o", o), ("I_T", I_T), ("mu_T", mu_T)))
    s = _stream(stream)
    with torch.cuda.device(dev), torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
        if want_state:
            I_T = torch.empty(state, dtype=torch.float32, device=dev) if I_T is None else I_T
            mu_T = torch.empty(state, dtype=torch.float32, device=dev) if mu_T is None else mu_T
        rc = lib.kdn_diag_scan_fwd_noalloc(B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(beta), _ptr(d), _ptr(A), float(I_prior), _ptr(I0),
                                           _ptr(mu0), _ptr(o), _ptr(I_T), _ptr(mu_T), s.cuda_stream)
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_fwd_noalloc", rc)
    return o, I_T, mu_T


def kdn_diag_scan_varlen_fwd(q, k, v, beta, d, A, I_prior, cu_seqlens, I0=None, mu0=None,
                             want_state=True, segments=0, echo=None, info=None, timing=None,
                             stream=None):
    """Diagonal scan over a packed variable-length batch.

    q, k [H,total_T,d_k]; v, beta [H,total_T,d_v]; d [H,total_T] (float32 or
    bf16; beta None = Palimpsa-M gating); cu_seqlens int64 [N+1] on the device;
    I0, mu0 [N,H,d_k,d_v] float32 or None.  segments: 0 splits sequences
    longer than their fair share (kdn_diag_varlen_plan), 1 never splits.
    Returns (o [H,total_T,d_v], I_T, mu_T [N,H,d_k,d_v]).
    """
    torch = _torch()
    _rank(q, "q", 3)
    _rank(v, "v", 3)
    H, T, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (H, T, dk)), ("k", k, (H, T, dk)), ("v", v, (H, T, dv)),
                      ("beta", beta, (H, T, dv)), ("d", d, (H, T))):
        if t is None and n != "beta":
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)))
    _rank(cu_seqlens, "cu_seqlens", 1)
    _check(cu_seqlens, "cu_seqlens", (torch.int64,))
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    state = (N, H, dk, dv)
    for n, t, shp in (("A", A, (H,)), ("I0", I0, state), ("mu0", mu0, state)):
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d), ("A", A),
                   ("cu_seqlens", cu_seqlens), ("I0", I0), ("mu0", mu0), ("echo", echo)))
    s = _stream(stream)
    opts = _opts(segments, echo, timing, s)
    with torch.cuda.stream(s):
        o = torch.empty((H, T, dv), dtype=torch.float32, device=dev)
        I_T = mu_T = None
        if want_state:
            I_T = torch.empty(state, dtype=torch.float32, device=dev)
            mu_T = torch.empty(state, dtype=torch.float32, device=dev)

        def args(ws, nbytes):
            return (N, H, T, dk, dv, _in_dtype(q), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                    _ptr(beta), _ptr(d), _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(o),
                    _ptr(I_T), _ptr(mu_T), ctypes.byref(opts), ws, nbytes, s.cuda_stream)

        ws, need = _workspace(lib.kdn_diag_scan_varlen_fwd_ex, "kdn_diag_scan_varlen_fwd", args, dev)
        rc = lib.kdn_diag_scan_varlen_fwd_ex(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_varlen_fwd", rc)
    if info is not None:
        info["echo_words"] = opts.echo_words
    return o, I_T, mu_T


def kdn_diag_noise_scan_fwd(q, k, v, beta, a, p, lambda0=None, mu0=None, want_state=True,
                            stream=None):
    """Diagonal KDN with process noise on [B,H,T,.] GPU tensors.

    q, k [B,H,T,d_k]; v, beta [B,H,T,d_v] (float32 or bf16); a, p [B,H,T]
    float32; optional lambda0, mu0 [B,H,d_k,d_v] float32.  Returns
    (o, lambda_T, mu_T) (states None when want_state is False).
    """
    torch = _torch()
    _rank(q, "q", 4)
    _rank(v, "v", 4)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                      ("beta", beta, (B, H, T, dv))):
        if t is None:
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta)))
    state = (B, H, dk, dv)
    for n, t, shp in (("a", a, (B, H, T)), ("p", p, (B, H, T)), ("lambda0", lambda0, state),
                      ("mu0", mu0, state)):
        if t is None and n in ("a", "p"):
            raise ValueError(f"{n} is required")
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("a", a), ("p", p),
                   ("lambda0", lambda0), ("mu0", mu0)))
    s = _stream(stream)
    with torch.cuda.stream(s):
        o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
        lam_T = mu_T = None
        if want_state:
            lam_T = torch.empty(state, dtype=torch.float32, device=dev)
            mu_T = torch.empty(state, dtype=torch.float32, device=dev)
        rc = lib.kdn_diag_noise_scan_fwd(B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(beta), _ptr(a), _ptr(p), _ptr(lambda0), _ptr(mu0),
                                         _ptr(o), _ptr(lam_T), _ptr(mu_T), s.cuda_stream)
    if rc != KDN_OK:
        raise KdnError("kdn_diag_noise_scan_fwd", rc)
    return o, lam_T, mu_T


def kdn_diag_scan_bwd(q, k, v, beta, d, A, I_prior, d_o, I0=None, mu0=None, d_I_T=None,
                      d_mu_T=None, want_prior=True, segments=0, stream=None):
    """Gradient of kdn_diag_scan_fwd for L = sum(d_o o) + sum(d_I_T I_T) + sum(d_mu_T mu_T).

    Inputs as for the forward call plus d_o [B,H,T,d_v] and optional d_I_T,
    d_mu_T [B,H,d_k,d_v] (all float32).  segments: 0 = automatic plan, n =
    n segments per row.  Returns a dict of float32 tensors: dq, dk
    [B,H,T,d_k]; dv, dbeta [B,H,T,d_v]; dd [B,H,T]; dA [H]; dI_prior [1]
    (when want_prior); dI0 / dmu0 [B,H,d_k,d_v] when I0 / mu0 are given.
    """
    torch = _torch()
    _rank(q, "q", 4)
    _rank(v, "v", 4)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                      ("beta", beta, (B, H, T, dv)), ("d", d, (B, H, T))):
        if t is None and n != "beta":
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)))
    state = (B, H, dk, dv)
    for n, t, shp in (("A", A, (H,)), ("d_o", d_o, (B, H, T, dv)), ("I0", I0, state),
                      ("mu0", mu0, state), ("d_I_T", d_I_T, state), ("d_mu_T", d_mu_T, state)):
        if t is None and n == "d_o":
            raise ValueError("d_o is required")
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d), ("A", A), ("d_o", d_o),
                   ("I0", I0), ("mu0", mu0), ("d_I_T", d_I_T), ("d_mu_T", d_mu_T)))
    s = _stream(stream)
    with torch.cuda.stream(s):
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
        o = lambda n: _ptr(g.get(n))

        opts = ScanOpts()
        opts.segments = segments

        def args(ws, nbytes):
            return (B, H, T, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                    _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(d_o), _ptr(d_I_T),
                    _ptr(d_mu_T), o("dq"), o("dk"), o("dv"), o("dbeta"), o("dd"), o("dA"),
                    o("dI_prior"), o("dI0"), o("dmu0"), ctypes.byref(opts), ws, nbytes,
                    s.cuda_stream)

        ws, need = _workspace(lib.kdn_diag_scan_bwd_ex, "kdn_diag_scan_bwd", args, dev)
        rc = lib.kdn_diag_scan_bwd_ex(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_bwd", rc)
    return g


def kdn_diag_scan_varlen_bwd(q, k, v, beta, d, A, I_prior, cu_seqlens, d_o, I0=None, mu0=None,
                             d_I_T=None, d_mu_T=None, want_prior=True, stream=None):
    """Gradient of kdn_diag_scan_varlen_fwd over a packed batch.

    q, k [H,total_T,d_k]; v, beta [H,total_T,d_v]; d [H,total_T] (float32 or
    bf16; beta None = Palimpsa-M gating); cu_seqlens int64 [N+1] on the device;
    d_o [H,total_T,d_v]; I0, mu0, d_I_T, d_mu_T [N,H,d_k,d_v] float32 or None.
    Returns a dict: dq, dk [H,total_T,d_k]; dv, dbeta [H,total_T,d_v];
    dd [H,total_T]; dA [H]; dI_prior [1] (when want_prior); dI0 / dmu0
    [N,H,d_k,d_v] when I0 / mu0 are given.
    """
    torch = _torch()
    _rank(q, "q", 3)
    _rank(v, "v", 3)
    H, T, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (H, T, dk)), ("k", k, (H, T, dk)), ("v", v, (H, T, dv)),
                      ("beta", beta, (H, T, dv)), ("d", d, (H, T))):
        if t is None and n != "beta":
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)))
    _rank(cu_seqlens, "cu_seqlens", 1)
    _check(cu_seqlens, "cu_seqlens", (torch.int64,))
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    state = (N, H, dk, dv)
    for n, t, shp in (("A", A, (H,)), ("d_o", d_o, (H, T, dv)), ("I0", I0, state),
                      ("mu0", mu0, state), ("d_I_T", d_I_T, state), ("d_mu_T", d_mu_T, state)):
        if t is None and n == "d_o":
            raise ValueError("d_o is required")
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d), ("A", A),
                   ("cu_seqlens", cu_seqlens), ("d_o", d_o), ("I0", I0), ("mu0", mu0),
                   ("d_I_T", d_I_T), ("d_mu_T", d_mu_T)))
    s = _stream(stream)
    with torch.cuda.stream(s):
        new = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
        g = {"dq": new(H, T, dk), "dk": new(H, T, dk), "dv": new(H, T, dv), "dd": new(H, T),
             "dA": new(H)}
        if beta is not None:
            g["dbeta"] = new(H, T, dv)
        if want_prior:
            g["dI_prior"] = new(1)
        if I0 is not None:
            g["dI0"] = new(*state)
        if mu0 is not None:
            g["dmu0"] = new(*state)
        o = lambda n: _ptr(g.get(n))

        def args(ws, nbytes):
            return (N, H, T, dk, dv, _in_dtype(q), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                    _ptr(beta), _ptr(d), _ptr(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(d_o),
                    _ptr(d_I_T), _ptr(d_mu_T), o("dq"), o("dk"), o("dv"), o("dbeta"), o("dd"),
                    o("dA"), o("dI_prior"), o("dI0"), o("dmu0"), ws, nbytes, s.cuda_stream)

        ws, need = _workspace(lib.kdn_diag_scan_varlen_bwd, "kdn_diag_scan_varlen_bwd", args, dev)
        rc = lib.kdn_diag_scan_varlen_bwd(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_diag_scan_varlen_bwd", rc)
    return g


def kdn_mobius_precision_scan(a, p, Lam, lambda0=None, q=None, k=None, v=None, mu0=None,
                              want_lambda=True, want_state=True, segments=0, echo=None,
                              info=None, timing=None, stream=None):
    """Isotropic filter: Mobius precision scan, then (if q, k, v given) the gated mean scan.

    a, p, Lam [B,H,T] float32; lambda0 [B,H] or None (-> 1); q, k [B,H,T,d_k],
    v [B,H,T,d_v], mu0 [B,H,d_k,d_v] float32.  segments: 0 = automatic plan
    of the mean scan, n = n segments; echo / info as for kdn_diag_scan_fwd.
    Returns (lambda, o, mu_T).
    """
    torch = _torch()
    _rank(a, "a", 3)
    B, H, T = a.shape
    f32 = (torch.float32,)
    for n, t, shp in (("a", a, (B, H, T)), ("p", p, (B, H, T)), ("Lambda", Lam, (B, H, T)),
                      ("lambda0", lambda0, (B, H))):
        if t is None and n != "lambda0":
            raise ValueError(f"{n} is required")
        _check(t, n, f32, shp)
    dk = dv = 0
    if q is not None or k is not None or v is not None:
        if q is None or k is None or v is None:
            raise ValueError("the mean scan needs q, k and v")
        _rank(q, "q", 4)
        _rank(v, "v", 4)
        dk, dv = q.shape[-1], v.shape[-1]
        for n, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                          ("mu0", mu0, (B, H, dk, dv))):
            _check(t, n, f32, shp)
    elif mu0 is not None:
        raise ValueError("mu0 without q, k, v")
    dev = _on_gpu((("a", a), ("p", p), ("Lambda", Lam), ("lambda0", lambda0), ("q", q), ("k", k),
                   ("v", v), ("mu0", mu0), ("echo", echo)))
    s = _stream(stream)
    opts = _opts(segments, echo, timing, s)
    with torch.cuda.stream(s):
        lam = torch.empty((B, H, T), dtype=torch.float32, device=dev) if want_lambda else None
        o = mu_T = None
        if q is not None:
            o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
            if want_state:
                mu_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)

        def args(ws, nbytes):
            return (B, H, T, _ptr(a), _ptr(p), _ptr(Lam), _ptr(lambda0), _ptr(lam), dk, dv,
                    _ptr(q), _ptr(k), _ptr(v), _ptr(mu0), _ptr(o), _ptr(mu_T), ctypes.byref(opts),
                    ws, nbytes, s.cuda_stream)

        ws, need = _workspace(lib.kdn_mobius_precision_scan_ex, "kdn_mobius_precision_scan", args, dev)
        rc = lib.kdn_mobius_precision_scan_ex(*args(_ptr(ws), _nbytes(ws, need)))
    if rc != KDN_OK:
        raise KdnError("kdn_mobius_precision_scan", rc)
    if info is not None:
        info["echo_words"] = opts.echo_words
    return lam, o, mu_T


def kdn_decode_step(q, k, v, beta, d, A, I_prior, I, mu, o=None, stream=None):
    """One decode token: q, k [B,H,d_k]; v, beta [B,H,d_v]; d [B,H] (one
    dtype: float32 or bf16; beta None = Palimpsa-M gating); A [H]; I, mu
    [B,H,d_k,d_v] float32 updated in place.  Returns o [B,H,d_v]."""
    torch = _torch()
    _rank(q, "q", 3)
    _rank(v, "v", 3)
    B, H, dk = q.shape
    dv = v.shape[-1]
    dts, f32 = _in_dtypes(), (torch.float32,)
    for n, t, shp in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("v", v, (B, H, dv)),
                      ("beta", beta, (B, H, dv)), ("d", d, (B, H))):
        if t is None and n != "beta":
            raise ValueError(f"{n} is required")
        _check(t, n, dts, shp)
    _same_dtype((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d)))
    state = (B, H, dk, dv)
    for n, t, shp in (("A", A, (H,)), ("I", I, state), ("mu", mu, state), ("o", o, (B, H, dv))):
        if t is None and n != "o":
            raise ValueError(f"{n} is required")
        _check(t, n, f32, shp)
    dev = _on_gpu((("q", q), ("k", k), ("v", v), ("beta", beta), ("d", d), ("A", A), ("I", I),
                   ("mu", mu), ("o", o)))
    s = _stream(stream)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
        rc = lib.kdn_decode_step(B, H, dk, dv, _in_dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                 _ptr(d), _ptr(A), float(I_prior), _ptr(I), _ptr(mu), _ptr(o),
                                 s.cuda_stream)
    if rc != KDN_OK:
        raise KdnError("kdn_decode_step", rc)
    return o

"""CPU oracle for the precision-tracking memory scans -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It is independent of the HIP library: it shares no code
with it and never reads anything the library produced.

The arithmetic lives in ``kdn_oracle.c`` (plain sequential fp64, one head per
call).  This module only loads it, decodes stored inputs to float64, and runs
independent heads on a thread pool (heads never interact, so this changes no
arithmetic).  It also enumerates the chunk/segment plan of the diagonal scan
from its definition, for the bit-exact bookkeeping checks.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, special cases, brute force); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c99", "-fno-fast-math", "-ffp-contract=off"]

_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *_CFLAGS, *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB):
    """Load (building first if absent) a compiled oracle library."""
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    D = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.oracle_diag_head.argtypes = [L, L, L, D, D, D, D, D, ctypes.c_double, ctypes.c_double,
                                     D, D, D, D, D, D]
    lib.oracle_diag_head.restype = ctypes.c_int
    lib.oracle_iso_head.argtypes = [L, D, D, D, ctypes.c_double, L, L, D, D, D, D, D, D, D, D]
    lib.oracle_iso_head.restype = ctypes.c_int
    lib.oracle_diag_noise_head.argtypes = [L, L, L, D, D, D, D, D, D, D, D, D, D, D, D]
    lib.oracle_diag_noise_head.restype = ctypes.c_int
    lib.oracle_kdn_exact_head.argtypes = [L, L, L, D, D, D, D, D, D, D, D, D, D, D]
    lib.oracle_kdn_exact_head.restype = ctypes.c_int
    PP = ctypes.POINTER(D)
    lib.oracle_diag_head_bwd.argtypes = [L, L, L, D, D, D, D, D, ctypes.c_double, ctypes.c_double,
                                         D, D, D, D, D, PP, PP]
    lib.oracle_diag_head_bwd.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input -> float64.  bf16 is raw uint16 bits: the top half of a float32."""
    if dtype == "bf16":
        b = np.asarray(x)
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x).astype(np.float64)   # float32 storage widens exactly


def _threads(threads):
    if threads:
        return threads
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def diag_head(q, k, v, beta, d, A, I_prior, I0=None, mu0=None, lib=None):
    """One head of the diagonal-precision recurrence; float64 arrays in, dict out."""
    lib = lib or load()
    q, k, v, beta, d = (np.ascontiguousarray(x, np.float64) for x in (q, k, v, beta, d))
    T, dk = q.shape
    dv = v.shape[1]
    o = np.empty((T, dv))
    s = np.empty((T, dv))
    I_T = np.empty((dk, dv))
    mu_T = np.empty((dk, dv))
    I0 = None if I0 is None else np.ascontiguousarray(I0, np.float64)
    mu0 = None if mu0 is None else np.ascontiguousarray(mu0, np.float64)
    rc = lib.oracle_diag_head(T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                              float(A), float(I_prior), _ptr(I0), _ptr(mu0),
                              _ptr(o), _ptr(s), _ptr(I_T), _ptr(mu_T))
    if rc != 0:
        raise MemoryError("oracle_diag_head failed")
    return {"o": o, "s": s, "I_T": I_T, "mu_T": mu_T}


def gate_beta(inp: dict, b: int, h: int, t0=0, t1=None) -> np.ndarray:
    """beta_t[i] of head (b, h) as float64 [T, dv].  A workload without beta
    uses Palimpsa-M gating ("Learning to Remember, Learn, and Forget in
    Attention-Based Models", Metodologia 3): the step gate d_t is also the
    input gate, beta_t[i] = d_t for every value channel i."""
    spec = inp["spec"]
    t1 = inp["q"].shape[2] if t1 is None else t1
    if inp["beta"] is not None:
        return decode(inp["beta"][b, h, t0:t1], spec.dtype)
    d = decode(inp["d"][b, h, t0:t1], spec.dtype)
    return np.repeat(d[:, None], inp["v"].shape[-1], axis=1)


GRAD_NAMES = ("dq", "dk", "dv", "dbeta", "dd", "dA", "dI_prior", "dI0", "dmu0")


def diag_head_bwd(q, k, v, beta, d, A, I_prior, dout, I0=None, mu0=None, dI_T=None,
                  dmu_T=None, lib=None):
    """Gradient of one head of the diagonal recurrence (float64 in).

    Returns {name: array} for GRAD_NAMES (dI0 / dmu0 only when I0 / mu0 are
    given) and {"scale_" + name: array}, the same sums taken over absolute
    values of their terms.
    """
    lib = lib or load()
    q, k, v, beta, d, dout = (np.ascontiguousarray(x, np.float64) for x in (q, k, v, beta, d, dout))
    T, dk = q.shape
    dv = v.shape[1]
    shapes = {"dq": (T, dk), "dk": (T, dk), "dv": (T, dv), "dbeta": (T, dv), "dd": (T,),
              "dA": (1,), "dI_prior": (1,), "dI0": (dk, dv), "dmu0": (dk, dv)}
    out = {n: np.zeros(shapes[n]) for n in GRAD_NAMES}
    sc = {n: np.zeros(shapes[n]) for n in GRAD_NAMES}
    opt = lambda x: None if x is None else np.ascontiguousarray(x, np.float64)
    I0, mu0, dI_T, dmu_T = opt(I0), opt(mu0), opt(dI_T), opt(dmu_T)
    D = ctypes.POINTER(ctypes.c_double)
    gp = (D * 9)(*[_ptr(out[n]) for n in GRAD_NAMES])
    sp = (D * 9)(*[_ptr(sc[n]) for n in GRAD_NAMES])
    rc = lib.oracle_diag_head_bwd(T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                                  float(A), float(I_prior), _ptr(I0), _ptr(mu0), _ptr(dout),
                                  _ptr(dI_T), _ptr(dmu_T), gp, sp)
    if rc != 0:
        raise MemoryError("oracle_diag_head_bwd failed")
    res = {n: out[n] for n in GRAD_NAMES if not (n == "dI0" and I0 is None)
           and not (n == "dmu0" and mu0 is None)}
    res.update({"scale_" + n: sc[n] for n in res})
    res["dA"], res["dI_prior"] = float(res["dA"][0]), float(res["dI_prior"][0])
    res["scale_dA"], res["scale_dI_prior"] = float(res["scale_dA"][0]), float(res["scale_dI_prior"][0])
    return res


def diag_scan_bwd(inp: dict, dout: np.ndarray, heads=None, threads=None, I0=None, mu0=None,
                  dI_T=None, dmu_T=None, lib=None):
    """Gradients over heads of a synthetic-input dict; dout [B,H,T,dv] float.

    Returns {(b,h): diag_head_bwd(...) result}.
    """
    spec = inp["spec"]
    B, H = inp["q"].shape[:2]
    heads = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    lib = lib or load()
    pick = lambda x, b, h: None if x is None else np.asarray(x[b, h], np.float64)

    def one(bh):
        b, h = bh
        args = [decode(inp[n][b, h], spec.dtype) for n in ("q", "k", "v", "d")]
        args.insert(3, gate_beta(inp, b, h))
        g = diag_head_bwd(*args, A=float(inp["A"][h]), I_prior=inp["I_prior"],
                          dout=np.asarray(dout[b, h], np.float64),
                          I0=pick(I0, b, h), mu0=pick(mu0, b, h),
                          dI_T=pick(dI_T, b, h), dmu_T=pick(dmu_T, b, h), lib=lib)
        if inp["beta"] is None:
            # Palimpsa-M gating: beta_t[i] = d_t, so d_t also collects every dbeta_t[i]
            g["dd"] = g["dd"] + g["dbeta"].sum(axis=1)
            g["scale_dd"] = g["scale_dd"] + g["scale_dbeta"].sum(axis=1)
            del g["dbeta"], g["scale_dbeta"]
        return bh, g

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, heads))


def diag_noise_head(q, k, v, beta, a, p, lam0=None, mu0=None, lib=None):
    """One head of the diagonal KDN with process noise (float64 in)."""
    lib = lib or load()
    q, k, v, beta, a, p = (np.ascontiguousarray(x, np.float64) for x in (q, k, v, beta, a, p))
    T, dk = q.shape
    dv = v.shape[1]
    o = np.empty((T, dv))
    s = np.empty((T, dv))
    lam_T = np.empty((dk, dv))
    mu_T = np.empty((dk, dv))
    opt = lambda x: None if x is None else np.ascontiguousarray(x, np.float64)
    lam0, mu0 = opt(lam0), opt(mu0)
    rc = lib.oracle_diag_noise_head(T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(a),
                                    _ptr(p), _ptr(lam0), _ptr(mu0), _ptr(o), _ptr(s),
                                    _ptr(lam_T), _ptr(mu_T))
    if rc != 0:
        raise MemoryError("oracle_diag_noise_head failed")
    return {"o": o, "s": s, "I_T": lam_T, "mu_T": mu_T}


def kdn_exact_head(q, k, v, beta, a, p, P0=None, mu0=None, lib=None):
    """Exact (dense-covariance) Kalman filter of one head: float64 in, dict
    out with o [T,dv], P_T [dv,dk,dk] (one covariance per value column) and
    mu_T [dk,dv]."""
    lib = lib or load()
    q, k, v, beta, a, p = (np.ascontiguousarray(x, np.float64) for x in (q, k, v, beta, a, p))
    T, dk = q.shape
    dv = v.shape[1]
    o = np.empty((T, dv))
    P_T = np.empty((dv, dk, dk))
    mu_T = np.empty((dk, dv))
    opt = lambda x: None if x is None else np.ascontiguousarray(x, np.float64)
    P0, mu0 = opt(P0), opt(mu0)
    rc = lib.oracle_kdn_exact_head(T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(a),
                                   _ptr(p), _ptr(P0), _ptr(mu0), _ptr(o), _ptr(P_T), _ptr(mu_T))
    if rc != 0:
        raise MemoryError("oracle_kdn_exact_head failed")
    return {"o": o, "P_T": P_T, "mu_T": mu_T}


def diag_noise_scan(inp: dict, heads=None, threads=None, lam0=None, mu0=None, lib=None):
    """The process-noise diagonal filter over heads of a synthetic-input dict
    (q, k, v, beta in storage dtype, a, p float32 [B,H,T])."""
    spec = inp["spec"]
    B, H = inp["q"].shape[:2]
    heads = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    lib = lib or load()
    pick = lambda x, b, h: None if x is None else np.asarray(x[b, h], np.float64)

    def one(bh):
        b, h = bh
        args = [decode(inp[n][b, h], spec.dtype) for n in ("q", "k", "v", "beta")]
        ap = [np.asarray(inp[n][b, h], np.float64) for n in ("a", "p")]
        return bh, diag_noise_head(*args, *ap, lam0=pick(lam0, b, h), mu0=pick(mu0, b, h), lib=lib)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, heads))


def diag_scan(inp: dict, heads=None, threads=None, t_range=None, I0=None, mu0=None, lib=None):
    """Run the diagonal recurrence over heads of a synthetic-input dict.

    inp: q, k, v, beta, d [B,H,T,.] in storage dtype (spec.dtype), A [H], I_prior.
    heads: iterable of (b, h); default all.  t_range: (t0, t1) slice of tokens.
    I0, mu0: optional [B,H,dk,dv] starting state.
    Returns {(b,h): {"o","s","I_T","mu_T"}} in float64.
    """
    spec = inp["spec"]
    B, H = inp["q"].shape[:2]
    heads = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    t0, t1 = t_range if t_range is not None else (0, inp["q"].shape[2])
    lib = lib or load()

    def one(bh):
        b, h = bh
        args = [decode(inp[n][b, h, t0:t1], spec.dtype) for n in ("q", "k", "v", "d")]
        args.insert(3, gate_beta(inp, b, h, t0, t1))
        return bh, diag_head(*args, A=float(inp["A"][h]), I_prior=inp["I_prior"],
                             I0=None if I0 is None else I0[b, h],
                             mu0=None if mu0 is None else mu0[b, h], lib=lib)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, heads))


def diag_scan_varlen(inp: dict, cu_seqlens, I0=None, mu0=None, threads=None, lib=None):
    """Packed variable-length batch: inputs [1,H,total_T,.]; sequence s owns
    packed tokens [cu[s], cu[s+1]) and starts from its own state (I0, mu0
    [N,H,dk,dv] or the prior).  Each (sequence, head) is an independent run
    of the diagonal recurrence.  Returns {(s, h): diag_head result}."""
    spec = inp["spec"]
    H = inp["q"].shape[1]
    cu = [int(x) for x in cu_seqlens]
    runs = [(s, h) for s in range(len(cu) - 1) for h in range(H)]
    lib = lib or load()
    pick = lambda x, s, h: None if x is None else np.asarray(x[s, h], np.float64)

    def one(sh):
        s, h = sh
        t0, t1 = cu[s], cu[s + 1]
        args = [decode(inp[n][0, h, t0:t1], spec.dtype) for n in ("q", "k", "v", "d")]
        args.insert(3, gate_beta(inp, 0, h, t0, t1))
        return sh, diag_head(*args, A=float(inp["A"][h]), I_prior=inp["I_prior"],
                             I0=pick(I0, s, h), mu0=pick(mu0, s, h), lib=lib)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, runs))


def iso_head(a, p, Lam, lambda0, q=None, k=None, v=None, mu0=None, lib=None):
    """One head of the isotropic (scalar precision) filter; float64 in, dict out."""
    lib = lib or load()
    a, p, Lam = (np.ascontiguousarray(x, np.float64) for x in (a, p, Lam))
    T = a.shape[0]
    lam = np.empty(T)
    if q is None:
        rc = lib.oracle_iso_head(T, _ptr(a), _ptr(p), _ptr(Lam), float(lambda0), 0, 0,
                                 None, None, None, None, _ptr(lam), None, None, None)
        if rc != 0:
            raise MemoryError("oracle_iso_head failed")
        return {"lambda": lam}
    q, k, v = (np.ascontiguousarray(x, np.float64) for x in (q, k, v))
    dk, dv = q.shape[1], v.shape[1]
    o = np.empty((T, dv))
    s = np.empty((T, dv))
    mu_T = np.empty((dk, dv))
    mu0 = None if mu0 is None else np.ascontiguousarray(mu0, np.float64)
    rc = lib.oracle_iso_head(T, _ptr(a), _ptr(p), _ptr(Lam), float(lambda0), dk, dv,
                             _ptr(q), _ptr(k), _ptr(v), _ptr(mu0), _ptr(lam),
                             _ptr(o), _ptr(s), _ptr(mu_T))
    if rc != 0:
        raise MemoryError("oracle_iso_head failed")
    return {"lambda": lam, "o": o, "s": s, "mu_T": mu_T}


def iso_scan(inp: dict, heads=None, threads=None, with_mean=True, mu0=None, lib=None):
    """Run the isotropic filter over heads of a synthetic-input dict (float32
    arrays); mu0 [B,H,d_k,d_v] is an optional starting mean (default 0)."""
    B, H = inp["a"].shape[:2]
    heads = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    lib = lib or load()

    def one(bh):
        b, h = bh
        f = lambda n: np.asarray(inp[n][b, h], np.float32).astype(np.float64)
        mean = (f("q"), f("k"), f("v")) if with_mean else (None, None, None)
        m0 = None if mu0 is None else np.asarray(mu0[b, h], np.float64)
        return bh, iso_head(f("a"), f("p"), f("Lambda"), float(inp["lambda0"][b, h]),
                            *mean, mu0=m0, lib=lib)

    with ThreadPoolExecutor(_threads(threads)) as ex:
        return dict(ex.map(one, heads))


def plan(T: int, chunk: int, segments: int):
    """Chunk and segment bounds of a T-token scan, enumerated from the definition.

    Tokens are cut into n_chunks = ceil(T / chunk) chunks, the last one ragged.
    Segment s owns chunks [floor(s*n/S), floor((s+1)*n/S)), i.e. tokens from
    chunk*that up to min(chunk*next, T).  Returns (chunk_starts, chunk_lens,
    segment_token_bounds) as Python int lists.
    """
    n = -(-T // chunk)
    starts = [c * chunk for c in range(n)]
    lens = [min(chunk, T - c * chunk) for c in range(n)]
    bounds = [min((s * n // segments) * chunk, T) for s in range(segments + 1)]
    return starts, lens, bounds


def plan_sub(T: int, chunk: int, segments: int, subsegments: int):
    """Token bounds of every sub-segment of the composite segments 0..S-2:
    sub-segment r of segment s owns the segment's chunks
    [c0 + floor(r m / R), c0 + floor((r+1) m / R)), with [c0, c1) the
    segment's chunks (as in plan) and m = c1 - c0.  Returns
    {(s, r): (t_begin, t_end)} as Python ints."""
    n = -(-T // chunk)
    out = {}
    for s in range(segments - 1):
        c0, c1 = s * n // segments, (s + 1) * n // segments
        m = c1 - c0
        for r in range(subsegments):
            a = c0 + r * m // subsegments
            b = c0 + (r + 1) * m // subsegments
            out[(s, r)] = (min(a * chunk, T), min(b * chunk, T))
    return out


def varlen_plan(cu_seqlens, seg_tokens: int, subsegments: int, chunk: int = 16):
    """Plan of a packed batch's forward scan, enumerated from its definition.

    Sequences are ranked longest first, ties by index.  A sequence of len >
    seg_tokens tokens (seg_tokens > 0) runs as ceil(len / seg_tokens)
    segments, segment g owning its tokens [g*seg, min((g+1)*seg, len)); any
    other sequence is one segment.  The main-pass items are the sequences'
    segments in rank order, each sequence's in token order.  The composite
    segments are the split sequences' segments but their last, in the same
    order; sub-segment r of one owns the segment's chunks
    [floor(r m / R), floor((r+1) m / R)), m = seg_tokens / chunk.
    Returns (items, composites) with packed token offsets: items
    [(s, g, t_begin, t_end)], composites [(s, g, [(t_begin, t_end) per r])].
    """
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    lens = [cu[s + 1] - cu[s] for s in range(N)]
    order = sorted(range(N), key=lambda s: (-lens[s], s))
    items, comps = [], []
    for s in order:
        L = lens[s]
        nseg = -(-L // seg_tokens) if seg_tokens > 0 and L > seg_tokens else 1
        for g in range(nseg):
            if nseg == 1:
                items.append((s, 0, cu[s], cu[s + 1]))
            else:
                items.append((s, g, cu[s] + g * seg_tokens, cu[s] + min((g + 1) * seg_tokens, L)))
        m = seg_tokens // chunk if seg_tokens > 0 else 0
        for g in range(nseg - 1):
            base = cu[s] + g * seg_tokens
            subs = [(base + (r * m // subsegments) * chunk, base + ((r + 1) * m // subsegments) * chunk)
                    for r in range(subsegments)]
            comps.append((s, g, subs))
    return items, comps


def element_offset(b: int, h: int, t: int, x: int, H: int, T: int, D: int) -> int:
    """Element index of [b, h, t, x] in a contiguous [B, H, T, D] tensor (Python int)."""
    return ((b * H + h) * T + t) * D + x


class Timer:
    """Steady-clock wall time of a block (used by the CPU-baseline leg)."""

    def __enter__(self):
        self.t0 = time.perf_counter()
        return self

    def __exit__(self, *exc):
        self.seconds = time.perf_counter() - self.t0

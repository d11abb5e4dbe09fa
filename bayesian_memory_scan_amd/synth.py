"""Seeded synthetic inputs for the precision-tracking memory scans.

This module only draws random inputs with the shapes and distributions of the
workloads; it holds none of the recurrences' arithmetic.  Both the HIP path and
the CPU oracle read what it produces, so it imports neither of them.

Recipe (every workload):

* one PCG64 stream per (seed, b, h) head, so that any head can be regenerated
  alone; the per-head draw order is fixed (listed per workload below);
* draws are float32 standard normals, the activation is applied in float32,
  and values that the workload stores in bf16 are then rounded from float32 to
  bf16 with round-to-nearest-even;
* A (forget rate per head) comes from its own stream keyed (seed, 0xA).

Diagonal-precision workloads, per head, in this order:
  q ~ N(0,1) [T,d_k]; k ~ N(0,1) [T,d_k] then L2-normalised per token;
  v ~ N(0,1) [T,d_v]; beta = sigmoid(N(0,1)) [T,d_v]; d = softplus(N(0,1)) [T].
Gradient workloads reuse a diagonal workload's inputs and add, from a stream
keyed (seed, 0xD0): d_o ~ N(0,1) [B,H,T,d_v], then d_I_T, d_mu_T ~ N(0,1)
[B,H,d_k,d_v] (loss weights); a starting state comes from (seed, 0x50):
I0 ~ U(0.2, 3.2), mu0 ~ N(0,1).
Process-noise diagonal workloads take a diagonal workload's q, k, v, beta and
add, from a stream keyed (seed, 0xAB): a = exp(-softplus(N(0,1))) [B,H,T]
(decay in (0,1)), then p = softplus(N(0,1)) [B,H,T] (process-noise variance).
Palimpsa-M workloads are diagonal workloads with beta removed (the step gate
d_t doubles as the input gate).  Packed variable-length workloads draw one
[1,H,total_T,.] diagonal workload and cut it into N sequences at N-1 distinct
cut points drawn uniformly from [1, total_T) with a stream keyed (seed, 0x1E)
(so lengths follow the spacing of uniform points: many short, a few long).
Isotropic workload, per head, in this order:
  a = exp(-softplus(N(0,1))) [T]; p = softplus(N(0,1)) [T];
  Lambda = softplus(N(0,1)) [T]; then q, k (normalised), v as above.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

__all__ = [
    "DiagSpec", "IsoSpec", "WORKLOADS", "workload",
    "diag_head", "diag_inputs", "iso_head", "iso_inputs", "grad_inputs", "state_inputs",
    "noise_inputs", "VarlenSpec", "varlen_inputs", "varlen_grad_inputs",
    "f32_to_bf16_bits",
]


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


@dataclass(frozen=True)
class DiagSpec:
    """A diagonal-precision workload: shapes, storage dtype and seed."""
    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v, beta, d
    seed: int
    A_uniform: bool = True  # A_h ~ U(0.5, 2) per head; False -> A = 1
    I_prior: float = 1.0
    prefix: int = 0       # decode workloads: tokens that build the state first

    def with_(self, **kw) -> "DiagSpec":
        return replace(self, **kw)


@dataclass(frozen=True)
class IsoSpec:
    """An isotropic (scalar precision per head) workload."""
    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    seed: int
    lambda0: float = 1.0

    def with_(self, **kw) -> "IsoSpec":
        return replace(self, **kw)


@dataclass(frozen=True)
class VarlenSpec:
    """A packed variable-length batch of the diagonal scan."""
    name: str
    H: int
    N: int                # sequences
    total_T: int          # packed tokens per head
    d_k: int
    d_v: int
    dtype: str
    seed: int
    m_gating: bool = False
    I_prior: float = 1.0
    long_tokens: int = 0  # > 0: sequence 0 holds this many tokens, the rest cut at random

    def with_(self, **kw) -> "VarlenSpec":
        return replace(self, **kw)


WORKLOADS = {
    s.name: s for s in [
        DiagSpec("diag_b1h2t64d16_f32", 1, 2, 64, 16, 16, "f32", 1000, A_uniform=False),
        DiagSpec("diag_b8h16t2048d128_bf16", 8, 16, 2048, 128, 128, "bf16", 1001),
        DiagSpec("diag_b2h16t16384d128_bf16", 2, 16, 16384, 128, 128, "bf16", 1002),
        # diagonal KDN with process noise, at the headline shape
        DiagSpec("noise_b8h16t2048d128_bf16", 8, 16, 2048, 128, 128, "bf16", 1005),
        # Palimpsa-M gating (beta_t = d_t) at the headline shape
        DiagSpec("diagm_b8h16t2048d128_bf16", 8, 16, 2048, 128, 128, "bf16", 1006),
        # packed variable-length batch: 64 sequences, 16384 packed tokens per head
        VarlenSpec("varlen_n64h16t16384d128_bf16", 16, 64, 16384, 128, 128, "bf16", 1007),
        # gradient over the same packed batch
        VarlenSpec("varlenbwd_n64h16t16384d128_bf16", 16, 64, 16384, 128, 128, "bf16", 1007),
        # a skewed packed batch: one 8192-token sequence, 63 short ones in the other half
        VarlenSpec("varlenskew_n64h16t16384d128_bf16", 16, 64, 16384, 128, 128, "bf16", 1008,
                   long_tokens=8192),
        # gradient over the skewed batch
        VarlenSpec("varlenskewbwd_n64h16t16384d128_bf16", 16, 64, 16384, 128, 128, "bf16", 1008,
                   long_tokens=8192),
        # gradient of the headline forward workload (same inputs)
        DiagSpec("bwd_b8h16t2048d128_bf16", 8, 16, 2048, 128, 128, "bf16", 1001),
        # gradient of the long-sequence workload (same inputs)
        DiagSpec("bwd_b2h16t16384d128_bf16", 2, 16, 16384, 128, 128, "bf16", 1002),
        IsoSpec("iso_b1h32t65536d64_f32", 1, 32, 65536, 64, 64, 1003),
        # one decode token after a 512-token prefix that builds the state
        DiagSpec("decode_b256h16d128_bf16", 256, 16, 1, 128, 128, "bf16", 1004, prefix=512),
    ]
}


def workload(name: str):
    return WORKLOADS[name]


def _A(spec: DiagSpec) -> np.ndarray:
    if not spec.A_uniform:
        return np.ones(spec.H, dtype=np.float32)
    return _rng(spec.seed, 0xA).uniform(0.5, 2.0, size=spec.H).astype(np.float32)


def diag_head(spec: DiagSpec, b: int, h: int) -> dict:
    """Float32 draws for one head over prefix + T tokens (before any bf16 rounding)."""
    T = spec.prefix + spec.T
    g = _rng(spec.seed, b, h)
    q = g.standard_normal((T, spec.d_k), dtype=np.float32)
    k = g.standard_normal((T, spec.d_k), dtype=np.float32)
    k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
    v = g.standard_normal((T, spec.d_v), dtype=np.float32)
    beta = _sigmoid(g.standard_normal((T, spec.d_v), dtype=np.float32))
    d = _softplus(g.standard_normal(T, dtype=np.float32))
    return {"q": q, "k": k, "v": v, "beta": beta, "d": d}


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def diag_inputs(spec: DiagSpec) -> dict:
    """Whole-workload arrays [B,H,prefix+T,.] in storage dtype (bf16 as uint16 bits).

    Returns q, k, v, beta, d, A (float32 [H]), I_prior and the spec.
    """
    Tt = spec.prefix + spec.T
    shapes = {"q": (Tt, spec.d_k), "k": (Tt, spec.d_k), "v": (Tt, spec.d_v),
              "beta": (Tt, spec.d_v), "d": (Tt,)}
    npdt = np.uint16 if spec.dtype == "bf16" else np.float32
    out = {n: np.empty((spec.B, spec.H) + s, dtype=npdt) for n, s in shapes.items()}

    def one(bh):
        b, h = divmod(bh, spec.H)
        x = diag_head(spec, b, h)
        for n in shapes:
            out[n][b, h] = _store(x[n], spec.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(spec.B * spec.H)))
    out["A"] = _A(spec)
    out["I_prior"] = float(spec.I_prior)
    out["spec"] = spec
    return out


def grad_inputs(spec: DiagSpec, final_state: bool = True) -> dict:
    """Seeded upstream gradients for a gradient test: d_o [B,H,T,d_v] and, if
    final_state, d_I_T and d_mu_T [B,H,d_k,d_v]; all float32 standard normal
    (loss weights, so no structure beyond scale)."""
    g = _rng(spec.seed, 0xD0)
    out = {"d_o": g.standard_normal((spec.B, spec.H, spec.T, spec.d_v), dtype=np.float32)}
    if final_state:
        out["d_I_T"] = g.standard_normal((spec.B, spec.H, spec.d_k, spec.d_v), dtype=np.float32)
        out["d_mu_T"] = g.standard_normal((spec.B, spec.H, spec.d_k, spec.d_v), dtype=np.float32)
    return out


def varlen_grad_inputs(spec: VarlenSpec) -> dict:
    """Seeded upstream gradient of a packed batch: d_o [1,H,total_T,d_v]
    float32 standard normal."""
    g = _rng(spec.seed, 0xD1)
    return {"d_o": g.standard_normal((1, spec.H, spec.total_T, spec.d_v), dtype=np.float32)}


def noise_inputs(spec: DiagSpec) -> dict:
    """A diagonal workload's inputs plus the per-token decay a and process-noise
    variance p, float32 [B,H,T] (the d input is not used by this filter)."""
    out = diag_inputs(spec)
    g = _rng(spec.seed, 0xAB)
    shape = (spec.B, spec.H, spec.T)
    out["a"] = np.exp(-_softplus(g.standard_normal(shape, dtype=np.float32))).astype(np.float32)
    out["p"] = _softplus(g.standard_normal(shape, dtype=np.float32))
    return out


def varlen_inputs(spec: VarlenSpec) -> dict:
    """Packed inputs [1,H,total_T,.] (beta None under Palimpsa-M gating) plus
    cu_seqlens (int64 [N+1]) of the seeded length mix."""
    base = DiagSpec(spec.name, 1, spec.H, spec.total_T, spec.d_k, spec.d_v, spec.dtype, spec.seed,
                    I_prior=spec.I_prior)
    out = diag_inputs(base)
    if spec.m_gating:
        out["beta"] = None
    g = _rng(spec.seed, 0x1E)
    if spec.long_tokens > 0:
        L = spec.long_tokens
        cuts = np.sort(g.choice(np.arange(L + 1, spec.total_T), size=spec.N - 2, replace=False))
        cuts = np.concatenate([[L], cuts])
    elif spec.N > 1:
        cuts = np.sort(g.choice(np.arange(1, spec.total_T), size=spec.N - 1, replace=False))
    else:
        cuts = np.zeros(0, np.int64)
    out["cu_seqlens"] = np.concatenate([[0], cuts, [spec.total_T]]).astype(np.int64)
    return out


def state_inputs(spec: DiagSpec) -> dict:
    """A seeded starting state: I0 ~ U(0.2, 3.2) (positive precisions) and
    mu0 ~ N(0, 1), float32 [B,H,d_k,d_v]."""
    g = _rng(spec.seed, 0x50)
    shape = (spec.B, spec.H, spec.d_k, spec.d_v)
    return {"I0": (0.2 + 3.0 * g.random(shape)).astype(np.float32),
            "mu0": g.standard_normal(shape, dtype=np.float32)}


def iso_head(spec: IsoSpec, b: int, h: int) -> dict:
    g = _rng(spec.seed, b, h)
    T = spec.T
    a = np.exp(-_softplus(g.standard_normal(T, dtype=np.float32))).astype(np.float32)
    p = _softplus(g.standard_normal(T, dtype=np.float32))
    lam = _softplus(g.standard_normal(T, dtype=np.float32))
    q = g.standard_normal((T, spec.d_k), dtype=np.float32)
    k = g.standard_normal((T, spec.d_k), dtype=np.float32)
    k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
    v = g.standard_normal((T, spec.d_v), dtype=np.float32)
    return {"a": a, "p": p, "Lambda": lam, "q": q, "k": k, "v": v}


def iso_inputs(spec: IsoSpec, with_mean: bool = True) -> dict:
    """Whole-workload float32 arrays: a, p, Lambda [B,H,T]; q, k [B,H,T,d_k]; v [B,H,T,d_v]."""
    names = ["a", "p", "Lambda"] + (["q", "k", "v"] if with_mean else [])
    shp = {"a": (spec.T,), "p": (spec.T,), "Lambda": (spec.T,),
           "q": (spec.T, spec.d_k), "k": (spec.T, spec.d_k), "v": (spec.T, spec.d_v)}
    out = {n: np.empty((spec.B, spec.H) + shp[n], dtype=np.float32) for n in names}

    def one(bh):
        b, h = divmod(bh, spec.H)
        x = iso_head(spec, b, h)
        for n in names:
            out[n][b, h] = x[n]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(spec.B * spec.H)))
    out["lambda0"] = np.full((spec.B, spec.H), spec.lambda0, dtype=np.float32)
    out["spec"] = spec
    return out

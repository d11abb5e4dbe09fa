"""Helpers of the GPU parity tests: upload synthetic inputs, run the library,
compare with the oracle under the tolerance of the acceptance criterion."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from bayesian_memory_scan_amd import synth

RTOL = 1e-4  # acceptance: 1e-4 relative (fp32 state)


def dev_tensor(x: np.ndarray, device="cuda"):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def upload_diag(inp: dict, t_range=None, device="cuda"):
    sl = slice(None) if t_range is None else slice(*t_range)
    out = {n: dev_tensor(inp[n][:, :, sl], device) for n in ("q", "k", "v", "beta", "d")}
    out["A"] = dev_tensor(inp["A"], device)
    return out


def upload_iso(inp: dict, device="cuda"):
    out = {n: dev_tensor(inp[n], device) for n in ("a", "p", "Lambda") if n in inp}
    for n in ("q", "k", "v"):
        if n in inp:
            out[n] = dev_tensor(inp[n], device)
    out["lambda0"] = dev_tensor(inp["lambda0"], device)
    return out


def check_o(o_gpu: np.ndarray, ref: dict, what: str, rtol=RTOL):
    """|o - o_ref| <= rtol * s_ref, s_ref = sum_j |q_j mu_ref[j,i]| (bounds |o_ref|)."""
    err = np.abs(o_gpu.astype(np.float64) - ref["o"])
    bound = rtol * ref["s"] + 1e-30
    ratio = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert ratio <= 1.0, f"{what}: max |err|/(1e-4 s) = {ratio:.3f}"
    return ratio


def check_rel(x_gpu: np.ndarray, x_ref: np.ndarray, what: str, rtol=RTOL):
    """Elementwise relative error (values bounded away from 0, e.g. precisions)."""
    err = np.abs(x_gpu.astype(np.float64) - x_ref) / np.abs(x_ref)
    r = float(np.max(err)) if err.size else 0.0
    assert r <= rtol, f"{what}: max rel err {r:.3e}"
    return r


def check_state(x_gpu: np.ndarray, x_ref: np.ndarray, what: str, rtol=RTOL):
    """|dx| <= rtol * max(|x_ref|, rms(x_ref)) for a signed state (mu)."""
    scale = np.maximum(np.abs(x_ref), np.sqrt(np.mean(x_ref ** 2)) + 1e-30)
    r = float(np.max(np.abs(x_gpu.astype(np.float64) - x_ref) / scale)) if x_ref.size else 0.0
    assert r <= rtol, f"{what}: max scaled err {r:.3e}"
    return r


def diag_spec(B, H, T, dk, dv, dtype, seed=7, A_uniform=True, I_prior=1.0, prefix=0):
    return synth.DiagSpec(f"diag_test_{B}_{H}_{T}_{dk}_{dv}_{dtype}", B, H, T, dk, dv, dtype, seed,
                          A_uniform=A_uniform, I_prior=I_prior, prefix=prefix)


def compare_diag(inp, res, heads, ref=None, what="", I0=None, mu0=None):
    o, I_T, mu_T = (None if x is None else x.cpu().numpy() for x in res)
    ref = ref if ref is not None else oracle.diag_scan(inp, heads=heads, I0=I0, mu0=mu0)
    worst = 0.0
    for (b, h) in heads:
        r = ref[(b, h)]
        worst = max(worst, check_o(o[b, h], r, f"{what} o[{b},{h}]"))
        if I_T is not None:
            check_rel(I_T[b, h], r["I_T"], f"{what} I_T[{b},{h}]")
            check_state(mu_T[b, h], r["mu_T"], f"{what} mu_T[{b},{h}]")
    return worst

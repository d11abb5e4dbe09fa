"""How far the scan-compatible KDN approximations sit from the exact filter.

TEST INFRASTRUCTURE (CPU only): runs the oracle's exact dense-Riccati Kalman
filter (oracle_kdn_exact_head) beside its diagonal (per-entry, with process
noise) and isotropic (one precision per head) filters on the same seeded
inputs, and reports the relative read-out error of each approximation.

The Kalman Delta Networks abstract motivates both approximations by the cost
of exact tracking; this puts numbers on what they give up.  All three
filters share the model of the isotropic workload: decay a_t =
exp(-softplus(N(0,1))), process noise p_t = softplus(N(0,1)), observation
precision Lambda_t = softplus(N(0,1)) used for every value channel (beta_t[i]
= Lambda_t, so the isotropic filter sees the same evidence), unit-norm keys,
start P0 = Id, mean 0.  Regimes vary the keys and the dynamics.

Run:  python -m oracle.approx_study   (prints a markdown table)
"""
from __future__ import annotations

import numpy as np

import oracle


def _softplus(x):
    return np.logaddexp(0.0, x)


def regime_inputs(name: str, T: int, dk: int, dv: int, seed: int) -> dict:
    g = np.random.default_rng(seed)
    q = g.standard_normal((T, dk))
    v = g.standard_normal((T, dv))
    a = np.exp(-_softplus(g.standard_normal(T)))
    p = _softplus(g.standard_normal(T))
    lam = _softplus(g.standard_normal(T))
    if name == "axis keys":
        k = np.zeros((T, dk))
        k[np.arange(T), g.integers(0, dk, T)] = 1.0
    elif name == "low-rank keys":
        basis = np.linalg.qr(g.standard_normal((dk, 2)))[0]
        k = g.standard_normal((T, 2)) @ basis.T
    else:
        k = g.standard_normal((T, dk))
    if name == "slow decay, small noise":
        a = np.full(T, np.exp(-0.05))
        p = np.full(T, 0.01)
    k = k / np.linalg.norm(k, axis=1, keepdims=True)
    return {"q": q, "k": k, "v": v, "a": a, "p": p, "lam": lam}


REGIMES = ["random keys", "axis keys", "low-rank keys", "slow decay, small noise"]


def rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def study(T=256, dk=16, dv=16, heads=4, lib=None):
    """Mean over heads of ||o_approx - o_exact|| / ||o_exact|| per regime."""
    lib = lib or oracle.load()
    rows = []
    for name in REGIMES:
        ed, ei = [], []
        for h in range(heads):
            x = regime_inputs(name, T, dk, dv, seed=1000 + 17 * h + REGIMES.index(name))
            beta = np.repeat(x["lam"][:, None], dv, axis=1)
            ex = oracle.kdn_exact_head(x["q"], x["k"], x["v"], beta, x["a"], x["p"], lib=lib)
            dg = oracle.diag_noise_head(x["q"], x["k"], x["v"], beta, x["a"], x["p"], lib=lib)
            iso = oracle.iso_head(x["a"], x["p"], x["lam"], 1.0, x["q"], x["k"], x["v"], lib=lib)
            ed.append(rel(dg["o"], ex["o"]))
            ei.append(rel(iso["o"], ex["o"]))
        rows.append((name, float(np.mean(ed)), float(np.mean(ei))))
    return rows


def main():
    T, dk, dv, heads = 256, 16, 16, 4
    rows = study(T, dk, dv, heads)
    print(f"Relative read-out error vs the exact filter (T={T}, d_k=d_v={dk}, mean of {heads} heads)\n")
    print("| regime | diagonal KDN | isotropic KDN |")
    print("|---|---|---|")
    for name, d, i in rows:
        print(f"| {name} | {d:.3g} | {i:.3g} |")


if __name__ == "__main__":
    main()

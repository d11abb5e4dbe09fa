"""The pins catch plausible mistakes: each mutant is a copy of the oracle with
one planted error (a dropped term, a wrong sign, a wrong operand or index),
built on the CPU; at least one pin must fail on every mutant."""
import os

import pytest

import oracle
from tests import oracle_pins as pins

MUTANTS = {
    "prior_term_dropped": ("(1.0 - alpha) * I_prior", "0.0 * I_prior"),
    "prior_sign": ("(1.0 - alpha) * I_prior", "(1.0 + alpha) * I_prior"),
    "key_not_squared": ("bt[i] * kt[j] * kt[j]", "bt[i] * kt[j]"),
    "mean_not_decayed": ("alpha * (I_old / I_new) * mu[e]", "(I_old / I_new) * mu[e]"),
    "mean_ratio_inverted": ("alpha * (I_old / I_new) * mu[e]", "alpha * (I_new / I_old) * mu[e]"),
    "write_uses_query": ("bt[i] * vt[i] * kt[j]", "bt[i] * vt[i] * qt[j]"),
    "write_drops_beta": ("bt[i] * vt[i] * kt[j]", "vt[i] * kt[j]"),
    "forget_ignores_A": ("exp(-A * d[t])", "exp(-d[t])"),
    "readout_transposed": ("qt[j] * mu[j * dv + i];\n                acc", "qt[j] * mu[(i * dk + j) % n];\n                acc"),
    "iso_decay_not_squared": ("a[t] * a[t] / lambda + p[t]", "a[t] / lambda + p[t]"),
    "iso_noise_dropped": ("a[t] * a[t] / lambda + p[t]", "a[t] * a[t] / lambda"),
    "iso_mean_not_decayed": ("mean_pred = a[t] * mu[e]", "mean_pred = mu[e]"),
    "iso_write_uses_query": ("Lam[t] * kt[j] * vt[i]", "Lam[t] * qt[j] * vt[i]"),
    "iso_obs_precision_squared": ("lambda_pred + Lam[t];", "lambda_pred + Lam[t] * Lam[t];"),
    # gradient of the diagonal path
    "bwd_mean_ignores_precision": ("gIn = gI - gM * mn / In;", "gIn = gI;"),
    "bwd_key_square_factor": ("gIn * 2.0 * b * kk;", "gIn * b * kk;"),
    "bwd_gate_sign": ("g[4][t] += g_alpha * (-A * alpha);", "g[4][t] += g_alpha * (A * alpha);"),
    "bwd_gate_drops_prior": ("gIn * (Ip - I_prior);", "gIn * Ip;"),
    "bwd_mean_carry_undecayed": ("gM_prev = gM * alpha * Ip / In;", "gM_prev = gM * Ip / In;"),
    "bwd_precision_carry_drops_mean": ("gI_prev = gM * alpha * mp / In + gIn * alpha;",
                                       "gI_prev = gIn * alpha;"),
    "bwd_query_grad_uses_old_mean": ("g[0][t * dk + j] += mn * go;", "g[0][t * dk + j] += mp * go;"),
    "bwd_value_grad_drops_beta": ("g[2][t * dv + i] += gM * b * kk / In;",
                                  "g[2][t * dv + i] += gM * kk / In;"),
    "bwd_prior_start_dropped": ("g[6][0] += gI;", "g[6][0] += 0.0 * gI;"),
    "bwd_readout_uses_key": ("gM += qq * go;", "gM += kk * go;"),
    # diagonal KDN with process noise
    "noise_dropped": ("var_pred[j] = a[t] * a[t] / lam[e] + p[t];", "var_pred[j] = a[t] * a[t] / lam[e];"),
    "noise_decay_not_squared": ("var_pred[j] = a[t] * a[t] / lam[e] + p[t];", "var_pred[j] = a[t] / lam[e] + p[t];"),
    "noise_mean_not_decayed": ("mean_pred[j] = a[t] * mu[e];", "mean_pred[j] = mu[e];"),
    "noise_obs_not_squared": ("lam[e] = 1.0 / var_pred[j] + bt[i] * kt[j] * kt[j];", "lam[e] = 1.0 / var_pred[j] + bt[i] * kt[j];"),
    "noise_gain_ignores_obs_noise": ("double S = 1.0 / bt[i];", "double S = 0.0;"),
    "noise_write_not_residual": ("const double residual = vt[i] - prediction;", "const double residual = vt[i];"),
    "noise_gain_uses_query": ("var_pred[j] * kt[j] * residual / S;", "var_pred[j] * qt[j] * residual / S;"),
    # exact KDN
    "exact_noise_dropped": ("Pi[r * dk + r] += p[t];", "Pi[r * dk + r] += 0.0 * p[t];"),
    "exact_mean_not_decayed": ("mi[r] *= a[t];", "mi[r] *= 1.0;"),
    "exact_gain_unnormalised": ("mi[r] += u[r] / S * resid;", "mi[r] += u[r] * resid;"),
    "exact_cov_update_sign": ("Pi[r * dk + c] -= u[r] * u[c] / S;", "Pi[r * dk + c] += u[r] * u[c] / S;"),
    "exact_obs_noise_wrong": ("double S = 1.0 / beta[t * dv + i];", "double S = beta[t * dv + i];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(before, after, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = oracle.load(oracle.build(src=str(path), out=str(tmp_path / f"lib_{name}.so")))
    failures = 0
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, FloatingPointError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught mutant {name}"

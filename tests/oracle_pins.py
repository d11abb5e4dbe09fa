"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each pin takes a loaded oracle library, so the same checks also run against
deliberately broken copies of the oracle (tests/test_oracle_mutants.py).  None
of them retypes the oracle's own update lines: they use closed forms, special
cases, an independently coded textbook filter, Mobius-matrix products and
structural identities.

Sources (page title and section):
  Palimpsa = "Learning to Remember, Learn, and Forget in Attention-Based
             Models", Metodologia 1-2 (forget gate, I_t and mu_t updates) and
             4 (Mamba2 as the limit where I_t stays at I_prior).
  KLA      = "Riassunto Tecnico: Kalman Linear Attention (KLA)", Metodologia
             1 (OU prior, observation precision, query read-out), 2 (precision
             as a Mobius map, affine information mean), 3 (gates from
             precision ratios).
  KDN      = "Kalman Delta Networks" abstract (scalar-precision isotropic
             variant, Mobius uncertainty recurrences, constant-memory decoding).
"""
from __future__ import annotations

import numpy as np

import oracle

RTOL = 1e-11  # fp64 sequential vs. closed form: tiny inputs, well conditioned


def _close(x, y, rtol=RTOL, atol=0.0, what=""):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    scale = np.maximum(np.abs(y), np.max(np.abs(y)) * 1e-3 + 1e-300)
    err = np.max(np.abs(x - y) / scale) if x.size else 0.0
    assert np.all(np.abs(x - y) <= rtol * scale + atol), f"{what}: max rel err {err:.3e}"


def diag_case(seed=7, T=9, dk=3, dv=5, A=0.7, I_prior=1.3, with_state=True):
    g = np.random.default_rng(seed)
    k = g.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    c = dict(
        q=g.standard_normal((T, dk)), k=k, v=g.standard_normal((T, dv)),
        beta=1.0 / (1.0 + np.exp(-g.standard_normal((T, dv)))),
        d=np.log1p(np.exp(g.standard_normal(T))), A=A, I_prior=I_prior,
    )
    if with_state:
        c["I0"] = 0.5 + g.random((dk, dv)) * 2.0
        c["mu0"] = g.standard_normal((dk, dv))
    return c


def _run_diag(lib, c, **over):
    c = {**c, **over}
    return oracle.diag_head(c["q"], c["k"], c["v"], c["beta"], c["d"], c["A"], c["I_prior"],
                            I0=c.get("I0"), mu0=c.get("mu0"), lib=lib)


# ---------------------------------------------------------------------------
# Diagonal-precision path
# ---------------------------------------------------------------------------

def pin_diag_closed_form(lib):
    """P-1.  Multiplying the Palimpsa mean update by I_t gives the affine
    information-form recurrence eta_t = alpha_t eta_{t-1} + (beta_t v_t) (outer) k_t,
    and I_t - I_prior decays by the same alpha.  Unrolled, with
    G(s,t) = prod_{r=s+1..t} alpha_r:
      I_t   = I_prior + G(0,t)(I_0 - I_prior) + sum_s G(s,t) beta_s (outer) k_s^2
      eta_t = G(0,t) I_0 mu_0 + sum_s G(s,t) (beta_s v_s) (outer) k_s
      mu_t  = eta_t / I_t,  o_t = mu_t^T q_t.
    Checked at every prefix length so every o_t is covered."""
    for c in (diag_case(), diag_case(seed=11, T=6, dk=4, dv=2, A=1.9, I_prior=0.4)):
        T = c["q"].shape[0]
        alpha = np.exp(-c["A"] * c["d"])
        res = _run_diag(lib, c)
        for t in range(1, T + 1):
            G = lambda s: np.prod(alpha[s:t])  # tokens are 1-based: G(s,t) = alpha_{s+1..t}
            I = c["I_prior"] + G(0) * (c["I0"] - c["I_prior"])
            eta = G(0) * c["I0"] * c["mu0"]
            for s in range(1, t + 1):
                ks, bs, vs = c["k"][s - 1], c["beta"][s - 1], c["v"][s - 1]
                I = I + G(s) * np.outer(ks ** 2, bs)
                eta = eta + G(s) * np.outer(ks, bs * vs)
            mu = eta / I
            _close(res["o"][t - 1], mu.T @ c["q"][t - 1], what=f"o_{t}")
            if t == T:
                _close(res["I_T"], I, what="I_T")
                _close(res["mu_T"], mu, what="mu_T")
        # the error scale bounds the read-out
        assert np.all(res["s"] >= np.abs(res["o"]) * (1 - 1e-15))


def pin_diag_no_write(lib):
    """P-2.  beta = 0 and I_0 = I_prior: the precision stays at the prior and
    the mean only decays, mu_t = (prod alpha) mu_0."""
    c = diag_case(seed=3, with_state=True)
    c["beta"] = np.zeros_like(c["beta"])
    c["I0"] = np.full_like(c["I0"], c["I_prior"])
    res = _run_diag(lib, c)
    _close(res["I_T"], np.full_like(c["I0"], c["I_prior"]), rtol=1e-14, what="I_T")
    decay = np.prod(np.exp(-c["A"] * c["d"]))
    _close(res["mu_T"], decay * c["mu0"], rtol=1e-13, what="mu_T")
    _close(res["o"][-1], (decay * c["mu0"]).T @ c["q"][-1], rtol=1e-12, what="o_T")


def pin_diag_positive(lib):
    """P-3.  With beta >= 0 the precision never drops below min(I_0, I_prior)
    (induction on the Palimpsa I_t update); it also never decreases below the
    prior once it starts above it."""
    for seed in range(4):
        c = diag_case(seed=100 + seed, T=12)
        c["I0"] = c["I0"] * 0.1
        lo = min(np.min(c["I0"]), c["I_prior"])
        for t in range(1, 13):
            res = _run_diag(lib, c, q=c["q"][:t], k=c["k"][:t], v=c["v"][:t],
                            beta=c["beta"][:t], d=c["d"][:t])
            assert np.all(res["I_T"] >= lo * (1 - 1e-15)), "precision fell below its floor"


def pin_diag_mamba2_limit(lib):
    """P-4.  Palimpsa Metodologia 4: when the importance stays at I_prior the
    model is Mamba2.  With I_prior much larger than beta k^2 the oracle must
    approach the scalar-decay gated linear-attention recurrence
    S_t = alpha_t S_{t-1} + k_t (beta_t v_t)^T,  o_t = S_t^T q_t / I_prior,
    with relative gap of order max(beta k^2) / I_prior."""
    c = diag_case(seed=5, T=10, dk=4, dv=3, with_state=False)
    big = 1e9
    res = _run_diag(lib, c, I_prior=big)
    alpha = np.exp(-c["A"] * c["d"])
    S = np.zeros((4, 3))
    for t in range(10):
        S = alpha[t] * S + np.outer(c["k"][t], c["beta"][t] * c["v"][t])
        _close(res["o"][t] * big, S.T @ c["q"][t], rtol=1e-7, what=f"GLA o_{t}")


def pin_diag_special_gates(lib):
    """P-5.  d = 0 (alpha = 1, nothing forgotten): the mean is the running
    precision-weighted average (I_0 mu_0 + sum beta v (outer) k) / (I_0 + sum beta (outer) k^2).
    d huge (alpha = 0, everything forgotten): memoryless,
    mu_t = (beta v (outer) k) / (I_prior + beta (outer) k^2)."""
    c = diag_case(seed=9)
    res = _run_diag(lib, c, d=np.zeros_like(c["d"]))
    num = c["I0"] * c["mu0"] + sum(np.outer(c["k"][t], c["beta"][t] * c["v"][t]) for t in range(9))
    den = c["I0"] + sum(np.outer(c["k"][t] ** 2, c["beta"][t]) for t in range(9))
    _close(res["I_T"], den, what="I_T (alpha=1)")
    _close(res["mu_T"], num / den, what="mu_T (alpha=1)")

    res = _run_diag(lib, c, d=np.full_like(c["d"], 1e4))
    kT, bT, vT = c["k"][-1], c["beta"][-1], c["v"][-1]
    den = c["I_prior"] + np.outer(kT ** 2, bT)
    _close(res["I_T"], den, what="I_T (alpha=0)")
    _close(res["mu_T"], np.outer(kT, bT * vT) / den, what="mu_T (alpha=0)")


def pin_diag_chaining(lib):
    """P-6.  Constant-memory decoding (KDN abstract): the state is all that
    carries over, so scan(T1) then scan(T2) from its final state equals
    scan(T1 + T2), token for token."""
    c = diag_case(seed=21, T=11)
    full = _run_diag(lib, c)
    cut = 4
    first = _run_diag(lib, c, **{n: c[n][:cut] for n in ("q", "k", "v", "beta", "d")})
    second = _run_diag(lib, c, I0=first["I_T"], mu0=first["mu_T"],
                       **{n: c[n][cut:] for n in ("q", "k", "v", "beta", "d")})
    np.testing.assert_array_equal(np.vstack([first["o"], second["o"]]), full["o"])
    np.testing.assert_array_equal(second["I_T"], full["I_T"])
    np.testing.assert_array_equal(second["mu_T"], full["mu_T"])


DIAG_PINS = [pin_diag_closed_form, pin_diag_no_write, pin_diag_positive,
             pin_diag_mamba2_limit, pin_diag_special_gates, pin_diag_chaining]


# ---------------------------------------------------------------------------
# Isotropic (scalar precision) path
# ---------------------------------------------------------------------------

def iso_case(seed=13, T=10, dk=3, dv=4):
    g = np.random.default_rng(seed)
    sp = lambda x: np.log1p(np.exp(x))
    k = g.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    return dict(a=np.exp(-sp(g.standard_normal(T))), p=sp(g.standard_normal(T)),
                Lam=sp(g.standard_normal(T)), lambda0=1.0 + g.random(),
                q=g.standard_normal((T, dk)), k=k, v=g.standard_normal((T, dv)),
                mu0=g.standard_normal((dk, dv)))


def mobius_matrix(a, p, Lam):
    """Predict (variance a^2/l + p) then add Lam, as a 2x2 fractional-linear map
    l -> ((1 + Lam p) l + Lam a^2) / (p l + a^2)   (KLA Metodologia 2)."""
    return np.array([[1.0 + Lam * p, Lam * a * a], [p, a * a]])


def _apply(M, lam0):
    return (M[0, 0] * lam0 + M[0, 1]) / (M[1, 0] * lam0 + M[1, 1])


def _compose(Ms, rng):
    """Product M_n ... M_1 in a random bracketing (later factors on the left)."""
    items = list(Ms)
    while len(items) > 1:
        i = int(rng.integers(0, len(items) - 1))
        items[i:i + 2] = [items[i + 1] @ items[i]]
    return items[0]


def pin_iso_mobius(lib):
    """P-7.  Mobius maps compose associatively (KLA Metodologia 2): lambda_t
    from the oracle's predict/update equals the composed matrix product applied
    to lambda_0, in any bracketing.  det M_t = a_t^2 > 0 and every entry is
    positive, so lambda_t > 0."""
    c = iso_case(T=40)
    res = oracle.iso_head(c["a"], c["p"], c["Lam"], c["lambda0"], lib=lib)
    rng = np.random.default_rng(0)
    Ms = [mobius_matrix(c["a"][t], c["p"][t], c["Lam"][t]) for t in range(40)]
    for t in range(1, 41):
        P = _compose(Ms[:t], rng)
        P = P / np.max(P)  # projective scale does not change the map
        _close(res["lambda"][t - 1], _apply(P, c["lambda0"]), rtol=1e-12, what=f"lambda_{t}")
        assert abs(np.linalg.det(Ms[t - 1]) - c["a"][t - 1] ** 2) < 1e-12
    assert np.all(res["lambda"] > 0)


def pin_iso_scalar_kalman(lib):
    """P-8.  d_k = d_v = 1 with k = q = 1: the oracle is a scalar Kalman filter
    observing y_t = v_t with noise variance 1/Lambda_t.  Compare with the
    covariance-form textbook filter:
      P- = a^2 P + p;  K = P- / (P- + 1/Lambda);  m = a m + K (y - a m);
      P = (1 - K) P-;  then lambda_t = 1/P and o_t = m."""
    c = iso_case(seed=17, T=25, dk=1, dv=1)
    ones = np.ones((25, 1))
    res = oracle.iso_head(c["a"], c["p"], c["Lam"], c["lambda0"], q=ones, k=ones,
                          v=c["v"], mu0=np.array([[0.3]]), lib=lib)
    P, m = 1.0 / c["lambda0"], 0.3
    for t in range(25):
        a, p, L, y = c["a"][t], c["p"][t], c["Lam"][t], c["v"][t, 0]
        Pm = a * a * P + p
        K = Pm / (Pm + 1.0 / L)
        m = a * m + K * (y - a * m)
        P = (1.0 - K) * Pm
        _close(res["lambda"][t], 1.0 / P, rtol=1e-12, what=f"lambda_{t}")
        _close(res["o"][t, 0], m, rtol=1e-12, what=f"m_{t}")


def pin_iso_fixed_point(lib):
    """P-9.  Constant (a, p, Lambda): lambda_t converges to the positive root of
    p l^2 + (a^2 - 1 - Lambda p) l - Lambda a^2 = 0 (steady-state scalar
    Riccati).  p = 0 reduces to the affine l_t = l_{t-1} / a^2 + Lambda, and
    a = 1, p = 0 to l_t = l_0 + t Lambda."""
    for a, p, L in [(0.8, 0.3, 1.2), (0.95, 2.0, 0.05), (0.3, 0.01, 3.0)]:
        T = 400
        res = oracle.iso_head(np.full(T, a), np.full(T, p), np.full(T, L), 1.0, lib=lib)
        b = a * a - 1.0 - L * p
        star = (-b + np.sqrt(b * b + 4 * p * L * a * a)) / (2 * p)
        _close(res["lambda"][-1], star, rtol=1e-12, what="fixed point")
    T = 12
    res = oracle.iso_head(np.full(T, 0.9), np.zeros(T), np.full(T, 0.5), 2.0, lib=lib)
    lam, ref = 2.0, []
    for _ in range(T):
        lam = lam / 0.81 + 0.5
        ref.append(lam)
    _close(res["lambda"], ref, rtol=1e-13, what="p=0 affine")
    res = oracle.iso_head(np.ones(T), np.zeros(T), np.full(T, 0.25), 2.0, lib=lib)
    _close(res["lambda"], 2.0 + 0.25 * np.arange(1, T + 1), rtol=1e-14, what="a=1,p=0")


def pin_iso_mean_closed_form(lib):
    """P-10.  KLA Metodologia 2-3: with the precisions known, the mean is the
    affine recurrence mu_t = F_t mu_{t-1} + G_t k_t v_t^T, forget gate
    F_t = a_t lambda^-_t / lambda_t, write gate G_t = Lambda_t / lambda_t,
    where lambda^-_t = lambda_{t-1} / (a_t^2 + p_t lambda_{t-1}).  Unrolled:
    mu_t = (prod F) mu_0 + sum_s (prod_{r>s} F_r) G_s k_s v_s^T.  The
    precisions here come from Mobius products, not from the oracle."""
    c = iso_case(seed=29, T=9, dk=3, dv=4)
    T = 9
    res = oracle.iso_head(c["a"], c["p"], c["Lam"], c["lambda0"], q=c["q"], k=c["k"],
                          v=c["v"], mu0=c["mu0"], lib=lib)
    lam = [c["lambda0"]]
    P = np.eye(2)
    for t in range(T):
        P = mobius_matrix(c["a"][t], c["p"][t], c["Lam"][t]) @ P
        lam.append(_apply(P, c["lambda0"]))
    lam_pred = [lam[t] / (c["a"][t] ** 2 + c["p"][t] * lam[t]) for t in range(T)]
    F = np.array([c["a"][t] * lam_pred[t] / lam[t + 1] for t in range(T)])
    G = np.array([c["Lam"][t] / lam[t + 1] for t in range(T)])
    assert np.all((F > 0) & (F < c["a"])) and np.all((G > 0) & (G <= 1))
    for t in range(1, T + 1):
        mu = np.prod(F[:t]) * c["mu0"]
        for s in range(1, t + 1):
            mu = mu + np.prod(F[s:t]) * G[s - 1] * np.outer(c["k"][s - 1], c["v"][s - 1])
        _close(res["o"][t - 1], mu.T @ c["q"][t - 1], rtol=1e-12, what=f"o_{t}")
        if t == T:
            _close(res["mu_T"], mu, rtol=1e-12, what="mu_T")


ISO_PINS = [pin_iso_mobius, pin_iso_scalar_kalman, pin_iso_fixed_point, pin_iso_mean_closed_form]


# ---------------------------------------------------------------------------
# Gradient of the diagonal path (the pages print none: it is pinned to the
# forward oracle by central finite differences, which share no code with it)
# ---------------------------------------------------------------------------
def _bwd_loss_weights(c, seed=99):
    g = np.random.default_rng(seed)
    T, dk = c["q"].shape
    dv = c["v"].shape[1]
    return g.standard_normal((T, dv)), g.standard_normal((dk, dv)), g.standard_normal((dk, dv))


def _loss(lib, c, W):
    r = _run_diag(lib, c)
    return float(np.sum(W[0] * r["o"]) + np.sum(W[1] * r["I_T"]) + np.sum(W[2] * r["mu_T"]))


def _finite_difference(lib, c, W, name, idx, rel_h=1e-5):
    x = c[name]
    base = float(x if np.isscalar(x) else x[idx])
    h = rel_h * max(1.0, abs(base))

    def at(val):
        if np.isscalar(x):
            return _loss(lib, {**c, name: val}, W)
        y = np.array(x, dtype=np.float64, copy=True)
        y[idx] = val
        return _loss(lib, {**c, name: y}, W)

    return (at(base + h) - at(base - h)) / (2.0 * h)


def _run_bwd(lib, c, W, with_final=True):
    return oracle.diag_head_bwd(c["q"], c["k"], c["v"], c["beta"], c["d"], c["A"], c["I_prior"],
                                W[0], I0=c.get("I0"), mu0=c.get("mu0"),
                                dI_T=W[1] if with_final else None,
                                dmu_T=W[2] if with_final else None, lib=lib)


def _check_fd(lib, c, W, grads, names):
    for gname, iname in names:
        x = c[iname]
        idxs = [()] if np.isscalar(x) else list(np.ndindex(np.shape(x)))
        fd = np.array([_finite_difference(lib, c, W, iname, ix) for ix in idxs])
        got = np.atleast_1d(np.asarray(grads[gname], np.float64)).reshape(-1)
        _close(got, fd, rtol=2e-6, atol=1e-9, what=f"{gname} vs finite differences")


def pin_bwd_finite_differences(lib):
    """Every gradient, with a starting state and gradients into the final
    state, equals the central finite difference of the forward oracle's loss."""
    c = diag_case(seed=21, T=6, dk=3, dv=2, A=0.9, I_prior=0.8)
    W = _bwd_loss_weights(c)
    g = _run_bwd(lib, c, W)
    _check_fd(lib, c, W, g, [("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"),
                             ("dd", "d"), ("dA", "A"), ("dI_prior", "I_prior"),
                             ("dI0", "I0"), ("dmu0", "mu0")])


def pin_bwd_prior_start(lib):
    """Without a starting state the memory starts at I_prior (mean 0): the
    start's dependence on I_prior is part of dI_prior, and no state gradients
    are returned."""
    c = diag_case(seed=22, T=5, dk=2, dv=3, A=1.4, I_prior=1.7, with_state=False)
    W = _bwd_loss_weights(c, seed=5)
    g = _run_bwd(lib, c, W)
    assert "dI0" not in g and "dmu0" not in g
    _check_fd(lib, c, W, g, [("dI_prior", "I_prior"), ("dd", "d"), ("dk", "k"), ("dbeta", "beta")])


def pin_bwd_readout_only(lib):
    """Loss on the outputs alone (no final-state gradient) still matches."""
    c = diag_case(seed=23, T=7, dk=2, dv=2, A=0.3, I_prior=2.2)
    W = _bwd_loss_weights(c, seed=6)
    W = (W[0], np.zeros_like(W[1]), np.zeros_like(W[2]))
    g = _run_bwd(lib, c, W, with_final=False)
    _check_fd(lib, c, W, g, [("dq", "q"), ("dv", "v"), ("dI0", "I0"), ("dmu0", "mu0"),
                             ("dA", "A")])


def pin_bwd_empty_sequence(lib):
    """T = 0: the final state is the starting state, so its gradient passes
    straight through and every per-token gradient is empty."""
    c = diag_case(seed=24, T=0, dk=3, dv=2)
    W = _bwd_loss_weights(c)
    g = _run_bwd(lib, c, W)
    _close(g["dI0"], W[1], what="dI0 at T=0")
    _close(g["dmu0"], W[2], what="dmu0 at T=0")
    assert g["dA"] == 0.0 and g["dI_prior"] == 0.0 and g["dq"].size == 0


def pin_bwd_scale_bounds(lib):
    """Each returned scale is the sum of the absolute values of the terms of
    its gradient, so it bounds it; and it is not vacuous (a gradient that is a
    single product has |g| equal to its scale)."""
    c = diag_case(seed=25, T=8, dk=3, dv=3)
    W = _bwd_loss_weights(c)
    g = _run_bwd(lib, c, W)
    for n in oracle.GRAD_NAMES:
        assert np.all(np.abs(g[n]) <= g["scale_" + n] * (1 + 1e-12) + 1e-300), n
    # dq_t[j] = sum_i mu_t[j,i] dout_t[i] with dv = 1 is one product
    c1 = diag_case(seed=26, T=4, dk=2, dv=1)
    W1 = _bwd_loss_weights(c1)
    g1 = _run_bwd(lib, c1, W1)
    _close(np.abs(g1["dq"]), g1["scale_dq"], what="single-term scale")


# ---------------------------------------------------------------------------
# Diagonal KDN with process noise (per-entry scalar Kalman filter)
# ---------------------------------------------------------------------------
def noise_case(seed=41, T=11, dk=3, dv=4):
    g = np.random.default_rng(seed)
    k = g.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    return dict(q=g.standard_normal((T, dk)), k=k, v=g.standard_normal((T, dv)),
                beta=1.0 / (1.0 + np.exp(-g.standard_normal((T, dv)))),
                a=np.exp(-np.log1p(np.exp(g.standard_normal(T)))),
                p=np.log1p(np.exp(g.standard_normal(T))),
                lam0=0.5 + g.random((dk, dv)) * 2.0, mu0=g.standard_normal((dk, dv)))


def _run_noise(lib, c, **over):
    c = {**c, **over}
    return oracle.diag_noise_head(c["q"], c["k"], c["v"], c["beta"], c["a"], c["p"],
                                  lam0=c.get("lam0"), mu0=c.get("mu0"), lib=lib)


def pin_noise_equals_isotropic_single_entry(lib):
    """With one key and one value channel and k_t = +-1, the entry's
    observation precision beta k^2 is beta and its write beta v k: exactly the
    isotropic filter with Lambda_t = beta_t (an independent, pinned oracle)."""
    g = np.random.default_rng(42)
    T = 13
    c = noise_case(seed=42, T=T, dk=1, dv=1)
    c["k"] = np.where(g.random((T, 1)) < 0.5, -1.0, 1.0)
    c["lam0"] = np.array([[1.7]])
    c["mu0"] = np.array([[0.4]])
    r = _run_noise(lib, c)
    iso = oracle.iso_head(c["a"], c["p"], c["beta"][:, 0], 1.7, c["q"], c["k"], c["v"],
                          mu0=c["mu0"], lib=lib)
    _close(r["I_T"][0, 0], iso["lambda"][-1], what="precision vs isotropic")
    _close(r["o"], iso["o"], what="read-out vs isotropic")
    _close(r["mu_T"], iso["mu_T"], what="mean vs isotropic")


def pin_noise_mobius(lib):
    """Each entry's precision is the ordered product of its Mobius maps
    [[1 + w p, w a^2], [p, a^2]] (w = beta k^2) applied to lambda_0."""
    c = noise_case(seed=43)
    r = _run_noise(lib, c)
    T, dk = c["q"].shape
    dv = c["v"].shape[1]
    for j in range(dk):
        for i in range(dv):
            P = np.eye(2)
            for t in range(T):
                w = c["beta"][t, i] * c["k"][t, j] ** 2
                M = np.array([[1 + w * c["p"][t], w * c["a"][t] ** 2], [c["p"][t], c["a"][t] ** 2]])
                P = M @ P
            lam0 = c["lam0"][j, i]
            _close(r["I_T"][j, i], (P[0, 0] * lam0 + P[0, 1]) / (P[1, 0] * lam0 + P[1, 1]),
                   what="precision vs Mobius product")


def pin_noise_mean_field_step(lib):
    """Every step is the mean-field projection of an exact one-step posterior:
    starting from the diagonal filter's state after t tokens (means mu, a
    diagonal covariance diag(1/lambda) per column), one step of the exact
    dense filter gives the diagonal filter's mean after t + 1 tokens, and the
    diagonal of the exact posterior precision is its lambda.  The exact
    filter is an independently coded covariance-form Riccati recursion."""
    c = noise_case(seed=44, T=9, dk=4, dv=3)
    T, dk = c["q"].shape
    dv = c["v"].shape[1]
    for t in range(T):
        before = _run_noise(lib, {**c, **{n: c[n][:t] for n in ("q", "k", "v", "beta", "a", "p")}})
        after = _run_noise(lib, {**c, **{n: c[n][:t + 1] for n in ("q", "k", "v", "beta", "a", "p")}})
        P0 = np.stack([np.diag(1.0 / before["I_T"][:, i]) for i in range(dv)])
        sl = lambda n: c[n][t:t + 1]
        ex = oracle.kdn_exact_head(sl("q"), sl("k"), sl("v"), sl("beta"), sl("a"), sl("p"), P0=P0,
                                   mu0=before["mu_T"], lib=lib)
        _close(after["mu_T"], ex["mu_T"], rtol=1e-10, what=f"mean-field mean, step {t}")
        for i in range(dv):
            _close(after["I_T"][:, i], np.diag(np.linalg.inv(ex["P_T"][i])), rtol=1e-10,
                   what=f"mean-field precision, step {t}")


def pin_noise_residual_write(lib):
    """A token whose value the current mean already predicts exactly
    (v = k^T a mu) writes nothing: only the precision and the decay move."""
    c = noise_case(seed=45, T=1, dk=3, dv=2)
    c["v"] = (c["k"][0] @ (c["a"][0] * c["mu0"]))[None, :]
    r = _run_noise(lib, c)
    _close(r["mu_T"], c["a"][0] * c["mu0"], what="no residual, no write")


# ---------------------------------------------------------------------------
# Palimpsa-M gating (beta_t = d_t) and the packed variable-length batch
# ---------------------------------------------------------------------------
def _m_inputs(T=9, dk=3, dv=4, seed=51, H=2):
    from bayesian_memory_scan_amd import synth
    spec = synth.DiagSpec(f"m_pin_{seed}", 1, H, T, dk, dv, "f32", seed)
    inp = synth.diag_inputs(spec)
    inp["beta"] = None
    return inp


def pin_m_gating_mamba2_limit(lib):
    """Palimpsa Metodologia 3-4: with d_t as both forget and input gate and
    I_prior far above d k^2 the model is Mamba2's recurrence
    S_t = exp(-A d_t) S_{t-1} + d_t k_t v_t^T, o_t = S_t^T q_t / I_prior."""
    inp = _m_inputs()
    inp["I_prior"] = 1e9
    res = oracle.diag_scan(inp, lib=lib)
    for h in range(2):
        q, k, v, d = (inp[n][0, h].astype(np.float64) for n in ("q", "k", "v", "d"))
        alpha = np.exp(-float(inp["A"][h]) * d)
        S = np.zeros((q.shape[1], v.shape[1]))
        for t in range(q.shape[0]):
            S = alpha[t] * S + d[t] * np.outer(k[t], v[t])
            _close(res[(0, h)]["o"][t] * 1e9, S.T @ q[t], rtol=1e-7, what=f"Mamba2 o_{t}")


def pin_m_gating_gradient(lib):
    """With d_t in both gates, dL/dd_t (forget path plus input path) equals the
    central finite difference of the forward loss in d_t."""
    inp = _m_inputs(T=6, dk=2, dv=3, seed=52, H=1)
    W = np.random.default_rng(53).standard_normal((1, 1, 6, 3))
    g = oracle.diag_scan_bwd(inp, W, lib=lib)[(0, 0)]
    assert "dbeta" not in g

    def loss(d):
        x = dict(inp)
        x["d"] = d.astype(np.float32) if d.dtype == np.float32 else d
        return float(np.sum(W[0, 0] * oracle.diag_scan(x, lib=lib)[(0, 0)]["o"]))

    d0 = inp["d"].astype(np.float64)
    fd = []
    for t in range(6):
        h = 1e-5 * max(1.0, abs(d0[0, 0, t]))
        dp, dm = d0.copy(), d0.copy()
        dp[0, 0, t] += h
        dm[0, 0, t] -= h
        fd.append((loss(dp) - loss(dm)) / (2 * h))
    _close(g["dd"], np.array(fd), rtol=2e-6, atol=1e-9, what="dd under Palimpsa-M gating")


def pin_varlen_continuation(lib):
    """A packed batch of two sequences, the second started from the first's
    final state, equals one run over their concatenation; an empty sequence
    returns its starting state."""
    from bayesian_memory_scan_amd import synth
    spec = synth.DiagSpec("varlen_pin", 1, 2, 20, 3, 2, "f32", 54)
    inp = synth.diag_inputs(spec)
    whole = oracle.diag_scan(inp, lib=lib)
    first = oracle.diag_scan_varlen(inp, [0, 7], lib=lib)
    I7 = np.stack([first[(0, h)]["I_T"] for h in range(2)])[None]
    m7 = np.stack([first[(0, h)]["mu_T"] for h in range(2)])[None]
    I0 = np.concatenate([np.ones((1, 2, 3, 2)) * 2.0, I7, np.ones((1, 2, 3, 2)) * 0.5])
    m0 = np.concatenate([np.zeros((1, 2, 3, 2)), m7, np.full((1, 2, 3, 2), 0.3)])
    runs = oracle.diag_scan_varlen(inp, [0, 7, 20, 20], I0=I0, mu0=m0, lib=lib)
    for h in range(2):
        _close(np.concatenate([first[(0, h)]["o"], runs[(1, h)]["o"]]), whole[(0, h)]["o"],
               what="continued read-out")
        _close(runs[(1, h)]["I_T"], whole[(0, h)]["I_T"], what="continued precision")
        _close(runs[(2, h)]["I_T"], I0[2, h], what="empty sequence precision")
        _close(runs[(2, h)]["mu_T"], m0[2, h], what="empty sequence mean")


M_PINS = [pin_m_gating_mamba2_limit, pin_m_gating_gradient, pin_varlen_continuation]


# ---------------------------------------------------------------------------
# Exact KDN (dense Riccati)
# ---------------------------------------------------------------------------
def pin_exact_axis_keys_equal_diagonal(lib):
    """With keys on the coordinate axes (k_t = +-e_j) and diagonal starting
    covariances, the covariance stays diagonal, so the exact filter and the
    diagonal (mean-field) filter are the same filter."""
    g = np.random.default_rng(61)
    c = noise_case(seed=61, T=15, dk=4, dv=3)
    T, dk = c["q"].shape
    dv = c["v"].shape[1]
    k = np.zeros((T, dk))
    k[np.arange(T), g.integers(0, dk, T)] = np.where(g.random(T) < 0.5, -1.0, 1.0)
    c["k"] = k
    P0 = np.stack([np.diag(1.0 / c["lam0"][:, i]) for i in range(dv)])
    ex = oracle.kdn_exact_head(c["q"], k, c["v"], c["beta"], c["a"], c["p"], P0=P0, mu0=c["mu0"], lib=lib)
    dg = _run_noise(lib, c)
    _close(ex["o"], dg["o"], rtol=1e-10, what="exact vs diagonal, axis keys")
    _close(ex["mu_T"], dg["mu_T"], rtol=1e-10, what="means, axis keys")
    for i in range(dv):
        _close(np.diag(ex["P_T"][i]), 1.0 / dg["I_T"][:, i], rtol=1e-10, what="variances, axis keys")


def pin_exact_static_regression(lib):
    """a = 1, p = 0: the posterior of a static column is Bayesian linear
    regression: precision P0^-1 + sum beta k k^T, mean by a linear solve."""
    c = noise_case(seed=62, T=12, dk=3, dv=2)
    T, dk = c["q"].shape
    dv = c["v"].shape[1]
    g = np.random.default_rng(62)
    P0 = []
    for i in range(dv):
        X = g.standard_normal((dk, dk))
        P0.append(X @ X.T + dk * np.eye(dk))
    P0 = np.stack(P0)
    ex = oracle.kdn_exact_head(c["q"], c["k"], c["v"], c["beta"], np.ones(T), np.zeros(T), P0=P0,
                               mu0=c["mu0"], lib=lib)
    for i in range(dv):
        Lam = np.linalg.inv(P0[i]) + sum(c["beta"][t, i] * np.outer(c["k"][t], c["k"][t]) for t in range(T))
        rhs = np.linalg.inv(P0[i]) @ c["mu0"][:, i] + sum(c["beta"][t, i] * c["v"][t, i] * c["k"][t]
                                                           for t in range(T))
        _close(ex["mu_T"][:, i], np.linalg.solve(Lam, rhs), rtol=1e-9, what="regression mean")
        _close(ex["P_T"][i], np.linalg.inv(Lam), rtol=1e-9, what="regression covariance")


def pin_exact_covariance_valid(lib):
    """Every final covariance is symmetric positive definite, and no larger
    than the prediction alone would give (observations only add information)."""
    c = noise_case(seed=63, T=30, dk=5, dv=2)
    ex = oracle.kdn_exact_head(c["q"], c["k"], c["v"], c["beta"], c["a"], c["p"], lib=lib)
    none = oracle.kdn_exact_head(c["q"], c["k"], c["v"], np.full_like(c["beta"], 1e-300), c["a"],
                                 c["p"], lib=lib)
    for i in range(2):
        P = ex["P_T"][i]
        _close(P, P.T, rtol=1e-12, what="symmetric")
        assert np.all(np.linalg.eigvalsh(P) > 0)
        assert np.all(np.linalg.eigvalsh(none["P_T"][i] - P) > -1e-12)


EXACT_PINS = [pin_exact_axis_keys_equal_diagonal, pin_exact_static_regression, pin_exact_covariance_valid]


NOISE_PINS = [pin_noise_equals_isotropic_single_entry, pin_noise_mobius, pin_noise_mean_field_step,
              pin_noise_residual_write]


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_prior_start, pin_bwd_readout_only,
            pin_bwd_empty_sequence, pin_bwd_scale_bounds]
ALL_PINS = DIAG_PINS + ISO_PINS + BWD_PINS + NOISE_PINS + M_PINS + EXACT_PINS

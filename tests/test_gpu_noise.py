"""Diagonal KDN with process noise: HIP path vs the fp64 oracle, element by element.

Tolerance as for the diagonal scan: |o - o_ref| <= 1e-4 * sum_j |q_j mu_ref|,
precisions elementwise relative 1e-4, means 1e-4 * max(|mu_ref|, rms(mu_ref)).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def _run(kdn, inp, st=None):
    x = gu.upload_diag(inp)
    a, p = gu.dev_tensor(inp["a"]), gu.dev_tensor(inp["p"])
    lam0 = None if st is None else gu.dev_tensor(st["I0"])
    mu0 = None if st is None else gu.dev_tensor(st["mu0"])
    res = kdn.kdn_diag_noise_scan_fwd(x["q"], x["k"], x["v"], x["beta"], a, p, lambda0=lam0, mu0=mu0)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in res]


def _compare(inp, res, heads, st=None, what=""):
    o, lam, mu = res
    f = lambda n: None if st is None else st[n].astype(np.float64)
    ref = oracle.diag_noise_scan(inp, heads=heads, lam0=f("I0"), mu0=f("mu0"))
    for (b, h) in heads:
        r = ref[(b, h)]
        gu.check_o(o[b, h], r, f"{what} o[{b},{h}]")
        gu.check_rel(lam[b, h], r["I_T"], f"{what} lambda_T[{b},{h}]")
        gu.check_state(mu[b, h], r["mu_T"], f"{what} mu_T[{b},{h}]")


SMALL = [
    (1, 2, 64, 16, 16, "f32"),
    (2, 3, 37, 32, 64, "bf16"),
    (1, 2, 100, 128, 128, "bf16"),
    (1, 1, 1, 64, 16, "f32"),
    (2, 2, 33, 16, 128, "f32"),
    (1, 3, 300, 128, 32, "bf16"),
]


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_noise_small(kdn, shape, with_state):
    B, H, T, dk, dv, dt = shape
    spec = gu.diag_spec(B, H, T, dk, dv, dt, seed=61 + T)
    inp = synth.noise_inputs(spec)
    st = synth.state_inputs(spec) if with_state else None
    _compare(inp, _run(kdn, inp, st), _heads(B, H), st, what=str(shape))


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_noise_head_sizes(kdn, dk, dv):
    spec = gu.diag_spec(1, 2, 40, dk, dv, "bf16", seed=71)
    inp = synth.noise_inputs(spec)
    _compare(inp, _run(kdn, inp), _heads(1, 2), what=f"{dk}x{dv}")


def test_noise_empty_sequence(kdn):
    spec = gu.diag_spec(1, 2, 0, 32, 16, "f32", seed=3)
    inp = synth.noise_inputs(spec)
    st = synth.state_inputs(spec)
    o, lam, mu = _run(kdn, inp, st)
    assert o.size == 0
    assert np.array_equal(lam, st["I0"]) and np.array_equal(mu, st["mu0"])


def test_noise_full_size_sampled(kdn):
    """The process-noise workload at full size (B8 H16 T2048 d128 bf16) in
    the launch configuration the benchmark times; sampled heads."""
    spec = synth.workload("noise_b8h16t2048d128_bf16")
    inp = synth.noise_inputs(spec)
    res = _run(kdn, inp)
    _compare(inp, res, [(0, 0), (4, 9), (7, 15)], what="full")

"""Gradient of the diagonal scan: HIP path vs the fp64 oracle, element by element.

The oracle differentiates the printed direct-mu recurrence entry by entry; the
HIP path runs the adjoint of the information form in scaled frames.  Both see
the same seeded inputs (bf16 inputs decoded exactly).  Tolerance: for every
gradient element |g - g_ref| <= 1e-4 * scale_ref, where scale_ref is the
oracle's sum of the absolute values of all terms of that gradient, carried
through the adjoint recursion -- the natural error scale of a sum that may
cancel (it bounds |g_ref|).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

RTOL = 1e-4


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def _run(kdn, inp, gr, st=None):
    x = gu.upload_diag(inp)
    opt = lambda n, src: None if (src is None or n not in src) else gu.dev_tensor(src[n])
    g = kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], inp["I_prior"],
                              gu.dev_tensor(gr["d_o"]), I0=opt("I0", st), mu0=opt("mu0", st),
                              d_I_T=opt("d_I_T", gr), d_mu_T=opt("d_mu_T", gr))
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}


def _ref(inp, gr, heads, st=None):
    f = lambda n, src: None if (src is None or n not in src) else src[n].astype(np.float64)
    return oracle.diag_scan_bwd(inp, gr["d_o"], heads=heads, I0=f("I0", st), mu0=f("mu0", st),
                                dI_T=f("d_I_T", gr), dmu_T=f("d_mu_T", gr))


def _check(got, ref, scale, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - ref)
    bound = RTOL * np.asarray(scale) + 1e-30
    ratio = err / bound
    r = float(np.max(ratio)) if err.size else 0.0
    if r > 1.0:
        bad = np.argwhere(ratio > 1.0)
        raise AssertionError(f"{what}: max |err| / (1e-4 scale) = {r:.3f}; {len(bad)} of "
                             f"{ratio.size} elements out, first at {tuple(bad[0])}, last at "
                             f"{tuple(bad[-1])}")
    return r


def _compare(g, ref, heads, whole=False, what=""):
    """Per-head gradients; with whole (every head present), also dA and dI_prior."""
    worst = 0.0
    fails = []
    for (b, h) in heads:
        r = ref[(b, h)]
        for n in ("dq", "dk", "dv", "dbeta", "dd", "dI0", "dmu0"):
            if n in r:
                try:
                    worst = max(worst, _check(g[n][b, h], r[n], r["scale_" + n], f"{what} {n}[{b},{h}]"))
                except AssertionError as e:
                    fails.append(str(e))
    assert not fails, "\n".join(fails)
    if whole:
        H = g["dA"].shape[0]
        for h in range(H):
            hs = [bh for bh in heads if bh[1] == h]
            _check(g["dA"][h], sum(ref[x]["dA"] for x in hs), sum(ref[x]["scale_dA"] for x in hs),
                   f"{what} dA[{h}]")
        _check(g["dI_prior"][0], sum(ref[x]["dI_prior"] for x in heads),
               sum(ref[x]["scale_dI_prior"] for x in heads), f"{what} dI_prior")
    return worst


SMALL = [
    (1, 2, 37, 64, 16, "f32"),
    (1, 1, 50, 128, 128, "bf16"),
    (2, 2, 33, 64, 64, "bf16"),
    (1, 2, 16, 128, 32, "f32"),
    (1, 1, 1, 64, 64, "f32"),
    (2, 1, 100, 128, 64, "bf16"),
    (1, 3, 47, 128, 16, "bf16"),
]


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small(kdn, shape, with_state):
    B, H, T, dk, dv, dt = shape
    spec = gu.diag_spec(B, H, T, dk, dv, dt, seed=31 + T)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec, final_state=with_state)
    st = synth.state_inputs(spec) if with_state else None
    g = _run(kdn, inp, gr, st)
    assert ("dI0" in g) == with_state
    _compare(g, _ref(inp, gr, _heads(B, H), st), _heads(B, H), whole=True, what=str(shape))


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_bwd_head_sizes(kdn, dk, dv):
    spec = gu.diag_spec(1, 2, 21, dk, dv, "f32", seed=5)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec)
    st = synth.state_inputs(spec)
    g = _run(kdn, inp, gr, st)
    _compare(g, _ref(inp, gr, _heads(1, 2), st), _heads(1, 2), whole=True, what=f"{dk}x{dv}")


def test_bwd_frame_cuts(kdn):
    """Strong forgetting (A d up to ~16 per token) cuts scaled frames inside
    chunks; the adjoint must follow every cut."""
    spec = gu.diag_spec(1, 2, 70, 128, 64, "f32", seed=9)
    inp = synth.diag_inputs(spec)
    inp["d"] = (inp["d"] * 4.0).astype(np.float32)
    gr = synth.grad_inputs(spec)
    st = synth.state_inputs(spec)
    g = _run(kdn, inp, gr, st)
    _compare(g, _ref(inp, gr, _heads(1, 2), st), _heads(1, 2), whole=True, what="frames")


def test_bwd_empty_sequence(kdn):
    """T = 0: the gradients of the final state pass to the starting state."""
    spec = gu.diag_spec(1, 2, 0, 64, 32, "f32", seed=3)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec)
    st = synth.state_inputs(spec)
    g = _run(kdn, inp, gr, st)
    np.testing.assert_allclose(g["dI0"], gr["d_I_T"], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(g["dmu0"], gr["d_mu_T"], rtol=1e-6, atol=1e-7)
    assert np.all(g["dA"] == 0.0) and g["dq"].size == 0
    # without a starting state the final precision's gradient is I_prior's
    g2 = _run(kdn, inp, gr, None)
    assert abs(g2["dI_prior"][0] - gr["d_I_T"].astype(np.float64).sum()) <= 1e-4 * np.abs(gr["d_I_T"]).sum()


def test_bwd_deterministic(kdn):
    spec = gu.diag_spec(2, 2, 77, 128, 128, "bf16", seed=11)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec)
    a = _run(kdn, inp, gr)
    b = _run(kdn, inp, gr)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_bwd_long_sequence(kdn):
    spec = gu.diag_spec(1, 2, 1000, 128, 128, "bf16", seed=13)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec)
    g = _run(kdn, inp, gr)
    _compare(g, _ref(inp, gr, _heads(1, 2)), _heads(1, 2), whole=True, what="T=1000")


def test_bwd_full_size_sampled(kdn):
    """The gradient workload at full size (B8 H16 T2048 d128, bf16), in the
    launch configuration the benchmark times; sampled heads against the oracle."""
    spec = synth.workload("bwd_b8h16t2048d128_bf16")
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec, final_state=False)
    g = _run(kdn, inp, gr)
    heads = [(0, 0), (3, 7), (7, 15)]
    _compare(g, _ref(inp, gr, heads), heads, what="full")

"""Gradient of rows cut into segments, on the GPU, against the oracle.

Rows too few to fill the chip are cut into the forward plan's segments.
Each segment's checkpoint pass starts from the state the forward composites
carry in; the adjoint recurrence, linear in the adjoint, is composed over
each later segment during that pass and carried from the row's end
(associative composition, KLA summary, Metodologia 2), so every segment's
reverse pass starts from the adjoint flowing into its end.  The oracle
differentiates each row as one sequential recurrence (Palimpsa page,
Metodologia 1-2); gradients are compared element by element at the
tolerance of the other gradient tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402
from tests.test_gpu_bwd import _compare, _heads, _ref  # noqa: E402


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _run(kdn, inp, gr, st=None, segments=0):
    x = gu.upload_diag({**inp, "beta": inp["d"] if inp["beta"] is None else inp["beta"]})
    beta = None if inp["beta"] is None else x["beta"]
    opt = lambda n, src: None if (src is None or n not in src) else gu.dev_tensor(src[n])
    g = kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], beta, x["d"], x["A"], inp["I_prior"],
                              gu.dev_tensor(gr["d_o"]), I0=opt("I0", st), mu0=opt("mu0", st),
                              d_I_T=opt("d_I_T", gr), d_mu_T=opt("d_mu_T", gr), segments=segments)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}


CASES = [
    # (B, H, T, d_k, d_v, dtype, segments)
    (1, 2, 600, 64, 64, "f32", 3),
    (1, 1, 1000, 128, 128, "bf16", 4),
    (2, 1, 333, 128, 64, "bf16", 5),      # ragged last chunk
    (1, 2, 257, 64, 16, "f32", 17),       # one chunk per segment (clamped to 17 chunks)
    (1, 1, 512, 128, 32, "bf16", 2),
]


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_segmented_gradient(kdn, case, with_state):
    B, H, T, dk, dv, dt, S = case
    spec = gu.diag_spec(B, H, T, dk, dv, dt, seed=401 + T, I_prior=0.6)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec, final_state=with_state)
    st = synth.state_inputs(spec) if with_state else None
    assert kdn.kdn_diag_plan(B, H, T, dk, dv, segments=S)[1] > 1
    print(f"segmented bwd {case} state={with_state}", flush=True)
    g = _run(kdn, inp, gr, st, segments=S)
    _compare(g, _ref(inp, gr, _heads(B, H), st), _heads(B, H), whole=True, what=f"S={S} {case}")


def test_segmented_m_gating(kdn):
    """Palimpsa-M gating (beta = d), dbeta's share in dd, with segments."""
    spec = gu.diag_spec(1, 2, 700, 128, 64, "bf16", seed=451)
    inp = synth.diag_inputs(spec)
    inp["beta"] = None
    gr = synth.grad_inputs(spec)
    g = _run(kdn, inp, gr, segments=4)
    assert "dbeta" not in g
    _compare(g, _ref(inp, gr, _heads(1, 2)), _heads(1, 2), whole=True, what="M S=4")


def test_segments_agree_with_one(kdn):
    """The segmented gradient agrees with the unsegmented one to the oracle
    tolerance; both are deterministic."""
    spec = gu.diag_spec(1, 2, 800, 128, 128, "bf16", seed=452)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec)
    a = _run(kdn, inp, gr, segments=5)
    b = _run(kdn, inp, gr, segments=1)
    a2 = _run(kdn, inp, gr, segments=5)
    ref = _ref(inp, gr, _heads(1, 2))
    _compare(a, ref, _heads(1, 2), whole=True, what="S=5")
    _compare(b, ref, _heads(1, 2), whole=True, what="S=1")
    for n in a:
        assert np.array_equal(a[n], a2[n]), n


def test_long_workload_sampled(kdn):
    """The long-sequence gradient workload (B2 H16 T16384 d128 bf16) with the
    automatic plan the benchmark times (4 segments a row); two heads against
    the oracle."""
    spec = synth.workload("bwd_b2h16t16384d128_bf16")
    assert kdn.kdn_diag_plan(spec.B, spec.H, spec.T, spec.d_k, spec.d_v)[1] > 1
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec, final_state=False)
    print("long workload", flush=True)
    g = _run(kdn, inp, gr)
    heads = [(0, 0), (1, 15)]
    _compare(g, _ref(inp, gr, heads), heads, what="long")

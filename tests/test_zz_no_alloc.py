"""The no-allocation entry point against the workspace entry point.

kdn_diag_scan_fwd_noalloc runs the diagonal scan with the library's fixed
per-GPU scratch array instead of a caller-supplied workspace.  Two calls in a
row, the second on a smaller input (the scratch keeps the first call's
contents): where the plan is the same as the workspace entry's the results
must be identical bit for bit; where the long-sequence plan's composite
sub-segments had to be reduced to fit the scratch, they must agree to the
parity tolerance (1e-4 of sum_j |q_j mu_j| for o, relative for I, scaled for
mu), and match the oracle on sampled heads.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _both(kdn, x, I_prior=1.0):
    ref = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], I_prior)
    got = kdn.kdn_diag_scan_fwd_noalloc(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], I_prior)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_two_calls_second_smaller(kdn):
    # first call: the long-sequence shape (B2 H16 T16384 d128, automatic plan
    # with segment composites), larger than the scratch holds at the plain
    # plan's sub-segment count
    spec = synth.workload("diag_b2h16t16384d128_bf16")
    inp = synth.diag_inputs(spec)
    x = gu.upload_diag(inp)
    ref, got = _both(kdn, x)
    o_r, I_r, m_r = (t.cpu().numpy() for t in ref)
    o_g, I_g, m_g = (t.cpu().numpy() for t in got)
    assert np.all(np.isfinite(o_g))
    scale = np.abs(o_r).max()
    assert np.max(np.abs(o_g - o_r)) <= 1e-4 * scale
    gu.check_rel(I_g, I_r.astype(np.float64), "noalloc I_T")
    gu.check_state(m_g, m_r.astype(np.float64), "noalloc mu_T")
    gu.compare_diag(inp, got, [(0, 3), (1, 14)], what="noalloc long")
    del x, ref, got
    # second call, smaller (segments and composites, ragged tail): same plan,
    # so identical to the workspace entry bit for bit
    for shape in [(1, 2, 4100, 128, 128, "bf16"), (2, 3, 77, 64, 32, "f32")]:
        B, H, T, dk, dv, dt = shape
        inp = synth.diag_inputs(gu.diag_spec(B, H, T, dk, dv, dt, seed=97))
        ref, got = _both(kdn, gu.upload_diag(inp))
        for a, b, n in zip(ref, got, ("o", "I_T", "mu_T")):
            assert torch.equal(a, b), f"{shape} {n} differs from the workspace entry"
        gu.compare_diag(inp, got, [(b, h) for b in range(B) for h in range(H)], what=f"noalloc {shape}")

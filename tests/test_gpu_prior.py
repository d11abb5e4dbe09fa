"""Every path that takes I_prior, at prior precisions other than 1: HIP vs the oracle.

The prior enters the recurrence as (1 - alpha_t) I_prior (Palimpsa page,
Metodologia 2), as the default starting precision I_0 = I_prior, through the
carry of segment composites (I = I_prior + J), in the decode step, in the
packed variable-length batch and in the gradient (dI_prior).  Each is run at
I_prior = 0.37 and 4.2 and compared element by element with the oracle at the
tolerances of the other parity tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402
from tests.test_gpu_bwd import _compare as compare_grads, _ref as ref_grads, _run as run_grads  # noqa: E402

PRIORS = [0.37, 4.2]


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def _fwd(kdn, inp, S, I0=None, mu0=None, beta=True):
    x = gu.upload_diag({**inp, "beta": inp["beta"] if beta else inp["d"]})
    res = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"] if beta else None, x["d"], x["A"],
                                inp["I_prior"], I0=I0, mu0=mu0, segments=S)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("prior", PRIORS)
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("dv", [128, 32])
def test_forward_prior(kdn, prior, with_state, S, dv):
    """64-column block kernel (d_v = 128) and narrow-tile kernel (d_v = 32),
    one segment and three (composites + carry), default and given start."""
    B, H, T, dk = 2, 2, 203, 128
    spec = gu.diag_spec(B, H, T, dk, dv, "bf16", seed=9100 + dv, I_prior=prior)
    inp = synth.diag_inputs(spec)
    st = synth.state_inputs(spec) if with_state else None
    print(f"prior={prior} state={with_state} S={S} dv={dv}", flush=True)
    res = _fwd(kdn, inp, S, I0=gu.dev_tensor(st["I0"]) if st else None,
               mu0=gu.dev_tensor(st["mu0"]) if st else None)
    gu.compare_diag(inp, res, _heads(B, H), what=f"prior={prior} S={S} dv={dv}",
                    I0=st["I0"].astype(np.float64) if st else None,
                    mu0=st["mu0"].astype(np.float64) if st else None)


@pytest.mark.parametrize("prior", PRIORS)
def test_forward_prior_m_gating(kdn, prior):
    B, H, T, dk, dv = 1, 3, 150, 128, 128
    spec = gu.diag_spec(B, H, T, dk, dv, "bf16", seed=9200, I_prior=prior)
    inp = synth.diag_inputs(spec)
    inp["beta"] = None
    res = _fwd(kdn, {**inp, "beta": inp["d"]}, 2, beta=False)
    gu.compare_diag(inp, res, _heads(B, H), what=f"M gating prior={prior}")


@pytest.mark.parametrize("prior", PRIORS)
@pytest.mark.parametrize("dv", [128, 32])
def test_decode_prior(kdn, prior, dv):
    """A prefix scan, then one decode token, equals the oracle's scan."""
    B, H, T, dk = 3, 2, 41, 64
    spec = gu.diag_spec(B, H, T, dk, dv, "bf16", seed=9300 + dv, I_prior=prior)
    inp = synth.diag_inputs(spec)
    ref = oracle.diag_scan(inp)
    x = gu.upload_diag(inp, (0, T - 1))
    _, I, mu = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], prior)
    last = {n: gu.dev_tensor(np.ascontiguousarray(inp[n][:, :, T - 1])) for n in
            ("q", "k", "v", "beta", "d")}
    o = kdn.kdn_decode_step(last["q"], last["k"], last["v"], last["beta"], last["d"], x["A"], prior,
                            I, mu)
    torch.cuda.synchronize()
    o, I, mu = o.cpu().numpy(), I.cpu().numpy(), mu.cpu().numpy()
    for b, h in _heads(B, H):
        r = ref[(b, h)]
        gu.check_o(o[b, h], {"o": r["o"][-1], "s": r["s"][-1]}, f"decode o[{b},{h}] prior={prior}")
        gu.check_rel(I[b, h], r["I_T"], f"decode I prior={prior}")
        gu.check_state(mu[b, h], r["mu_T"], f"decode mu prior={prior}")


@pytest.mark.parametrize("prior", PRIORS)
def test_varlen_prior(kdn, prior):
    spec = synth.VarlenSpec("varlen_prior", 3, 7, 500, 128, 128, "bf16", 9400, I_prior=prior)
    inp = synth.varlen_inputs(spec)
    x = {n: gu.dev_tensor(inp[n][0]) for n in ("q", "k", "v", "beta", "d")}
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    o, I_T, mu_T = kdn.kdn_diag_scan_varlen_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"],
                                                gu.dev_tensor(inp["A"]), prior, cu)
    torch.cuda.synchronize()
    ref = oracle.diag_scan_varlen(inp, inp["cu_seqlens"])
    o, I_T, mu_T = o.cpu().numpy(), I_T.cpu().numpy(), mu_T.cpu().numpy()
    cu_l = [int(c) for c in inp["cu_seqlens"]]
    for (s, h), r in ref.items():
        gu.check_o(o[h, cu_l[s]:cu_l[s + 1]], r, f"varlen o seq {s} head {h} prior={prior}")
        gu.check_rel(I_T[s, h], r["I_T"], f"varlen I_T seq {s} head {h}")
        gu.check_state(mu_T[s, h], r["mu_T"], f"varlen mu_T seq {s} head {h}")


@pytest.mark.parametrize("prior", PRIORS)
@pytest.mark.parametrize("with_state", [False, True])
def test_backward_prior(kdn, prior, with_state):
    """Gradients of every input, dI_prior included, at a prior other than 1."""
    B, H, T, dk, dv = 2, 2, 45, 128, 64
    spec = gu.diag_spec(B, H, T, dk, dv, "bf16", seed=9500, I_prior=prior)
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec, final_state=True)
    st = synth.state_inputs(spec) if with_state else None
    g = run_grads(kdn, inp, gr, st)
    compare_grads(g, ref_grads(inp, gr, _heads(B, H), st), _heads(B, H), whole=True,
                  what=f"prior={prior} state={with_state}")

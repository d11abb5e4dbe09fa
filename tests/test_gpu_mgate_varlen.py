"""Palimpsa-M gating (beta_t = d_t) and the packed variable-length batch:
HIP path vs the fp64 oracle, element by element.

Tolerances as for the diagonal scan (forward: 1e-4 of sum_j |q_j mu_ref| for
o, relative for precisions, 1e-4 of max(|mu|, rms mu) for means; gradients:
1e-4 of the oracle's absolute-term scale).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402
from tests.test_gpu_bwd import _check as check_grad  # noqa: E402


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def _m_inputs(spec):
    inp = synth.diag_inputs(spec)
    inp["beta"] = None
    return inp


def _fwd(kdn, inp, S=0):
    x = gu.upload_diag({**inp, "beta": inp["d"]})   # beta slot unused below
    res = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], None, x["d"], x["A"], inp["I_prior"],
                                segments=S)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("shape", [(1, 2, 64, 16, 16, "f32"), (2, 3, 37, 32, 64, "bf16"),
                                   (1, 2, 300, 128, 128, "bf16"), (1, 1, 129, 64, 32, "f32")],
                         ids=lambda s: "x".join(map(str, s)))
def test_m_gating_forward(kdn, shape, S):
    B, H, T, dk, dv, dt = shape
    inp = _m_inputs(gu.diag_spec(B, H, T, dk, dv, dt, seed=81 + T))
    gu.compare_diag(inp, _fwd(kdn, inp, S), _heads(B, H), what=f"M S={S}")


@pytest.mark.parametrize("dk,dv", [(16, 128), (128, 16), (32, 32), (64, 128)], ids=lambda d: str(d))
def test_m_gating_composite_shapes(kdn, dk, dv):
    """Palimpsa-M gating through the bf16 composite pass at tile shapes
    where its J and X waves differ in count (two segments, T = 601)."""
    inp = _m_inputs(gu.diag_spec(1, 2, 601, dk, dv, "bf16", seed=8100 + dk + dv))
    print(f"M composite dk={dk} dv={dv}", flush=True)
    gu.compare_diag(inp, _fwd(kdn, inp, 2), _heads(1, 2), what=f"M composite dk={dk} dv={dv}")


def test_m_gating_forward_full_size_sampled(kdn):
    spec = synth.workload("diagm_b8h16t2048d128_bf16")
    inp = _m_inputs(spec)
    gu.compare_diag(inp, _fwd(kdn, inp), [(0, 0), (5, 11), (7, 15)], what="M full")


def test_m_gating_decode(kdn):
    """One decode token after a prefix, both under Palimpsa-M gating."""
    B, H, P, dk, dv = 2, 3, 40, 64, 32
    spec = gu.diag_spec(B, H, P + 1, dk, dv, "bf16", seed=83)
    inp = _m_inputs(spec)
    pre = {**inp, "q": inp["q"][:, :, :P], "k": inp["k"][:, :, :P], "v": inp["v"][:, :, :P],
           "d": inp["d"][:, :, :P]}
    _, I, mu = _fwd(kdn, pre)
    tok = lambda n: gu.dev_tensor(np.ascontiguousarray(inp[n][:, :, P]))
    o = kdn.kdn_decode_step(tok("q"), tok("k"), tok("v"), None, tok("d"), gu.dev_tensor(inp["A"]),
                            inp["I_prior"], I, mu)
    torch.cuda.synchronize()
    ref = oracle.diag_scan(inp, heads=_heads(B, H))
    o = o.cpu().numpy()
    for (b, h) in _heads(B, H):
        r = ref[(b, h)]
        gu.check_o(o[b, h][None], {"o": r["o"][P][None], "s": r["s"][P][None]}, f"decode o[{b},{h}]")
        gu.check_rel(I[b, h].cpu().numpy(), r["I_T"], f"decode I[{b},{h}]")
        gu.check_state(mu[b, h].cpu().numpy(), r["mu_T"], f"decode mu[{b},{h}]")


@pytest.mark.parametrize("shape", [(1, 2, 37, 64, 16, "f32"), (1, 1, 50, 128, 128, "bf16"),
                                   (2, 2, 33, 64, 64, "bf16"), (1, 2, 21, 128, 32, "f32")],
                         ids=lambda s: "x".join(map(str, s)))
def test_m_gating_backward(kdn, shape):
    B, H, T, dk, dv, dt = shape
    spec = gu.diag_spec(B, H, T, dk, dv, dt, seed=91 + T)
    inp = _m_inputs(spec)
    gr = synth.grad_inputs(spec)
    x = gu.upload_diag({**inp, "beta": inp["d"]})
    g = kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], None, x["d"], x["A"], inp["I_prior"],
                              gu.dev_tensor(gr["d_o"]), d_I_T=gu.dev_tensor(gr["d_I_T"]),
                              d_mu_T=gu.dev_tensor(gr["d_mu_T"]))
    torch.cuda.synchronize()
    assert "dbeta" not in g
    g = {n: t.cpu().numpy() for n, t in g.items()}
    ref = oracle.diag_scan_bwd(inp, gr["d_o"], heads=_heads(B, H),
                               dI_T=gr["d_I_T"].astype(np.float64), dmu_T=gr["d_mu_T"].astype(np.float64))
    for (b, h) in _heads(B, H):
        r = ref[(b, h)]
        for n in ("dq", "dk", "dv", "dd"):
            check_grad(g[n][b, h], r[n], r["scale_" + n], f"M bwd {n}[{b},{h}]")
    for h in range(H):
        hs = [(b, h) for b in range(B)]
        check_grad(g["dA"][h], sum(ref[x]["dA"] for x in hs), sum(ref[x]["scale_dA"] for x in hs),
                   f"M bwd dA[{h}]")


def _varlen(kdn, inp, st=None):
    x = gu.upload_diag({**inp, "beta": inp["d"] if inp["beta"] is None else inp["beta"]})
    sq = lambda t: t[0]   # [1,H,T,.] -> [H,T,.]
    beta = None if inp["beta"] is None else sq(x["beta"])
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    I0 = None if st is None else gu.dev_tensor(st["I0"])
    mu0 = None if st is None else gu.dev_tensor(st["mu0"])
    res = kdn.kdn_diag_scan_varlen_fwd(sq(x["q"]), sq(x["k"]), sq(x["v"]), beta, sq(x["d"]), x["A"],
                                       inp["I_prior"], cu, I0=I0, mu0=mu0)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in res]


def _compare_varlen(inp, res, st=None, runs=None, what=""):
    o, I_T, mu_T = res
    f = lambda n: None if st is None else st[n].astype(np.float64)
    ref = oracle.diag_scan_varlen(inp, inp["cu_seqlens"], I0=f("I0"), mu0=f("mu0"))
    cu = inp["cu_seqlens"]
    for (s, h) in (runs or sorted(ref)):
        r = ref[(s, h)]
        t0, t1 = int(cu[s]), int(cu[s + 1])
        if t1 > t0:
            gu.check_o(o[h, t0:t1], r, f"{what} o[seq {s}, head {h}]")
        gu.check_rel(I_T[s, h], r["I_T"], f"{what} I_T[{s},{h}]")
        gu.check_state(mu_T[s, h], r["mu_T"], f"{what} mu_T[{s},{h}]")


LENGTHS = [0, 1, 15, 16, 17, 40, 0, 100, 33]


@pytest.mark.parametrize("m_gating", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("dims", [(64, 64, "bf16"), (128, 128, "bf16"), (16, 32, "f32")],
                         ids=lambda s: "x".join(map(str, s)))
def test_varlen(kdn, dims, with_state, m_gating):
    dk, dv, dt = dims
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)
    spec = gu.diag_spec(1, 2, int(cu[-1]), dk, dv, dt, seed=95)
    inp = synth.diag_inputs(spec)
    inp["cu_seqlens"] = cu
    if m_gating:
        inp["beta"] = None
    st = None
    if with_state:
        st = synth.state_inputs(spec.with_(B=len(LENGTHS)))
    _compare_varlen(inp, _varlen(kdn, inp, st), st, what=f"varlen {dims}")


def test_varlen_workload_sampled(kdn):
    """The packed workload the benchmark times (64 sequences x 16 heads,
    16384 packed tokens, d 128, bf16); sampled (sequence, head) runs."""
    spec = synth.workload("varlen_n64h16t16384d128_bf16")
    inp = synth.varlen_inputs(spec)
    lens = np.diff(inp["cu_seqlens"])
    longest = int(np.argmax(lens))
    runs = [(0, 0), (longest, 3), (63, 15), (31, 8)]
    _compare_varlen(inp, _varlen(kdn, inp), runs=runs, what="varlen full")

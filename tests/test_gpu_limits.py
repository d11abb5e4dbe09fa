"""Large grids: element-wise passes whose element count exceeds what one
sweep of their capped grid covers (65536 workgroups x 256 threads =
16,777,216 elements), so the grid-stride loop takes a second turn.  The
elements of that second turn are the ones checked against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

ONE_SWEEP = 65536 * 256


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def test_diag_many_heads(kdn):
    """16384 heads x 1025 chunks of frame scalars (more than one sweep): 16
    seeded heads tiled 1024 times over the head axis, so every head has an
    oracle result; heads 16368..16383 come from the second sweep."""
    spec = gu.diag_spec(1, 16, 16400, 16, 16, "bf16", seed=23)
    inp = synth.diag_inputs(spec)
    rep = 1024
    H = 16 * rep
    assert H * ((spec.T + 15) // 16) > ONE_SWEEP
    x = gu.upload_diag(inp)
    big = {n: x[n].repeat(1, rep, *([1] * (x[n].dim() - 2))).contiguous()
           for n in ("q", "k", "v", "beta", "d")}
    A = x["A"].repeat(rep).contiguous()
    del x
    o, I_T, mu_T = kdn.kdn_diag_scan_fwd(big["q"], big["k"], big["v"], big["beta"], big["d"], A, 1.0)
    torch.cuda.synchronize()
    del big
    picks = [0, 5003, 16368, 16375, 16383]
    ref = oracle.diag_scan(inp, heads=sorted({(0, h % 16) for h in picks}))
    for h in picks:
        r = ref[(0, h % 16)]
        gu.check_o(o[0, h].cpu().numpy(), r, f"o[0,{h}]")
        gu.check_rel(I_T[0, h].cpu().numpy(), r["I_T"], f"I_T[0,{h}]")
        gu.check_state(mu_T[0, h].cpu().numpy(), r["mu_T"], f"mu_T[0,{h}]")


def _big_state(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    I0 = 0.2 + 3.0 * torch.rand(shape, generator=g, device="cuda")
    mu0 = torch.randn(shape, generator=g, device="cuda")
    return I0, mu0


def test_zero_length_big_state(kdn):
    """T = 0 over 33.5 M state entries: the final state is the starting state,
    bit for bit, in the diagonal scan and in the process-noise scan."""
    B, H, dk, dv = 128, 16, 128, 128
    assert B * H * dk * dv > ONE_SWEEP
    I0, mu0 = _big_state((B, H, dk, dv), 5)
    z = torch.zeros((B, H, 0, dk), dtype=torch.bfloat16, device="cuda")
    zd = torch.zeros((B, H, 0), dtype=torch.bfloat16, device="cuda")
    A = torch.ones(H, device="cuda")
    o, I_T, mu_T = kdn.kdn_diag_scan_fwd(z, z, z, z, zd, A, 1.0, I0=I0, mu0=mu0)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(I_T, I0) and torch.equal(mu_T, mu0)
    zf = torch.zeros((B, H, 0), device="cuda")
    o, lam_T, mu_T = kdn.kdn_diag_noise_scan_fwd(z, z, z, z, zf, zf, lambda0=I0, mu0=mu0)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(lam_T, I0) and torch.equal(mu_T, mu0)


def test_bwd_column_tile_sums_many_rows(kdn):
    """Gradient at B17 H16 T2048 d128 bf16: the column-tile sums of dq and dk
    cover 17.8 M float4s; heads 256..271 come from the second sweep."""
    spec = gu.diag_spec(17, 16, 2048, 128, 128, "bf16", seed=29)
    assert spec.B * spec.H * spec.T * spec.d_k // 4 > ONE_SWEEP
    inp = synth.diag_inputs(spec)
    gr = synth.grad_inputs(spec, final_state=False)
    x = gu.upload_diag(inp)
    g = kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], inp["I_prior"],
                              gu.dev_tensor(gr["d_o"]))
    torch.cuda.synchronize()
    heads = [(0, 3), (16, 0), (16, 15)]
    ref = oracle.diag_scan_bwd(inp, gr["d_o"], heads=heads)
    for (b, h) in heads:
        r = ref[(b, h)]
        for n in ("dq", "dk"):
            got = g[n][b, h].cpu().numpy().astype(np.float64)
            err = np.abs(got - r[n])
            bound = 1e-4 * np.asarray(r["scale_" + n]) + 1e-30
            worst = float(np.max(err / bound))
            assert worst <= 1.0, f"{n}[{b},{h}]: max |err| / (1e-4 scale) = {worst:.3f}"

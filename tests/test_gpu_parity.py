"""HIP path vs the CPU oracle, element by element, on seeded inputs.

Tolerance: the acceptance bound of 1e-4 relative with fp32 state, read as
|o - o_ref| <= 1e-4 * sum_j |q_j mu_ref[j,i]| for the read-out (the natural
error scale of a sum that may cancel), elementwise relative for precisions,
and 1e-4 * max(|mu_ref|, rms(mu_ref)) for the signed mean state.
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


def _all_heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def _run_diag(kdn, x, I0=None, mu0=None, S=0):
    res = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], 1.0,
                                I0=I0, mu0=mu0, segments=S)
    torch.cuda.synchronize()
    return res


SMALL = [
    (1, 2, 64, 16, 16, "f32"),
    (2, 3, 37, 32, 64, "bf16"),
    (1, 2, 100, 128, 128, "bf16"),
    (1, 1, 1, 64, 16, "f32"),
    (2, 2, 33, 16, 128, "f32"),
    (1, 3, 300, 128, 32, "bf16"),
    (1, 2, 50, 128, 64, "f32"),
    (3, 1, 129, 64, 64, "bf16"),
]


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_diag_small(kdn, shape, S):
    B, H, T, dk, dv, dt = shape
    inp = synth.diag_inputs(gu.diag_spec(B, H, T, dk, dv, dt, seed=11))
    print(f"diag small {shape} S={S}", flush=True)
    res = _run_diag(kdn, gu.upload_diag(inp), S=S)
    gu.compare_diag(inp, res, _all_heads(B, H), what=f"{shape} S={S}")


def test_diag_tiny_workload(kdn):
    """The B1 H2 T64 d16 fp32 workload with A = 1 exactly as specified."""
    spec = synth.workload("diag_b1h2t64d16_f32")
    inp = synth.diag_inputs(spec)
    res = _run_diag(kdn, gu.upload_diag(inp))
    gu.compare_diag(inp, res, _all_heads(1, 2), what=spec.name)


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_diag_head_sizes(kdn, dk, dv):
    inp = synth.diag_inputs(gu.diag_spec(1, 2, 21, dk, dv, "f32", seed=dk * 1000 + dv))
    res = _run_diag(kdn, gu.upload_diag(inp))
    gu.compare_diag(inp, res, _all_heads(1, 2), what=f"dk={dk} dv={dv}")


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_diag_composite_head_sizes(kdn, dk, dv):
    """Two segments, so the first is a composite cut into several sub-segments:
    every (d_k, d_v) pairing of the composite pass's one-wave tiles, with a
    ragged final chunk (T = 601)."""
    dt = "bf16" if (dk + dv) % 64 == 0 else "f32"
    inp = synth.diag_inputs(gu.diag_spec(1, 2, 601, dk, dv, dt, seed=7000 + dk + dv))
    print(f"diag composite dk={dk} dv={dv} {dt}", flush=True)
    res = _run_diag(kdn, gu.upload_diag(inp), S=2)
    gu.compare_diag(inp, res, _all_heads(1, 2), what=f"composite dk={dk} dv={dv}")


@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_diag_composite_head_sizes_bf16(kdn, dk, dv):
    """bf16 inputs at every (d_k, d_v): the composite pass's J waves (tiles
    of at most 32 key rows x 128 value columns) and X waves (128 x 32) take
    different shapes and counts at each pairing; two segments, ragged final
    chunk (T = 601)."""
    inp = synth.diag_inputs(gu.diag_spec(1, 2, 601, dk, dv, "bf16", seed=7100 + dk + dv))
    print(f"diag composite bf16 dk={dk} dv={dv}", flush=True)
    res = _run_diag(kdn, gu.upload_diag(inp), S=2)
    gu.compare_diag(inp, res, _all_heads(1, 2), what=f"composite bf16 dk={dk} dv={dv}")


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("dv", [32, 128])
def test_diag_frame_restarts_inside_chunks(kdn, dv, S):
    """Fast decays: A = 6 gives about 5 nats of decay per token, so the scaled
    frame restarts two or three times inside every 16-token chunk (not only at
    chunk starts), in the 64-column block kernel (d_v = 128) and the narrow-tile
    kernel (d_v = 32), with a ragged last chunk and with composites (S = 2)."""
    inp = synth.diag_inputs(gu.diag_spec(1, 2, 203, 128, dv, "bf16", seed=8100 + dv))
    inp["A"] = np.full_like(inp["A"], 6.0)
    print(f"diag frame restarts dv={dv} S={S}", flush=True)
    res = _run_diag(kdn, gu.upload_diag(inp), S=S)
    gu.compare_diag(inp, res, _all_heads(1, 2), what=f"frame restarts dv={dv} S={S}")


@pytest.mark.parametrize("S", [1, 4])
def test_diag_initial_state(kdn, S):
    """Nonzero starting state (I0 != I_prior, mu0 != 0), both segmentings."""
    B, H, T, dk, dv = 2, 2, 90, 64, 128
    inp = synth.diag_inputs(gu.diag_spec(B, H, T, dk, dv, "bf16", seed=5))
    g = np.random.default_rng(3)
    I0 = (0.2 + 3.0 * g.random((B, H, dk, dv))).astype(np.float32)
    mu0 = g.standard_normal((B, H, dk, dv)).astype(np.float32)
    res = _run_diag(kdn, gu.upload_diag(inp), I0=gu.dev_tensor(I0), mu0=gu.dev_tensor(mu0), S=S)
    gu.compare_diag(inp, res, _all_heads(B, H), I0=I0.astype(np.float64),
                    mu0=mu0.astype(np.float64), what=f"initial state S={S}")


def test_diag_empty_and_zero_length(kdn):
    x = gu.upload_diag(synth.diag_inputs(gu.diag_spec(1, 2, 5, 16, 16, "f32")))
    # T = 0: the final state is the starting state
    g = np.random.default_rng(1)
    I0 = torch.from_numpy((1 + g.random((1, 2, 16, 16))).astype(np.float32)).cuda()
    mu0 = torch.from_numpy(g.standard_normal((1, 2, 16, 16)).astype(np.float32)).cuda()
    z = {n: t[:, :, :0].contiguous() for n, t in x.items() if n != "A"}
    o, I_T, mu_T = kdn.kdn_diag_scan_fwd(z["q"], z["k"], z["v"], z["beta"], z["d"], x["A"], 1.0,
                                         I0=I0, mu0=mu0)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(I_T, I0) and torch.equal(mu_T, mu0)
    # B = 0: nothing to do, nothing touched
    e = {n: t[:0].contiguous() for n, t in x.items() if n != "A"}
    o, I_T, mu_T = kdn.kdn_diag_scan_fwd(e["q"], e["k"], e["v"], e["beta"], e["d"], x["A"], 1.0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and I_T.numel() == 0


def test_diag_deterministic(kdn):
    x = gu.upload_diag(synth.diag_inputs(gu.diag_spec(2, 2, 200, 128, 128, "bf16", seed=9)))
    r1 = [t.clone() for t in _run_diag(kdn, x, S=3)]
    r2 = _run_diag(kdn, x, S=3)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b), "two runs differ bitwise"


def test_diag_segmentings_agree(kdn):
    """Results do not depend on how the sequence is cut (up to rounding)."""
    inp = synth.diag_inputs(gu.diag_spec(1, 2, 700, 64, 64, "bf16", seed=13))
    x = gu.upload_diag(inp)
    ref = oracle.diag_scan(inp)
    for S in (1, 2, 5, 16):
        gu.compare_diag(inp, _run_diag(kdn, x, S=S), _all_heads(1, 2), ref=ref, what=f"S={S}")


def test_diag_chaining_in_place(kdn):
    """scan(T1) then scan(T2) from its state, written in place (I_T = I0),
    equals one scan over T1 + T2."""
    B, H, T, cut = 1, 2, 80, 33
    inp = synth.diag_inputs(gu.diag_spec(B, H, T, 32, 32, "bf16", seed=17))
    ref = oracle.diag_scan(inp)
    x1 = gu.upload_diag(inp, (0, cut))
    x2 = gu.upload_diag(inp, (cut, T))
    o1, I, mu = _run_diag(kdn, x1)
    o2, _, _ = kdn.kdn_diag_scan_fwd(x2["q"], x2["k"], x2["v"], x2["beta"], x2["d"], x2["A"], 1.0,
                                     I0=I, mu0=mu, I_T=I, mu_T=mu)
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=2)
    gu.compare_diag(inp, (o, I, mu), _all_heads(B, H), ref=ref, what="chained")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_matches_oracle(kdn, dt):
    """Decode after a scan equals the scan's next token (P-6 on the GPU)."""
    B, H, T, dk, dv = 3, 2, 40, 64, 128
    inp = synth.diag_inputs(gu.diag_spec(B, H, T, dk, dv, dt, seed=23))
    ref = oracle.diag_scan(inp)
    x = gu.upload_diag(inp, (0, T - 1))
    _, I, mu = _run_diag(kdn, x)
    last = {n: gu.dev_tensor(np.ascontiguousarray(inp[n][:, :, T - 1])) for n in
            ("q", "k", "v", "beta", "d")}
    o = kdn.kdn_decode_step(last["q"], last["k"], last["v"], last["beta"], last["d"], x["A"], 1.0,
                            I, mu)
    torch.cuda.synchronize()
    o, I, mu = o.cpu().numpy(), I.cpu().numpy(), mu.cpu().numpy()
    for b, h in _all_heads(B, H):
        r = ref[(b, h)]
        gu.check_o(o[b, h], {"o": r["o"][-1], "s": r["s"][-1]}, f"decode o[{b},{h}]")
        gu.check_rel(I[b, h], r["I_T"], "decode I")
        gu.check_state(mu[b, h], r["mu_T"], "decode mu")


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (128, 16), (32, 64), (128, 128)])
def test_decode_head_sizes(kdn, dk, dv):
    B, H = 2, 3
    spec = gu.diag_spec(B, H, 1, dk, dv, "f32", seed=dk + dv)
    inp = synth.diag_inputs(spec)
    g = np.random.default_rng(dk * dv)
    I0 = (0.5 + g.random((B, H, dk, dv))).astype(np.float32)
    mu0 = g.standard_normal((B, H, dk, dv)).astype(np.float32)
    ref = oracle.diag_scan(inp, I0=I0.astype(np.float64), mu0=mu0.astype(np.float64))
    one = {n: gu.dev_tensor(np.ascontiguousarray(inp[n][:, :, 0])) for n in
           ("q", "k", "v", "beta", "d")}
    I, mu = gu.dev_tensor(I0), gu.dev_tensor(mu0)
    o = kdn.kdn_decode_step(one["q"], one["k"], one["v"], one["beta"], one["d"],
                            gu.dev_tensor(inp["A"]), 1.0, I, mu)
    torch.cuda.synchronize()
    o, I, mu = o.cpu().numpy(), I.cpu().numpy(), mu.cpu().numpy()
    for b, h in _all_heads(B, H):
        r = ref[(b, h)]
        gu.check_o(o[b, h], {"o": r["o"][0], "s": r["s"][0]}, "decode o")
        gu.check_rel(I[b, h], r["I_T"], "decode I")
        gu.check_state(mu[b, h], r["mu_T"], "decode mu")


# ---------------------------------------------------------------------------
# isotropic path
# ---------------------------------------------------------------------------

ISO_SMALL = [(1, 2, 100, 16, 16), (2, 3, 5000, 64, 64), (1, 1, 4097, 32, 128), (1, 2, 257, 128, 64)]


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("shape", ISO_SMALL, ids=lambda s: "x".join(map(str, s)))
def test_iso_small(kdn, shape, S):
    B, H, T, dk, dv = shape
    spec = synth.IsoSpec("iso_test", B, H, T, dk, dv, 31)
    inp = synth.iso_inputs(spec)
    x = gu.upload_iso(inp)
    print(f"iso small {shape} S={S}", flush=True)
    lam, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"],
                                                 x["q"], x["k"], x["v"], segments=S)
    torch.cuda.synchronize()
    ref = oracle.iso_scan(inp)
    lam, o, mu_T = lam.cpu().numpy(), o.cpu().numpy(), mu_T.cpu().numpy()
    for b, h in _all_heads(B, H):
        r = ref[(b, h)]
        gu.check_rel(lam[b, h], r["lambda"], f"lambda[{b},{h}]")
        gu.check_o(o[b, h], r, f"iso o[{b},{h}]")
        gu.check_state(mu_T[b, h], r["mu_T"], f"iso mu_T[{b},{h}]")


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
def test_iso_head_sizes(kdn, dk, dv, S):
    """Every (d_k, d_v) pairing of the one-wave kernel: row and column tile
    interleaves, 1-4 column tiles per head, ragged last chunk (T = 45)."""
    spec = synth.IsoSpec("iso_sizes", 1, 2, 45, dk, dv, dk * 1000 + dv)
    inp = synth.iso_inputs(spec)
    x = gu.upload_iso(inp)
    print(f"iso head sizes dk={dk} dv={dv} S={S}", flush=True)
    _, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"],
                                               x["q"], x["k"], x["v"], segments=S)
    torch.cuda.synchronize()
    ref = oracle.iso_scan(inp)
    o, mu_T = o.cpu().numpy(), mu_T.cpu().numpy()
    for b, h in _all_heads(1, 2):
        r = ref[(b, h)]
        gu.check_o(o[b, h], r, f"iso o[{b},{h}] dk={dk} dv={dv}")
        gu.check_state(mu_T[b, h], r["mu_T"], f"iso mu_T[{b},{h}] dk={dk} dv={dv}")


@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 64])
def test_iso_short_sequences(kdn, T, S):
    """Chunks of one token, a single ragged chunk, exact chunk multiples, and
    more segments requested than there are chunks (the plan clamps)."""
    spec = synth.IsoSpec("iso_short", 2, 2, T, 64, 64, 4000 + T)
    inp = synth.iso_inputs(spec)
    x = gu.upload_iso(inp)
    print(f"iso short T={T} S={S}", flush=True)
    _, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"],
                                               x["q"], x["k"], x["v"], segments=S)
    torch.cuda.synchronize()
    ref = oracle.iso_scan(inp)
    o, mu_T = o.cpu().numpy(), mu_T.cpu().numpy()
    for b, h in _all_heads(2, 2):
        r = ref[(b, h)]
        gu.check_o(o[b, h], r, f"iso o[{b},{h}] T={T} S={S}")
        gu.check_state(mu_T[b, h], r["mu_T"], f"iso mu_T[{b},{h}] T={T} S={S}")


@pytest.mark.parametrize("S", [1, 3])
def test_iso_initial_state(kdn, S):
    """A nonzero starting mean (mu0) and precision (lambda0), both segmentings:
    the starting mean reaches the first segment through the carry pass."""
    B, H, T, dk, dv = 2, 2, 300, 64, 128
    spec = synth.IsoSpec("iso_state", B, H, T, dk, dv, 51)
    inp = synth.iso_inputs(spec)
    g = np.random.default_rng(52)
    inp["lambda0"] = (0.2 + 3.0 * g.random((B, H))).astype(np.float32)
    mu0 = g.standard_normal((B, H, dk, dv)).astype(np.float32)
    x = gu.upload_iso(inp)
    print(f"iso initial state S={S}", flush=True)
    _, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"],
                                               x["q"], x["k"], x["v"], mu0=gu.dev_tensor(mu0),
                                               segments=S)
    torch.cuda.synchronize()
    ref = oracle.iso_scan(inp, mu0=mu0)
    o, mu_T = o.cpu().numpy(), mu_T.cpu().numpy()
    for b, h in _all_heads(B, H):
        r = ref[(b, h)]
        gu.check_o(o[b, h], r, f"iso o[{b},{h}] S={S}")
        gu.check_state(mu_T[b, h], r["mu_T"], f"iso mu_T[{b},{h}] S={S}")


@pytest.mark.parametrize("with_mean", [False, True])
def test_mobius_long_sequence(kdn, with_mean):
    """T = 2^20 + 37: 257 Mobius blocks per head, so the carry pass walks
    five steps of 64 block composites (the last one ragged) and the last
    block is ragged too.  lambda elementwise against the oracle's sequential
    fp64 filter; with the mean path also o and mu_T (automatic segments)."""
    B, H, T = 1, 2, 2 ** 20 + 37
    dk = dv = 16
    spec = synth.IsoSpec("iso_long", B, H, T, dk, dv, 2020)
    inp = synth.iso_inputs(spec, with_mean=with_mean)
    x = gu.upload_iso(inp)
    print(f"mobius long T={T} mean={with_mean}", flush=True)
    if with_mean:
        lam, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"],
                                                     x["q"], x["k"], x["v"])
    else:
        lam, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"])
    torch.cuda.synchronize()
    ref = oracle.iso_scan(inp, with_mean=with_mean)
    lam = lam.cpu().numpy()
    for b, h in _all_heads(B, H):
        r = ref[(b, h)]
        gu.check_rel(lam[b, h], r["lambda"], f"lambda[{b},{h}] T={T}")
        if with_mean:
            gu.check_o(o[b, h].cpu().numpy(), r, f"iso o[{b},{h}] T={T}")
            gu.check_state(mu_T[b, h].cpu().numpy(), r["mu_T"], f"iso mu_T[{b},{h}] T={T}")


def test_iso_chaining(kdn):
    """scan(T1) then scan(T2) started from its last precision and final mean
    equals one scan over T1 + T2."""
    B, H, T, cut, dk, dv = 1, 2, 200, 77, 32, 64
    spec = synth.IsoSpec("iso_chain", B, H, T, dk, dv, 61)
    inp = synth.iso_inputs(spec)
    ref = oracle.iso_scan(inp)
    part = lambda a, b: {n: (np.ascontiguousarray(v[:, :, a:b])
                             if isinstance(v, np.ndarray) and v.ndim >= 3 else v)
                         for n, v in inp.items()}
    x1 = gu.upload_iso(part(0, cut))
    lam1, o1, mu1 = kdn.kdn_mobius_precision_scan(x1["a"], x1["p"], x1["Lambda"], x1["lambda0"],
                                                  x1["q"], x1["k"], x1["v"])
    x2 = gu.upload_iso(part(cut, T))
    lam2, o2, mu2 = kdn.kdn_mobius_precision_scan(x2["a"], x2["p"], x2["Lambda"],
                                                  lam1[:, :, -1].contiguous(), x2["q"], x2["k"],
                                                  x2["v"], mu0=mu1)
    torch.cuda.synchronize()
    lam = torch.cat([lam1, lam2], dim=2).cpu().numpy()
    o = torch.cat([o1, o2], dim=2).cpu().numpy()
    mu2 = mu2.cpu().numpy()
    for b, h in _all_heads(B, H):
        r = ref[(b, h)]
        gu.check_rel(lam[b, h], r["lambda"], f"chained lambda[{b},{h}]")
        gu.check_o(o[b, h], r, f"chained iso o[{b},{h}]")
        gu.check_state(mu2[b, h], r["mu_T"], f"chained iso mu_T[{b},{h}]")


@pytest.mark.parametrize("T", [1, 15, 4096, 4097, 3 * 4096 + 5])
def test_iso_precision_only(kdn, T):
    spec = synth.IsoSpec("iso_prec", 2, 2, T, 64, 64, 37)
    inp = synth.iso_inputs(spec, with_mean=False)
    g = np.random.default_rng(T)
    inp["lambda0"] = (0.1 + 5 * g.random((2, 2))).astype(np.float32)
    x = gu.upload_iso(inp)
    lam, o, mu = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"])
    torch.cuda.synchronize()
    assert o is None and mu is None
    ref = oracle.iso_scan(inp, with_mean=False)
    lam = lam.cpu().numpy()
    for b, h in _all_heads(2, 2):
        gu.check_rel(lam[b, h], ref[(b, h)]["lambda"], f"lambda T={T}")


# ---------------------------------------------------------------------------
# full-size workloads, sampled heads (the launch configuration the bench times)
# ---------------------------------------------------------------------------

def _sample(B, H, n, seed):
    g = np.random.default_rng(seed)
    allh = _all_heads(B, H)
    idx = sorted(g.choice(len(allh), size=min(n, len(allh)), replace=False))
    return [allh[i] for i in idx]


def test_full_diag_b8h16t2048d128(kdn):
    spec = synth.workload("diag_b8h16t2048d128_bf16")
    inp = synth.diag_inputs(spec)
    res = _run_diag(kdn, gu.upload_diag(inp))
    gu.compare_diag(inp, res, _sample(8, 16, 12, 1), what=spec.name)


@pytest.mark.parametrize("S", [0, 1])
def test_full_diag_b2h16t16384d128(kdn, S):
    spec = synth.workload("diag_b2h16t16384d128_bf16")
    inp = synth.diag_inputs(spec)
    res = _run_diag(kdn, gu.upload_diag(inp), S=S)   # S = 0: the automatic plan the bench uses
    gu.compare_diag(inp, res, _sample(2, 16, 4, 2), what=f"{spec.name} S={S}")


def test_full_iso_b1h32t65536d64(kdn):
    spec = synth.workload("iso_b1h32t65536d64_f32")
    inp = synth.iso_inputs(spec)
    x = gu.upload_iso(inp)
    lam, o, mu_T = kdn.kdn_mobius_precision_scan(x["a"], x["p"], x["Lambda"], x["lambda0"],
                                                 x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    heads = _sample(1, 32, 4, 3)
    ref = oracle.iso_scan(inp, heads=heads)
    lam, o, mu_T = lam.cpu().numpy(), o.cpu().numpy(), mu_T.cpu().numpy()
    for b, h in heads:
        r = ref[(b, h)]
        gu.check_rel(lam[b, h], r["lambda"], "lambda")
        gu.check_o(o[b, h], r, f"iso o[{b},{h}]")
        gu.check_state(mu_T[b, h], r["mu_T"], "iso mu_T")


def test_full_decode_b256h16d128(kdn):
    """State built by 512 seeded tokens, then one decode token."""
    spec = synth.workload("decode_b256h16d128_bf16")
    inp = synth.diag_inputs(spec)
    P = spec.prefix
    x = gu.upload_diag(inp, (0, P))
    _, I, mu = _run_diag(kdn, x)
    last = {n: gu.dev_tensor(np.ascontiguousarray(inp[n][:, :, P])) for n in
            ("q", "k", "v", "beta", "d")}
    o = kdn.kdn_decode_step(last["q"], last["k"], last["v"], last["beta"], last["d"], x["A"],
                            spec.I_prior, I, mu)
    torch.cuda.synchronize()
    heads = _sample(256, 16, 16, 4)
    ref = oracle.diag_scan(inp, heads=heads)
    o, I, mu = o.cpu().numpy(), I.cpu().numpy(), mu.cpu().numpy()
    for b, h in heads:
        r = ref[(b, h)]
        gu.check_o(o[b, h], {"o": r["o"][-1], "s": r["s"][-1]}, f"decode o[{b},{h}]")
        gu.check_rel(I[b, h], r["I_T"], "decode I")
        gu.check_state(mu[b, h], r["mu_T"], "decode mu")

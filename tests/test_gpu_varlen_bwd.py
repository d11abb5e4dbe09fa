"""Gradient over a packed variable-length batch: HIP path vs the oracle per sequence.

Each (sequence, head) run of a packed batch is the diagonal recurrence (Palimpsa
page, Metodologia 2) over that sequence's tokens from the sequence's own
starting state, read out after every token.  The oracle differentiates every
sequence on its own (fp64, the same adjoint as the fixed-length gradient
tests); the packed gradients are compared element by element at the same
tolerance (|g - g_ref| <= 1e-4 x the oracle's absolute-term scale), dA against
the sum over every sequence of a head and dI_prior against the sum over all.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402
from tests.test_gpu_bwd import _check  # noqa: E402


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _seq(inp, cu, s):
    """The inputs of sequence s as a one-row batch (token axis sliced)."""
    a, b = int(cu[s]), int(cu[s + 1])
    sub = dict(inp)
    for n in ("q", "k", "v", "beta", "d"):
        if inp.get(n) is not None:
            sub[n] = np.ascontiguousarray(inp[n][:, :, a:b])
    return sub


def _states(N, H, dk, dv, seed):
    g = np.random.default_rng(seed)
    shp = (N, H, dk, dv)
    return {"I0": (0.2 + 3.0 * g.random(shp)).astype(np.float32),
            "mu0": g.standard_normal(shp, dtype=np.float32),
            "d_I_T": g.standard_normal(shp, dtype=np.float32),
            "d_mu_T": g.standard_normal(shp, dtype=np.float32)}


def _run(kdn, inp, cu, d_o, st=None):
    x = {n: gu.dev_tensor(inp[n][0]) for n in ("q", "k", "v", "d")}
    beta = gu.dev_tensor(inp["beta"][0]) if inp.get("beta") is not None else None
    dt = lambda n: None if st is None else gu.dev_tensor(st[n])
    g = kdn.kdn_diag_scan_varlen_bwd(x["q"], x["k"], x["v"], beta, x["d"], gu.dev_tensor(inp["A"]),
                                     inp["I_prior"], torch.from_numpy(cu).cuda(), gu.dev_tensor(d_o),
                                     I0=dt("I0"), mu0=dt("mu0"), d_I_T=dt("d_I_T"), d_mu_T=dt("d_mu_T"))
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}


def _compare(g, inp, cu, d_o, st, seqs, heads, whole, what):
    N = len(cu) - 1
    H = inp["q"].shape[1]
    dA = {h: [0.0, 0.0] for h in range(H)}
    dip = [0.0, 0.0]
    fails = []
    for s in seqs:
        a, b = int(cu[s]), int(cu[s + 1])
        sub = _seq(inp, cu, s)
        pick = lambda n: None if st is None else st[n][s:s + 1].astype(np.float64)
        ref = oracle.diag_scan_bwd(sub, d_o[:, :, a:b], heads=[(0, h) for h in heads], I0=pick("I0"),
                                   mu0=pick("mu0"), dI_T=pick("d_I_T"), dmu_T=pick("d_mu_T"))
        for h in heads:
            r = ref[(0, h)]
            for n in ("dq", "dk", "dv", "dbeta", "dd"):
                if n in r and b > a:
                    try:
                        _check(g[n][h, a:b], r[n], r["scale_" + n], f"{what} {n} seq {s} head {h}")
                    except AssertionError as e:
                        fails.append(str(e))
            for n in ("dI0", "dmu0"):
                if n in r:
                    try:
                        _check(g[n][s, h], r[n], r["scale_" + n], f"{what} {n} seq {s} head {h}")
                    except AssertionError as e:
                        fails.append(str(e))
            dA[h][0] += r["dA"]
            dA[h][1] += r["scale_dA"]
            dip[0] += r["dI_prior"]
            dip[1] += r["scale_dI_prior"]
    assert not fails, "\n".join(fails[:10])
    if whole:
        for h in heads:
            _check(g["dA"][h], dA[h][0], dA[h][1], f"{what} dA[{h}]")
        _check(g["dI_prior"][0], dip[0], dip[1], f"{what} dI_prior")


CASES = [
    # (H, N, total_T, d_k, d_v, dtype, M gating, with state)
    (2, 5, 301, 128, 128, "bf16", False, False),
    (2, 4, 150, 64, 32, "f32", False, True),
    (3, 6, 200, 128, 64, "bf16", True, True),
    (1, 1, 77, 64, 16, "f32", False, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "h{}n{}t{}d{}x{}{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "_m" if c[6] else "", "_state" if c[7] else ""))
def test_varlen_bwd(kdn, case):
    H, N, T, dk, dv, dt, mg, with_state = case
    spec = synth.VarlenSpec("varlen_bwd", H, N, T, dk, dv, dt, 7700 + T, m_gating=mg, I_prior=0.8)
    inp = synth.varlen_inputs(spec)
    cu = inp["cu_seqlens"]
    d_o = np.random.default_rng(7701 + T).standard_normal((1, H, T, dv)).astype(np.float32)
    st = _states(N, H, dk, dv, 7702 + T) if with_state else None
    print(f"varlen bwd {case}", flush=True)
    g = _run(kdn, inp, cu, d_o[0], st)
    assert ("dbeta" in g) == (not mg)
    _compare(g, inp, cu, d_o, st, range(N), range(H), True, str(case))


def test_varlen_bwd_empty_sequences(kdn):
    """Sequences of length 0 (their final state is their starting state: dI0 =
    dI_T, dmu0 = dmu_T) next to ragged ones, one of them shorter than a chunk."""
    H, T, dk, dv = 2, 70, 64, 64
    spec = synth.VarlenSpec("varlen_bwd_empty", H, 2, T, dk, dv, "f32", 7800)
    inp = synth.varlen_inputs(spec)
    cu = np.array([0, 0, 9, 9, 70, 70], dtype=np.int64)
    N = len(cu) - 1
    d_o = np.random.default_rng(7801).standard_normal((1, H, T, dv)).astype(np.float32)
    st = _states(N, H, dk, dv, 7802)
    print("varlen bwd empty sequences", flush=True)
    g = _run(kdn, inp, cu, d_o[0], st)
    for s in (0, 2, 4):
        np.testing.assert_array_equal(g["dmu0"][s], st["d_mu_T"][s])
    _compare(g, inp, cu, d_o, st, range(N), range(H), True, "empty")


def test_varlen_bwd_packed_workload_sampled(kdn):
    """The packed workload the benchmark times (64 sequences x 16 heads, 16384
    tokens, d 128, bf16): the longest, the shortest and a middle sequence on two
    heads against the oracle."""
    spec = synth.workload("varlen_n64h16t16384d128_bf16")
    inp = synth.varlen_inputs(spec)
    cu = inp["cu_seqlens"]
    lens = np.diff(cu)
    order = np.argsort(lens)
    seqs = [int(order[-1]), int(order[0]), int(order[len(order) // 2])]
    d_o = np.random.default_rng(7900).standard_normal((1, spec.H, spec.total_T, spec.d_v)).astype(np.float32)
    print("varlen bwd packed workload", flush=True)
    g = _run(kdn, inp, cu, d_o[0])
    _compare(g, inp, cu, d_o, None, seqs, (0, spec.H - 1), False, "packed")


def test_varlen_bwd_deterministic(kdn):
    """Two calls on the same packed batch give bitwise equal gradients."""
    spec = synth.VarlenSpec("varlen_bwd_det", 2, 7, 260, 128, 128, "bf16", 7950)
    inp = synth.varlen_inputs(spec)
    d_o = np.random.default_rng(7951).standard_normal((2, 260, 128)).astype(np.float32)
    a = _run(kdn, inp, inp["cu_seqlens"], d_o)
    b = _run(kdn, inp, inp["cu_seqlens"], d_o)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# long sequences run in 512-token segments at these sizes (kdn_diag_varlen_plan)
SPLIT_LENGTHS = [1500, 30, 700, 0, 2100, 5, 1200, 513, 512]


@pytest.mark.parametrize("case", [(64, 64, "f32", False, True), (128, 128, "bf16", False, False),
                                  (128, 64, "bf16", True, True), (64, 32, "bf16", False, True)],
                         ids=lambda c: "d{}x{}{}{}{}".format(c[0], c[1], c[2], "_m" if c[3] else "",
                                                             "_state" if c[4] else ""))
def test_varlen_bwd_split_sequences(kdn, case):
    """Sequences longer than a fair share run in segments (forward composites
    for their starting states, adjoint composites carried from each sequence's
    end); every sequence against the oracle run on its own."""
    dk, dv, dt, mg, with_state = case
    H = 2
    cu = np.concatenate([[0], np.cumsum(SPLIT_LENGTHS)]).astype(np.int64)
    T, N = int(cu[-1]), len(SPLIT_LENGTHS)
    assert kdn.kdn_diag_varlen_plan(N, H, T, dk, dv)[0] == 512
    spec = synth.VarlenSpec("varlen_bwd_split", H, N, T, dk, dv, dt, 7990, m_gating=mg, I_prior=1.3)
    inp = synth.varlen_inputs(spec)
    inp["cu_seqlens"] = cu
    d_o = np.random.default_rng(7991).standard_normal((1, H, T, dv)).astype(np.float32)
    st = _states(N, H, dk, dv, 7992) if with_state else None
    print(f"varlen bwd split {case}", flush=True)
    g = _run(kdn, inp, cu, d_o[0], st)
    _compare(g, inp, cu, d_o, st, range(N), range(H), True, f"split {case}")


def test_varlen_bwd_skewed_workload_sampled(kdn):
    """The skewed packed batch (one 8192-token sequence among 63 short ones,
    16 heads, d 128 bf16): the long sequence on two heads and a short one
    against the oracle."""
    spec = synth.workload("varlenskew_n64h16t16384d128_bf16")
    inp = synth.varlen_inputs(spec)
    cu = inp["cu_seqlens"]
    d_o = synth.varlen_grad_inputs(spec)["d_o"]
    print("varlen bwd skewed workload", flush=True)
    g = _run(kdn, inp, cu, d_o[0])
    _compare(g, inp, cu, d_o, None, [0, 40], (0, spec.H - 1), False, "skew")


def test_varlen_bwd_split_streams(kdn):
    """With split sequences the whole sequences' checkpoint pass runs on a
    second stream and the reverse pass waits for it: repeated calls, on the
    default stream and on a caller's stream, give bitwise equal gradients."""
    H, dk, dv = 2, 128, 128
    cu = np.concatenate([[0], np.cumsum(SPLIT_LENGTHS)]).astype(np.int64)
    T, N = int(cu[-1]), len(SPLIT_LENGTHS)
    spec = synth.VarlenSpec("varlen_bwd_streams", H, N, T, dk, dv, "bf16", 7993)
    inp = synth.varlen_inputs(spec)
    inp["cu_seqlens"] = cu
    d_o = np.random.default_rng(7994).standard_normal((H, T, dv)).astype(np.float32)
    x = {n: gu.dev_tensor(inp[n][0]) for n in ("q", "k", "v", "beta", "d")}
    args = (x["q"], x["k"], x["v"], x["beta"], x["d"], gu.dev_tensor(inp["A"]), inp["I_prior"],
            torch.from_numpy(cu).cuda(), gu.dev_tensor(d_o))
    print("varlen bwd split streams", flush=True)
    ref = {n: t.cpu() for n, t in kdn.kdn_diag_scan_varlen_bwd(*args).items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for s in (None, side):
            g = kdn.kdn_diag_scan_varlen_bwd(*args, stream=s)
            torch.cuda.synchronize()
            for n in ref:
                assert torch.equal(g[n].cpu(), ref[n]), (rep, s is not None, n)


def test_varlen_bwd_split_host_threads(kdn):
    """Two host threads, each on its own stream, differentiate two different
    split batches at once (the second stream's fork and join are one unit per
    call): each result equals the same call made alone."""
    import threading
    H, dk, dv = 2, 128, 64
    cu = np.concatenate([[0], np.cumsum(SPLIT_LENGTHS)]).astype(np.int64)
    T, N = int(cu[-1]), len(SPLIT_LENGTHS)
    jobs = []
    for seed in (7995, 7997):
        spec = synth.VarlenSpec("varlen_bwd_threads", H, N, T, dk, dv, "bf16", seed)
        inp = synth.varlen_inputs(spec)
        d_o = np.random.default_rng(seed + 1).standard_normal((H, T, dv)).astype(np.float32)
        x = {n: gu.dev_tensor(inp[n][0]) for n in ("q", "k", "v", "beta", "d")}
        jobs.append((x["q"], x["k"], x["v"], x["beta"], x["d"], gu.dev_tensor(inp["A"]), inp["I_prior"],
                     torch.from_numpy(cu).cuda(), gu.dev_tensor(d_o)))
    print("varlen bwd split host threads", flush=True)
    alone = [{n: t.cpu() for n, t in kdn.kdn_diag_scan_varlen_bwd(*a).items()} for a in jobs]
    streams = [torch.cuda.Stream() for _ in jobs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    out = [None, None]
    errs = []

    def work(i):
        try:
            res = []
            for _ in range(4):
                g = kdn.kdn_diag_scan_varlen_bwd(*jobs[i], stream=streams[i])
                streams[i].synchronize()
                res.append({n: t.cpu() for n, t in g.items()})
            out[i] = res
        except Exception as e:  # reported below, in the test's own thread
            errs.append(repr(e))

    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not errs, errs
    for i in range(2):
        assert out[i] is not None, f"thread {i} did not finish"
        for rep, g in enumerate(out[i]):
            for n in alone[i]:
                assert torch.equal(g[n], alone[i][n]), (i, rep, n)

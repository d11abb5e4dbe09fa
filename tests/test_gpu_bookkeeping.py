"""Integer bookkeeping on the device, bit for bit, and buffer robustness.

Every work unit of a scan (main-pass workgroup, composite wave, isotropic
wave) takes its token bounds from the library's device-side bound functions.
With a bounds-echo buffer (kdn_scan_opts) each writes the bounds it used; the
records must equal the oracle's enumeration of the plan from its definition
(oracle.plan / oracle.plan_sub: whole 16-token chunks split evenly over
segments, then over sub-segments), cover every unit exactly once, and, for a
packed batch, follow the longest-first order with the offsets of cu_seqlens.

Also here: canary words around every output buffer (nothing written outside
its range), and a call on a side stream (outputs allocated on that stream).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

W = 8   # int64 words per echo record


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


def _records(echo, words):
    rec = echo[:words].view(-1, W).cpu().numpy()
    return [tuple(int(x) for x in r) for r in rec]


def _zeros_diag(B, H, T, dk, dv):
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    return z(B, H, T, dk), z(B, H, T, dk), z(B, H, T, dv), z(B, H, T, dv), z(B, H, T), \
        torch.ones(H, dtype=torch.float32, device="cuda")


def _check_diag_records(kdn, recs, B, H, T, dk, dv, S_req):
    chunk, S, R, _ = kdn.kdn_diag_plan(B, H, T, dk, dv, segments=S_req)
    _, _, bounds = oracle.plan(T, chunk, S)
    sub = oracle.plan_sub(T, chunk, S, R)
    ntile = dv // min(dv, 64)
    # composite waves of bf16 inputs, echoed by their index in the unit: J
    # waves over tiles of at most 32 key rows x 128 value columns, then X
    # waves over tiles of at most 128 x 32
    ctile = (dk // min(dk, 32)) * (dv // min(dv, 128)) + (dk // min(dk, 128)) * (dv // min(dv, 32))
    main = [r for r in recs if r[0] == 1]
    comp = [r for r in recs if r[0] == 2]
    assert all(r[0] in (1, 2) for r in recs), "records of an unknown kind"
    want_main = {(bh, s, t): (bounds[s], bounds[s + 1]) for bh in range(B * H) for s in range(S)
                 for t in range(ntile)}
    got_main = {}
    for r in main:
        key = (r[1], r[2], r[3])
        assert key not in got_main, f"main unit {key} echoed twice"
        got_main[key] = (r[4], r[5])
        assert r[6] == -1
    assert got_main == want_main
    want_comp = {(bh, s, r, t): sub[(s, r)] for bh in range(B * H) for s in range(S - 1)
                 for r in range(R) for t in range(ctile)}
    got_comp = {}
    for r in comp:
        key = (r[1], r[2], r[3], r[6])
        assert key not in got_comp, f"composite unit {key} echoed twice"
        got_comp[key] = (r[4], r[5])
    assert got_comp == want_comp
    return S, R


@pytest.mark.parametrize("S_req", [1, 3, 5, 0])
@pytest.mark.parametrize("dims", [(128, 128), (64, 32), (32, 64)], ids=lambda d: f"{d[0]}x{d[1]}")
def test_diag_echo_matches_plan(kdn, S_req, dims):
    """Main-pass and composite bounds of a ragged sequence (601 tokens: 38
    chunks, the last of 9 tokens) for several segment counts."""
    dk, dv = dims
    B, H, T = 2, 3, 601
    q, k, v, beta, d, A = _zeros_diag(B, H, T, dk, dv)
    echo = torch.zeros(1 << 16, dtype=torch.int64, device="cuda")
    info = {}
    kdn.kdn_diag_scan_fwd(q, k, v, beta, d, A, 1.0, segments=S_req, echo=echo, info=info)
    torch.cuda.synchronize()
    assert 0 < info["echo_words"] <= echo.numel()
    _check_diag_records(kdn, _records(echo, info["echo_words"]), B, H, T, dk, dv, S_req)


def test_diag_echo_full_size_auto_plan(kdn):
    """The long-sequence workload's shape (B2 H16 T16384 d128) with the
    automatic plan the benchmark uses: segments and sub-segments bit-exact."""
    B, H, T, dk, dv = 2, 16, 16384, 128, 128
    q, k, v, beta, d, A = _zeros_diag(B, H, T, dk, dv)
    echo = torch.zeros(1 << 18, dtype=torch.int64, device="cuda")
    info = {}
    kdn.kdn_diag_scan_fwd(q, k, v, beta, d, A, 1.0, echo=echo, info=info)
    torch.cuda.synchronize()
    S, R = _check_diag_records(kdn, _records(echo, info["echo_words"]), B, H, T, dk, dv, 0)
    assert S > 1 and R >= 1


def test_echo_capacity_is_respected(kdn):
    """Records past echo_capacity are dropped: the words after it stay 0."""
    B, H, T, dk, dv = 1, 2, 100, 64, 64
    q, k, v, beta, d, A = _zeros_diag(B, H, T, dk, dv)
    buf = torch.zeros(64, dtype=torch.int64, device="cuda")
    info = {}
    kdn.kdn_diag_scan_fwd(q, k, v, beta, d, A, 1.0, segments=3, echo=buf[:16], info=info)
    torch.cuda.synchronize()
    assert info["echo_words"] > 16
    assert torch.all(buf[16:] == 0)
    assert torch.any(buf[:16] != 0)


def test_varlen_echo_order_and_offsets(kdn):
    """Packed batch: run r of the dispatch order is (sequence seq_order[r // H],
    head r % H), sequences longest first (ties by index), with the token
    bounds of cu_seqlens; every (sequence, head, tile) exactly once."""
    lengths = [5, 40, 0, 17, 40, 1, 33, 16, 9, 40, 2]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    H, dk, dv = 3, 128, 128
    T = int(cu[-1])
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    echo = torch.zeros(1 << 14, dtype=torch.int64, device="cuda")
    info = {}
    kdn.kdn_diag_scan_varlen_fwd(z(H, T, dk), z(H, T, dk), z(H, T, dv), z(H, T, dv), z(H, T),
                                 torch.ones(H, dtype=torch.float32, device="cuda"), 1.0,
                                 torch.from_numpy(cu).cuda(), echo=echo, info=info)
    torch.cuda.synchronize()
    recs = _records(echo, info["echo_words"])
    N = len(lengths)
    order = sorted(range(N), key=lambda s: (-lengths[s], s))
    ntile = dv // 64
    seen = set()
    for slot, r in enumerate(recs):
        if r[0] == 0:
            continue   # padding of the last group of 8 runs
        within = slot % (8 * ntile)
        tile = within // 8
        run = slot // (8 * ntile) * 8 + within % 8
        seq = order[run // H]
        head = run % H
        assert r == (1, seq * H + head, 0, tile, int(cu[seq]), int(cu[seq + 1]), seq, 0), (slot, r)
        seen.add((seq, head, tile))
    assert seen == {(s, h, t) for s in range(N) for h in range(H) for t in range(ntile)}


@pytest.mark.parametrize("S_req", [1, 4, 0])
def test_iso_echo_matches_plan(kdn, S_req):
    B, H, T, dk, dv = 1, 3, 1000, 64, 64
    f = lambda *s: torch.rand(s, dtype=torch.float32, device="cuda") * 0.5 + 0.25
    echo = torch.zeros(1 << 15, dtype=torch.int64, device="cuda")
    info = {}
    kdn.kdn_mobius_precision_scan(f(B, H, T), f(B, H, T), f(B, H, T), None, f(B, H, T, dk),
                                  f(B, H, T, dk), f(B, H, T, dv), segments=S_req, echo=echo,
                                  info=info)
    torch.cuda.synchronize()
    recs = [r for r in _records(echo, info["echo_words"]) if r[0] != 0]
    mean = [r for r in recs if r[0] == 3]
    comp = [r for r in recs if r[0] == 4]
    S = 1 + max(r[2] for r in mean)
    if S_req:
        assert S == min(S_req, -(-T // 16))
    _, _, bounds = oracle.plan(T, 16, S)
    ntile = len({r[3] for r in mean})
    assert sorted((r[1], r[2], r[3]) for r in mean) == \
        [(bh, s, t) for bh in range(B * H) for s in range(S) for t in range(ntile)]
    for r in mean + comp:
        assert (r[4], r[5]) == (bounds[r[2]], bounds[r[2] + 1]), r
    assert sorted((r[1], r[2], r[3]) for r in comp) == \
        [(bh, s, t) for bh in range(B * H) for s in range(S - 1) for t in range(ntile)]


CANARY = 0x7fc0dead   # a NaN pattern no result can take


def _guarded(shape, pad=64):
    """A float32 tensor view with `pad` canary words on both sides."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * pad, dtype=torch.float32, device="cuda")
    buf.view(torch.int32).fill_(CANARY)
    return buf, buf[pad:pad + n].view(shape)


def _intact(buf, n, pad=64):
    w = buf.view(torch.int32)
    return bool(torch.all(w[:pad] == CANARY)) and bool(torch.all(w[pad + n:] == CANARY))


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("dv", [128, 32])
def test_outputs_stay_inside_their_buffers(kdn, S, dv):
    """Canary words before and after o, I_T and mu_T survive the call, on a
    ragged sequence, and the results inside still match the oracle."""
    B, H, T, dk = 2, 2, 77, 128
    inp = synth.diag_inputs(gu.diag_spec(B, H, T, dk, dv, "bf16", seed=71))
    x = gu.upload_diag(inp)
    bo, o = _guarded((B, H, T, dv))
    bi, I_T = _guarded((B, H, dk, dv))
    bm, mu_T = _guarded((B, H, dk, dv))
    kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], 1.0, o=o, I_T=I_T,
                          mu_T=mu_T, segments=S)
    torch.cuda.synchronize()
    assert _intact(bo, o.numel()) and _intact(bi, I_T.numel()) and _intact(bm, mu_T.numel())
    gu.compare_diag(inp, (o, I_T, mu_T), [(b, h) for b in range(B) for h in range(H)],
                    what=f"guarded S={S} dv={dv}")


def test_side_stream(kdn):
    """Forward, backward and Mobius calls enqueued on a side stream (outputs
    and workspace allocated there) give the oracle's results once that stream
    is synchronised."""
    B, H, T, dk, dv = 1, 2, 90, 128, 64
    spec = gu.diag_spec(B, H, T, dk, dv, "bf16", seed=73)
    inp = synth.diag_inputs(spec)
    x = gu.upload_diag(inp)
    gr = synth.grad_inputs(spec, final_state=False)
    d_o = gu.dev_tensor(gr["d_o"])
    ispec = synth.IsoSpec("iso_side", 1, 2, 300, 32, 32, 74)
    iinp = synth.iso_inputs(ispec)
    y = gu.upload_iso(iinp)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    res = kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], 1.0,
                                segments=2, stream=side)
    g = kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], 1.0, d_o,
                              stream=side)
    lam, io, _ = kdn.kdn_mobius_precision_scan(y["a"], y["p"], y["Lambda"], y["lambda0"], y["q"],
                                               y["k"], y["v"], stream=side)
    # churn the allocator on the default stream while the side stream runs
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    side.synchronize()
    del junk
    heads = [(0, 0), (0, 1)]
    gu.compare_diag(inp, res, heads, what="side stream")
    ref = oracle.diag_scan_bwd(inp, gr["d_o"], heads=heads)
    for (b, h) in heads:
        err = np.abs(g["dq"][b, h].cpu().numpy() - ref[(b, h)]["dq"])
        assert np.all(err <= 1e-4 * ref[(b, h)]["scale_dq"] + 1e-30)
    iref = oracle.iso_scan(iinp)
    for (b, h), r in iref.items():
        gu.check_rel(lam[b, h].cpu().numpy(), r["lambda"], "side stream lambda")
        gu.check_o(io[b, h].cpu().numpy(), r, "side stream iso o")


def test_main_pass_events(kdn):
    """The events of the options struct bracket the main pass alone: the
    composite passes come before main_begin, and the main pass sits inside
    the whole call's events (the benchmark times the main pass with them)."""
    B, H, T, dk, dv = 1, 4, 4000, 128, 128
    q, k, v, beta, d, A = _zeros_diag(B, H, T, dk, dv)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    print("main-pass events, diagonal S=3", flush=True)
    ev[0].record()
    kdn.kdn_diag_scan_fwd(q, k, v, beta, d, A, 1.0, segments=3, timing=(ev[1], ev[2]))
    ev[3].record()
    torch.cuda.synchronize()
    before, main, call = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0 < main <= call and before > 0, (before, main, call)
    # the isotropic call and the packed batch record them too
    f = lambda *s: torch.rand(s, device="cuda") + 0.5
    kdn.kdn_mobius_precision_scan(f(1, 2, 300), f(1, 2, 300), f(1, 2, 300), q=f(1, 2, 300, 64),
                                  k=f(1, 2, 300, 64), v=f(1, 2, 300, 64), timing=(ev[1], ev[2]))
    cu = torch.tensor([0, 100, 300], dtype=torch.int64, device="cuda")
    c = lambda x: x[0, :2, :300].contiguous()
    kdn.kdn_diag_scan_varlen_fwd(c(q), c(k), c(v), c(beta), c(d), A[:2].contiguous(), 1.0, cu,
                                 timing=(ev[0], ev[3]))
    torch.cuda.synchronize()
    assert ev[1].elapsed_time(ev[2]) > 0 and ev[0].elapsed_time(ev[3]) > 0

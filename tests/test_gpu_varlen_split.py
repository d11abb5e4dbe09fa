"""Packed batches whose long sequences run in segments, on the GPU.

A sequence longer than the plan's segment length is cut into segments; the
composite of every segment but its last is built on the matrix cores, the
composites are carried in order, and each segment's main pass starts from
the carried state (the associative composition of the KLA summary,
Metodologia 2).  Results are compared with the oracle, which runs every
(sequence, head) as one sequential recurrence (Palimpsa page, Metodologia
1-3), element by element at the usual tolerance; the bounds every work unit
used are compared bit for bit with the oracle's enumeration of the plan.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bayesian_memory_scan_amd import synth  # noqa: E402
from tests import gpu_util as gu  # noqa: E402
from tests.test_gpu_mgate_varlen import _compare_varlen  # noqa: E402

W = 8   # int64 words per echo record


@pytest.fixture(scope="module")
def kdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bayesian_memory_scan_amd import kdnscan
    return kdnscan


# 512-token segments at these sizes: 1500 -> 3 segments, 700 -> 2, 2100 -> 5,
# 1200 -> 3, 513 -> 2 (a 1-token last segment), 512 -> not split
LENGTHS = [1500, 30, 700, 0, 2100, 5, 1200, 513, 512]


def _inputs(dk, dv, dt, seed, m_gating=False, lengths=LENGTHS, H=2):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    spec = gu.diag_spec(1, H, int(cu[-1]), dk, dv, dt, seed=seed)
    inp = synth.diag_inputs(spec)
    inp["cu_seqlens"] = cu
    if m_gating:
        inp["beta"] = None
    return spec, inp


def _run(kdn, inp, st=None, segments=0, echo=None, info=None):
    x = gu.upload_diag({**inp, "beta": inp["d"] if inp["beta"] is None else inp["beta"]})
    sq = lambda t: t[0]
    beta = None if inp["beta"] is None else sq(x["beta"])
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    I0 = None if st is None else gu.dev_tensor(st["I0"])
    mu0 = None if st is None else gu.dev_tensor(st["mu0"])
    res = kdn.kdn_diag_scan_varlen_fwd(sq(x["q"]), sq(x["k"]), sq(x["v"]), beta, sq(x["d"]), x["A"],
                                       inp["I_prior"], cu, I0=I0, mu0=mu0, segments=segments,
                                       echo=echo, info=info)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in res]


def test_plan_splits_these_lengths(kdn):
    T = sum(LENGTHS)
    for dk, dv in ((64, 64), (128, 128), (64, 32)):
        seg, R, items, comps = kdn.kdn_diag_varlen_plan(len(LENGTHS), 2, T, dk, dv)
        assert seg == 512 and comps == T // 512 and items == len(LENGTHS) + comps and R >= 1


@pytest.mark.parametrize("m_gating", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("dims", [(64, 64, "f32"), (128, 128, "bf16"), (64, 32, "bf16"),
                                  (128, 64, "f32")], ids=lambda s: "x".join(map(str, s)))
def test_split_parity(kdn, dims, with_state, m_gating):
    dk, dv, dt = dims
    spec, inp = _inputs(dk, dv, dt, 301, m_gating)
    st = synth.state_inputs(spec.with_(B=len(LENGTHS))) if with_state else None
    print(f"split parity {dims} state={with_state} m={m_gating}", flush=True)
    _compare_varlen(inp, _run(kdn, inp, st), st, what=f"split {dims}")


def test_split_agrees_with_unsplit(kdn):
    """segments = 1 runs every sequence whole; both plans agree with the
    oracle, and with each other to the same tolerance."""
    spec, inp = _inputs(128, 128, "bf16", 302)
    a = _run(kdn, inp, segments=0)
    b = _run(kdn, inp, segments=1)
    _compare_varlen(inp, b, what="unsplit")
    ref = oracle.diag_scan_varlen(inp, inp["cu_seqlens"])
    cu = inp["cu_seqlens"]
    for (s, h), r in ref.items():
        t0, t1 = int(cu[s]), int(cu[s + 1])
        if t1 > t0:
            scale = np.asarray(r["s"]) + 1e-30
            assert np.max(np.abs(a[0][h, t0:t1] - b[0][h, t0:t1]) / scale) <= 2e-4, (s, h)


def test_split_echo_matches_plan(kdn):
    """Every main-pass workgroup and composite wave reports the bounds it
    used; they equal the oracle's enumeration of the plan (kdn_diag_varlen_plan's
    segment length and sub-segments), with the main-pass items in dispatch
    order, bit for bit."""
    H, dk, dv = 2, 128, 128
    spec, inp = _inputs(dk, dv, "bf16", 303, H=H)
    N, T = len(LENGTHS), int(inp["cu_seqlens"][-1])
    seg, R, items_cap, comps_cap = kdn.kdn_diag_varlen_plan(N, H, T, dk, dv)
    # sub-segments: the composite storage spread over the composite segments there are
    C = len(oracle.varlen_plan(inp["cu_seqlens"], seg, 1)[1])
    R_used = min(seg // 64, comps_cap * R // C)
    items, comps = oracle.varlen_plan(inp["cu_seqlens"], seg, R_used)
    echo = torch.zeros(1 << 17, dtype=torch.int64, device="cuda")
    info = {}
    _run(kdn, inp, echo=echo, info=info)
    words = info["echo_words"]
    assert 0 < words <= echo.numel()
    recs = [tuple(int(x) for x in r) for r in echo[:words].view(-1, W).cpu().numpy()]
    ntile = dv // 64
    main_grid = (items_cap * H + 7) // 8 * 8 * ntile
    # bf16 composite waves per unit at d_k = d_v = 128: four J waves (32 x 128
    # tiles) and four X waves (128 x 32)
    assert words == W * (main_grid + comps_cap * H * R * (4 + 4))
    seen = set()
    for slot, r in enumerate(recs[:main_grid]):
        within = slot % (8 * ntile)
        tile = within // 8
        run = slot // (8 * ntile) * 8 + within % 8
        item, head = divmod(run, H)
        if item >= len(items):
            assert r == (0,) * W, (slot, r)   # past the plan's items: untouched
            continue
        s, g, t0, t1 = items[item]
        assert r == (1, s * H + head, g, tile, t0, t1, s, 0), (slot, r, items[item])
        seen.add((item, head, tile))
    assert len(seen) == len(items) * H * ntile
    want = {}
    for s, g, subs in comps:
        for r_, (t0, t1) in enumerate(subs):
            for h in range(H):
                for tile in range(4 + 4):
                    want[(s * H + h, g, r_, tile)] = (t0, t1, s)
    got = {}
    for r in recs[main_grid:]:
        if r[0] == 0:
            continue   # composite capacity past the plan's composites
        assert r[0] == 2
        key = (r[1], r[2], r[3], r[6])
        assert key not in got, f"composite unit {key} echoed twice"
        got[key] = (r[4], r[5], r[7])
    assert got == want


def test_skewed_workload_sampled(kdn):
    """The skewed packed workload the benchmark times (one 8192-token sequence
    and 63 short ones, 16 heads, d 128 bf16): the long sequence on two heads
    and two short ones against the oracle."""
    spec = synth.workload("varlenskew_n64h16t16384d128_bf16")
    inp = synth.varlen_inputs(spec)
    seg = kdn.kdn_diag_varlen_plan(spec.N, spec.H, spec.total_T, spec.d_k, spec.d_v)[0]
    assert 0 < seg < 8192
    print("skewed workload", flush=True)
    _compare_varlen(inp, _run(kdn, inp), runs=[(0, 0), (0, 15), (1, 7), (63, 3)], what="skew")

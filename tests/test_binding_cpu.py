"""The torch front ends and the extended entry points on the CPU.

Every mismatch of a tensor's shape or dtype against the sizes taken from q
and v (or a, p, Lambda) raises before the library is called, as does a tensor
off the GPU: the C ABI takes bare pointers and could not tell.  The extended
entry points validate their options before any HIP call, and report the size
of the bounds echo on a workspace query.  No GPU is needed.
"""
import ctypes

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
kdn = pytest.importorskip("bayesian_memory_scan_amd.kdnscan")
lib = kdn.lib
FAKE = 0x10000


def _diag_tensors(B=2, H=3, T=5, dk=16, dv=32, dtype=torch.bfloat16):
    z = lambda *s: torch.zeros(s, dtype=dtype)
    return dict(q=z(B, H, T, dk), k=z(B, H, T, dk), v=z(B, H, T, dv), beta=z(B, H, T, dv),
                d=z(B, H, T), A=torch.ones(H))


def _call_fwd(x, **kw):
    return kdn.kdn_diag_scan_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], 1.0, **kw)


@pytest.mark.parametrize("name,shape", [
    ("k", (2, 3, 5, 8)), ("v", (2, 3, 4, 32)), ("beta", (2, 3, 5, 16)), ("d", (2, 3, 4)),
    ("d", (2, 3, 5, 1)), ("A", (1,)), ("A", (4,))])
def test_forward_shape_mismatch_raises(name, shape):
    x = _diag_tensors()
    x[name] = torch.zeros(shape, dtype=x[name].dtype)
    with pytest.raises(ValueError, match=name):
        _call_fwd(x)


@pytest.mark.parametrize("name", ["I0", "mu0", "o", "I_T", "mu_T"])
def test_forward_state_shape_mismatch_raises(name):
    x = _diag_tensors()
    bad = torch.zeros((2, 3, 16, 16))   # d_v is 32
    with pytest.raises(ValueError, match=name):
        _call_fwd(x, **{name: bad})


def test_forward_dtype_rules():
    x = _diag_tensors()
    x["k"] = x["k"].float()
    with pytest.raises(TypeError, match="share one dtype"):
        _call_fwd(x)
    x = _diag_tensors()
    x["A"] = x["A"].double()
    with pytest.raises(TypeError, match="A"):
        _call_fwd(x)


def test_forward_needs_gpu_tensors():
    with pytest.raises(ValueError, match="GPU"):
        _call_fwd(_diag_tensors())


def test_forward_rejects_negative_segments_and_bad_echo():
    x = _diag_tensors()
    with pytest.raises(ValueError):
        _call_fwd(x, segments=-1)


def test_decode_shapes_and_dtypes():
    B, H, dk, dv = 2, 3, 16, 32
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt)
    args = dict(q=z(B, H, dk), k=z(B, H, dk), v=z(B, H, dv), beta=z(B, H, dv), d=z(B, H),
                A=torch.ones(H), I=z(B, H, dk, dv, dt=torch.float32), mu=z(B, H, dk, dv, dt=torch.float32))

    def call(**over):
        a = {**args, **over}
        return kdn.kdn_decode_step(a["q"], a["k"], a["v"], a["beta"], a["d"], a["A"], 1.0, a["I"],
                                   a["mu"])

    with pytest.raises(ValueError, match="I"):
        call(I=z(B, H, dk, dk, dt=torch.float32))
    with pytest.raises(ValueError, match="mu"):
        call(mu=z(B, H + 1, dk, dv, dt=torch.float32))
    with pytest.raises(TypeError, match="share one dtype"):
        call(k=z(B, H, dk, dt=torch.float32))
    with pytest.raises(ValueError, match="A"):
        call(A=torch.ones(1))
    with pytest.raises(ValueError, match="GPU"):
        call()


def test_varlen_and_mobius_shapes():
    H, T, dk, dv = 2, 9, 16, 16
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, 9], dtype=torch.int64)
    with pytest.raises(ValueError, match="I0"):
        kdn.kdn_diag_scan_varlen_fwd(z(H, T, dk), z(H, T, dk), z(H, T, dv), z(H, T, dv), z(H, T),
                                     torch.ones(H), 1.0, cu, I0=torch.zeros((3, H, dk, dv)))
    with pytest.raises(ValueError, match="d"):
        kdn.kdn_diag_scan_varlen_fwd(z(H, T, dk), z(H, T, dk), z(H, T, dv), z(H, T, dv), z(H, T + 1),
                                     torch.ones(H), 1.0, cu)
    f = lambda *s: torch.zeros(s)
    with pytest.raises(ValueError, match="p"):
        kdn.kdn_mobius_precision_scan(f(1, 2, 8), f(1, 2, 9), f(1, 2, 8))
    with pytest.raises(ValueError, match="lambda0"):
        kdn.kdn_mobius_precision_scan(f(1, 2, 8), f(1, 2, 8), f(1, 2, 8), lambda0=f(2, 1))
    with pytest.raises(ValueError, match="k"):
        kdn.kdn_mobius_precision_scan(f(1, 2, 8), f(1, 2, 8), f(1, 2, 8), q=f(1, 2, 8, 16),
                                      k=f(1, 2, 8, 32), v=f(1, 2, 8, 16))
    with pytest.raises(ValueError, match="q, k and v"):
        kdn.kdn_mobius_precision_scan(f(1, 2, 8), f(1, 2, 8), f(1, 2, 8), q=f(1, 2, 8, 16))


def test_backward_and_noise_shapes():
    x = _diag_tensors()
    with pytest.raises(ValueError, match="d_o"):
        kdn.kdn_diag_scan_bwd(x["q"], x["k"], x["v"], x["beta"], x["d"], x["A"], 1.0,
                              torch.zeros((2, 3, 5, 16)))
    with pytest.raises(ValueError, match="a"):
        kdn.kdn_diag_noise_scan_fwd(x["q"], x["k"], x["v"], x["beta"], torch.zeros((2, 3, 4)),
                                    torch.zeros((2, 3, 5)))


def test_varlen_backward_shapes():
    H, T, dk, dv = 2, 9, 64, 16
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    f = lambda *s: torch.zeros(s)
    cu = torch.tensor([0, 4, 9], dtype=torch.int64)
    args = lambda d_o: (z(H, T, dk), z(H, T, dk), z(H, T, dv), z(H, T, dv), z(H, T), torch.ones(H),
                        1.0, cu, d_o)
    with pytest.raises(ValueError, match="d_o"):
        kdn.kdn_diag_scan_varlen_bwd(*args(f(H, T + 1, dv)))
    with pytest.raises(ValueError, match="d_o"):
        kdn.kdn_diag_scan_varlen_bwd(*args(None))
    with pytest.raises(ValueError, match="d_mu_T"):
        kdn.kdn_diag_scan_varlen_bwd(*args(f(H, T, dv)), d_mu_T=f(3, H, dk, dv))
    with pytest.raises(TypeError, match="cu_seqlens"):
        kdn.kdn_diag_scan_varlen_bwd(*args(f(H, T, dv))[:7], cu.int(), f(H, T, dv))
    with pytest.raises(ValueError, match="GPU"):
        kdn.kdn_diag_scan_varlen_bwd(*args(f(H, T, dv)))


# --- the extended C entry points -----------------------------------------

def _fwd_ex(opts, B=1, H=2, T=100, dk=64, dv=64, nbytes=None):
    n = ctypes.c_size_t(0) if nbytes is None else nbytes
    return lib.kdn_diag_scan_fwd_ex(B, H, T, dk, dv, kdn.KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    1.0, None, None, FAKE, None, None,
                                    None if opts is None else ctypes.byref(opts), None,
                                    ctypes.byref(n), None), n


def test_ex_null_opts_equals_plain_call():
    rc, n_ex = _fwd_ex(None, B=2, H=16, T=16384, dk=128, dv=128)
    n = ctypes.c_size_t(0)
    rc2 = lib.kdn_diag_scan_fwd(2, 16, 16384, 128, 128, kdn.KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 1.0, None, None, FAKE, None, None, None, ctypes.byref(n), None)
    assert rc == rc2 == kdn.KDN_OK and n_ex.value == n.value


def test_ex_option_validation():
    o = kdn.ScanOpts()
    o.segments = -1
    assert _fwd_ex(o)[0] == kdn.KDN_EINVAL
    o = kdn.ScanOpts()
    o.bounds_echo = FAKE + 4      # not 8-byte aligned
    o.echo_capacity = 64
    assert _fwd_ex(o)[0] == kdn.KDN_EINVAL
    o = kdn.ScanOpts()
    o.echo_capacity = -1
    assert _fwd_ex(o)[0] == kdn.KDN_EINVAL


def test_ex_segments_change_the_workspace_and_echo_size():
    """The per-call segment request reaches the plan: more segments need
    more workspace (composites) and report more echo records."""
    sizes, words = [], []
    for S in (1, 2, 4):
        o = kdn.ScanOpts()
        o.segments = S
        rc, n = _fwd_ex(o, B=1, H=2, T=1000, dk=128, dv=128)
        assert rc == kdn.KDN_OK
        sizes.append(n.value)
        words.append(o.echo_words)
        _, S_plan, R, _ = kdn.kdn_diag_plan(1, 2, 1000, 128, 128, segments=S)
        # bf16 composites at d_k = d_v = 128: four J waves (32 x 128 tiles)
        # and four X waves (128 x 32) per sub-segment
        comp_units = 2 * (S_plan - 1) * R * (4 + 4)
        assert o.echo_words == kdn.KDN_ECHO_WORDS * (2 * S_plan * 2 + comp_units)
    assert sizes[0] < sizes[1] < sizes[2] and words[0] < words[1] < words[2]


def test_workspace_needed_at_one_segment():
    """The forward call always needs its per-token frame scalars (16 bytes
    per head and token), even with a single segment."""
    o = kdn.ScanOpts()
    o.segments = 1
    rc, n = _fwd_ex(o, B=1, H=2, T=100, dk=64, dv=64)
    assert rc == kdn.KDN_OK and n.value >= 16 * 2 * 100


def test_varlen_ex_rejects_segments():
    o = kdn.ScanOpts()
    o.segments = 2
    n = ctypes.c_size_t(0)
    rc = lib.kdn_diag_scan_varlen_fwd_ex(2, 2, 50, 64, 64, kdn.KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, 1.0, None, None, FAKE, None, None,
                                         ctypes.byref(o), None, ctypes.byref(n), None)
    assert rc == kdn.KDN_EINVAL


def test_mobius_ex_segments():
    words = []
    for S in (1, 3):
        o = kdn.ScanOpts()
        o.segments = S
        n = ctypes.c_size_t(0)
        rc = lib.kdn_mobius_precision_scan_ex(1, 2, 500, FAKE, FAKE, FAKE, None, FAKE, 64, 64, FAKE,
                                              FAKE, FAKE, None, FAKE, None, ctypes.byref(o), None,
                                              ctypes.byref(n), None)
        assert rc == kdn.KDN_OK
        words.append(o.echo_words)
    assert words[1] == 2 * 3 * words[0]   # 3 segments, each with a composite unit but the last


@pytest.mark.parametrize("T", [1, 17, 601, 16384])
@pytest.mark.parametrize("S", [0, 2, 3, 5])
def test_plan_subsegments_match_oracle(T, S):
    """Sub-segment counts and bounds: the library's plan against the oracle's
    enumeration (every sub-segment nonempty when the segment has chunks to give)."""
    chunk, segs, R, bounds = kdn.kdn_diag_plan(2, 16, T, 128, 128, segments=S)
    _, _, ref = oracle.plan(T, chunk, segs)
    assert bounds == ref
    sub = oracle.plan_sub(T, chunk, segs, R)
    assert len(sub) == (segs - 1) * R
    for s in range(segs - 1):
        assert sub[(s, 0)][0] == ref[s] and sub[(s, R - 1)][1] == ref[s + 1]
        for r in range(R - 1):
            assert sub[(s, r)][1] == sub[(s, r + 1)][0]
    assert np.all(np.diff(ref) >= 0)

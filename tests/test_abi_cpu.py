"""The C ABI on the CPU: symbols, argument validation, workspace protocol and
the chunk/segment plan (bit-exact against the oracle's enumeration).  Every
call here returns before any HIP call, so no GPU is needed."""
import ctypes
import subprocess

import pytest

import oracle

kdn = pytest.importorskip("bayesian_memory_scan_amd.kdnscan")
lib = kdn.lib

FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced
MIS = FAKE + 4


def test_exports_every_header_symbol():
    names = kdn.header_functions()
    assert {"kdn_diag_scan_fwd", "kdn_mobius_precision_scan", "kdn_decode_step",
            "kdn_status_string"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", kdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, f"{n} declared in kdnscan.h but not exported"
        assert hasattr(lib, n)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(kdn.kdn_status_string(code), str) and kdn.kdn_status_string(code)


def _diag(B=1, H=1, T=8, dk=16, dv=16, dt=kdn.KDN_F32, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, d=FAKE,
          A=FAKE, I_prior=1.0, I0=None, mu0=None, o=FAKE, I_T=None, mu_T=None, ws=None,
          nbytes=None):
    nb = None if nbytes is None else ctypes.byref(nbytes)
    return lib.kdn_diag_scan_fwd(B, H, T, dk, dv, dt, q, k, v, beta, d, A, I_prior, I0, mu0,
                                 o, I_T, mu_T, ws, nb, None)


def test_diag_validation():
    n = ctypes.c_size_t(0)
    q = dict(nbytes=n)  # query mode: validation then return, never a launch
    assert _diag(**q) == kdn.KDN_OK
    assert _diag(B=-1, **q) == kdn.KDN_EINVAL
    assert _diag(T=-5, **q) == kdn.KDN_EINVAL
    assert _diag(dk=24, **q) == kdn.KDN_EUNSUPPORTED
    assert _diag(dv=256, **q) == kdn.KDN_EUNSUPPORTED
    assert _diag(dt=7, **q) == kdn.KDN_EINVAL
    assert _diag(I_prior=0.0, **q) == kdn.KDN_EINVAL
    assert _diag(I_prior=float("nan"), **q) == kdn.KDN_EINVAL
    assert _diag(I_prior=-1.0, **q) == kdn.KDN_EINVAL
    for name in ("q", "k", "v", "d", "A", "o"):
        assert _diag(**{name: None}, **q) == kdn.KDN_EINVAL, name
    for name in ("q", "k", "v", "beta", "d", "A", "o"):
        assert _diag(**{name: MIS}, **q) == kdn.KDN_EINVAL, name
    # beta may be NULL: Palimpsa-M gating (the step gate d_t is the input gate)
    assert _diag(beta=None, **q) == kdn.KDN_OK
    for name in ("I0", "mu0", "I_T", "mu_T"):
        assert _diag(**{name: MIS}, **q) == kdn.KDN_EINVAL, name
    # empty batches need no input pointers
    assert _diag(B=0, q=None, k=None, v=None, beta=None, d=None, A=None, o=None, **q) == kdn.KDN_OK
    assert _diag(T=0, q=None, k=None, v=None, beta=None, d=None, o=None, **q) == kdn.KDN_OK


def test_size_limits():
    """T below 2^31; one dispatch within 2^32 - 1 work-items (512 threads per
    head, 64 per composite or isotropic wave)."""
    n = ctypes.c_size_t(0)
    assert _diag(T=2 ** 31, nbytes=n) == kdn.KDN_EINVAL
    assert _diag(T=2 ** 31 - 1, nbytes=n) == kdn.KDN_OK
    # 2^23 heads of one 16-column tile: 2^32 threads, one past the limit
    assert _diag(B=2 ** 23, nbytes=n) == kdn.KDN_EINVAL
    assert _diag(B=2 ** 23 - 1, nbytes=n) == kdn.KDN_OK
    call = lambda B, T=8: lib.kdn_mobius_precision_scan(B, 1, T, FAKE, FAKE, FAKE, None, FAKE, 0, 0,
                                                         None, None, None, None, None, None,
                                                         None, ctypes.byref(n), None)
    assert call(2 ** 23 - 1) == kdn.KDN_OK
    assert call(2 ** 23) == kdn.KDN_EINVAL
    assert call(1, T=2 ** 31) == kdn.KDN_EINVAL
    dec = lambda B: lib.kdn_decode_step(B, 1, 16, 16, kdn.KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, 1.0, FAKE, FAKE, FAKE, None)
    assert dec(2 ** 23) == kdn.KDN_EINVAL


def test_diag_workspace_protocol():
    n = ctypes.c_size_t(12345)
    assert _diag(B=8, H=16, T=2048, dk=128, dv=128, nbytes=n) == kdn.KDN_OK
    assert n.value == 16 * 8 * 16 * 2048  # one segment: per-token scalars only
    n = ctypes.c_size_t(0)
    assert _diag(B=2, H=16, T=16384, dk=128, dv=128, nbytes=n) == kdn.KDN_OK
    chunk, S, _, _ = kdn.kdn_diag_plan(2, 16, 16384, 128, 128)
    expect = 16 * 2 * 16 * 16384 + 4 * 2 * 16 * S * 2 * 128 * 128
    assert n.value >= expect and n.value % 256 == 0
    need = n.value
    # running with too little (or no) workspace is refused before any launch
    small = ctypes.c_size_t(need - 1)
    assert _diag(B=2, H=16, T=16384, dk=128, dv=128, ws=FAKE, nbytes=small) == kdn.KDN_EWORKSPACE
    assert small.value == need
    assert _diag(B=2, H=16, T=16384, dk=128, dv=128, ws=None, nbytes=None) == kdn.KDN_EWORKSPACE


def test_mobius_validation_and_workspace():
    n = ctypes.c_size_t(0)
    nb = ctypes.byref(n)
    call = lambda B=1, H=1, T=8, dk=0, dv=0, a=FAKE, p=FAKE, L=FAKE, q=FAKE, o=FAKE: \
        lib.kdn_mobius_precision_scan(B, H, T, a, p, L, None, FAKE, dk, dv, q, q, q, None, o,
                                      None, None, nb, None)
    assert call() == kdn.KDN_OK and n.value > 0          # precision path: block composites
    prec = n.value
    assert call(dk=64, dv=64) == kdn.KDN_OK and n.value > prec  # + gates (+ segment carry)
    assert call(dk=48, dv=64) == kdn.KDN_EUNSUPPORTED
    assert call(B=-1) == kdn.KDN_EINVAL
    assert call(a=None) == kdn.KDN_EINVAL
    assert call(L=MIS) == kdn.KDN_EINVAL
    assert call(dk=64, dv=64, q=None) == kdn.KDN_EINVAL
    assert call(dk=64, dv=64, o=None) == kdn.KDN_EINVAL
    assert call(T=0, a=None, p=None, L=None) == kdn.KDN_OK and n.value == 0


def test_decode_validation():
    call = lambda B=1, H=1, dk=16, dv=16, dt=kdn.KDN_BF16, I_prior=1.0, I=FAKE, q=FAKE: \
        lib.kdn_decode_step(B, H, dk, dv, dt, q, FAKE, FAKE, FAKE, FAKE, FAKE, I_prior, I, FAKE,
                            FAKE, None)
    assert call(B=-1) == kdn.KDN_EINVAL
    assert call(dk=8) == kdn.KDN_EUNSUPPORTED
    assert call(I_prior=0.0) == kdn.KDN_EINVAL
    assert call(I=None) == kdn.KDN_EINVAL
    assert call(q=MIS) == kdn.KDN_EINVAL
    assert call(dt=3) == kdn.KDN_EINVAL
    assert call(B=0, I=None, q=None) == kdn.KDN_OK


@pytest.mark.parametrize("T", [1, 15, 16, 17, 64, 100, 2048, 16383, 16384, 65536])
@pytest.mark.parametrize("S", [0, 1, 2, 3, 4, 7])
def test_plan_matches_oracle_enumeration(T, S):
    """P-11: the library's chunk and segment bounds equal the oracle's
    enumeration from the definition, bit for bit."""
    chunk, segs, _, bounds = kdn.kdn_diag_plan(2, 16, T, 128, 128, segments=S)
    _, _, ref = oracle.plan(T, chunk, segs)
    assert bounds == ref
    if S:
        assert segs == min(S, -(-T // chunk))


def test_plan_auto_segments_fill_the_chip():
    _, S1, _, _ = kdn.kdn_diag_plan(8, 16, 2048, 128, 128)
    _, S2, _, _ = kdn.kdn_diag_plan(2, 16, 16384, 128, 128)
    _, S3, _, _ = kdn.kdn_diag_plan(1, 2, 64, 16, 16)
    assert S1 == 1 and S2 == 4 and S3 == 1


def _bwd(B=1, H=1, T=8, dk=64, dv=16, dt=kdn.KDN_F32, ptr=FAKE, A=FAKE, I_prior=1.0, I0=None,
         mu0=None, d_o=FAKE, dI_T=None, dmu_T=None, outs=None, dA=FAKE, dIp=None, dI0=None,
         dmu0=None, ws=None, nbytes=None):
    o = outs if outs is not None else {}
    g = lambda n: o.get(n, FAKE)
    nb = None if nbytes is None else ctypes.byref(nbytes)
    return lib.kdn_diag_scan_bwd(B, H, T, dk, dv, dt, g("q") if "q" in o else ptr, ptr, ptr, ptr,
                                 ptr, A, I_prior, I0, mu0, d_o, dI_T, dmu_T, g("dq"), g("dk"),
                                 g("dv"), g("dbeta"), g("dd"), dA, dIp, dI0, dmu0, ws, nb, None)


def test_bwd_validation():
    n = ctypes.c_size_t(0)
    q = dict(nbytes=n)
    assert _bwd(**q) == kdn.KDN_OK
    assert _bwd(dk=32, **q) == kdn.KDN_EUNSUPPORTED      # the gradient needs d_k of 64 or 128
    assert _bwd(dk=16, **q) == kdn.KDN_EUNSUPPORTED
    assert _bwd(dv=24, **q) == kdn.KDN_EUNSUPPORTED
    assert _bwd(dk=128, dv=128, **q) == kdn.KDN_OK
    assert _bwd(B=-1, **q) == kdn.KDN_EINVAL
    assert _bwd(dt=5, **q) == kdn.KDN_EINVAL
    assert _bwd(I_prior=0.0, **q) == kdn.KDN_EINVAL
    assert _bwd(d_o=None, **q) == kdn.KDN_EINVAL
    assert _bwd(dA=None, **q) == kdn.KDN_EINVAL
    assert _bwd(A=MIS, **q) == kdn.KDN_EINVAL
    for name in ("dq", "dk", "dv", "dbeta", "dd"):
        assert _bwd(outs={name: None}, **q) == kdn.KDN_EINVAL, name
        assert _bwd(outs={name: MIS}, **q) == kdn.KDN_EINVAL, name
    # Palimpsa-M gating: no beta, so no dbeta (its share goes to dd)
    n2 = ctypes.c_size_t(0)
    call_m = lambda dbeta: lib.kdn_diag_scan_bwd(1, 1, 8, 64, 16, kdn.KDN_F32, FAKE, FAKE, FAKE, None,
                                                 FAKE, FAKE, 1.0, None, None, FAKE, None, None, FAKE,
                                                 FAKE, FAKE, dbeta, FAKE, FAKE, None, None, None,
                                                 None, ctypes.byref(n2), None)
    assert call_m(None) == kdn.KDN_OK
    assert call_m(FAKE) == kdn.KDN_EINVAL
    # state gradients need the state they differentiate
    assert _bwd(dI0=FAKE, **q) == kdn.KDN_EINVAL
    assert _bwd(dmu0=FAKE, **q) == kdn.KDN_EINVAL
    assert _bwd(I0=FAKE, mu0=FAKE, dI0=FAKE, dmu0=FAKE, dIp=FAKE, **q) == kdn.KDN_OK
    assert _bwd(I0=MIS, **q) == kdn.KDN_EINVAL
    assert _bwd(dI_T=MIS, **q) == kdn.KDN_EINVAL
    # an empty batch or sequence needs no token pointers
    assert _bwd(T=0, ptr=None, d_o=None, outs={n: None for n in ("dq", "dk", "dv", "dbeta", "dd")},
                **q) == kdn.KDN_OK
    assert _bwd(B=0, ptr=None, A=None, d_o=None, **q) == kdn.KDN_OK


def test_bwd_workspace():
    n = ctypes.c_size_t(0)
    assert _bwd(B=8, H=16, T=2048, dk=128, dv=128, nbytes=n) == kdn.KDN_OK
    BH, T, nch = 128, 2048, 128
    ckpt = 4 * BH * nch * 2 * 128 * 128
    rows = 2 * 4 * 2 * BH * T * 128        # two column tiles: dq and dk partials
    assert n.value >= 16 * BH * T + ckpt + rows and n.value % 256 == 0
    small = ctypes.c_size_t(n.value - 1)
    assert _bwd(B=8, H=16, T=2048, dk=128, dv=128, ws=FAKE, nbytes=small) == kdn.KDN_EWORKSPACE
    # one column tile: dq and dk are written directly, no row partials
    m = ctypes.c_size_t(0)
    assert _bwd(B=8, H=16, T=2048, dk=128, dv=64, nbytes=m) == kdn.KDN_OK
    assert m.value < 16 * BH * T + ckpt // 2 + rows // 2


def test_noise_validation():
    call = lambda B=1, H=1, T=8, dk=16, dv=16, dt=kdn.KDN_BF16, q=FAKE, a=FAKE, o=FAKE, lam0=None: \
        lib.kdn_diag_noise_scan_fwd(B, H, T, dk, dv, dt, q, FAKE, FAKE, FAKE, a, FAKE, lam0, None,
                                    o, None, None, None)
    assert call(B=-1) == kdn.KDN_EINVAL
    assert call(dk=24) == kdn.KDN_EUNSUPPORTED
    assert call(dt=9) == kdn.KDN_EINVAL
    assert call(q=None) == kdn.KDN_EINVAL
    assert call(a=MIS) == kdn.KDN_EINVAL
    assert call(o=None) == kdn.KDN_EINVAL
    assert call(lam0=MIS) == kdn.KDN_EINVAL
    assert call(B=0, q=None, a=None, o=None) == kdn.KDN_OK


def test_varlen_validation_and_workspace():
    n = ctypes.c_size_t(0)
    call = lambda N=3, H=2, T=40, dk=64, dv=64, cu=FAKE, q=FAKE, beta=FAKE, I0=None, nb=n, ws=None: \
        lib.kdn_diag_scan_varlen_fwd(N, H, T, dk, dv, kdn.KDN_BF16, cu, q, FAKE, FAKE, beta, FAKE,
                                     FAKE, 1.0, I0, None, FAKE, None, None, ws,
                                     None if nb is None else ctypes.byref(nb), None)
    assert call() == kdn.KDN_OK
    # frame scalars, then the plan's tables (order, item sequence, segment and
    # 32-byte record, first composite of each sequence, counts), 256 bytes
    # each at this size; 40 tokens cannot be split, so no composite tables or
    # states
    assert kdn.kdn_diag_varlen_plan(3, 2, 40, 64, 64) == (0, 1, 3, 0)
    assert n.value == 16 * 2 * 40 + 6 * 256
    assert call(N=-1) == kdn.KDN_EINVAL
    assert call(cu=None) == kdn.KDN_EINVAL
    assert call(cu=FAKE + 4) == kdn.KDN_EINVAL  # int64 offsets must be 8-byte aligned
    assert call(q=None) == kdn.KDN_EINVAL
    assert call(beta=None) == kdn.KDN_OK        # Palimpsa-M gating
    assert call(dk=24) == kdn.KDN_EUNSUPPORTED
    assert call(I0=MIS) == kdn.KDN_EINVAL
    assert call(N=0, cu=None) == kdn.KDN_OK and n.value == 0
    assert call(nb=None, ws=None) == kdn.KDN_EWORKSPACE


def test_varlen_split_plan():
    """The packed batch's split plan from the sizes: the fair share of the
    chip, H total_T tiles / 256 tokens, rounded up to 256, at least 512."""
    # 16 heads x 16384 tokens x 2 tiles: 2048 tokens a share, 8 composites at most
    seg, R, items, comps = kdn.kdn_diag_varlen_plan(64, 16, 16384, 128, 128)
    assert (seg, items, comps) == (2048, 72, 8)
    assert 1 <= R <= 2048 // 64 and R == min(8 * 256 // (8 * 16 * 4), 2048 // 64)
    # small batches: the 512-token floor
    assert kdn.kdn_diag_varlen_plan(4, 2, 3000, 64, 64)[:1] == (512,)
    assert kdn.kdn_diag_varlen_plan(4, 2, 3000, 64, 64)[2:] == (4 + 5, 5)
    # d_v < 64: one tile per head
    assert kdn.kdn_diag_varlen_plan(4, 64, 4096, 64, 32)[0] == 1024
    # no split requested, or nothing long enough to split
    assert kdn.kdn_diag_varlen_plan(64, 16, 16384, 128, 128, segments=1) == (0, 1, 64, 0)
    assert kdn.kdn_diag_varlen_plan(4, 2, 512, 64, 64) == (0, 1, 4, 0)
    seg = ctypes.c_int64(0)
    assert lib.kdn_diag_varlen_plan(4, 2, 512, 64, 64, 2, ctypes.byref(seg), None, None, None) \
        == kdn.KDN_EINVAL
    assert lib.kdn_diag_varlen_plan(4, 2, 512, 24, 64, 0, None, None, None, None) \
        == kdn.KDN_EUNSUPPORTED
    # the workspace grows by the composite tables and states when a split is possible
    n1, n2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    opts = kdn.ScanOpts()
    for segs, n in ((0, n1), (1, n2)):
        opts.segments = segs
        assert lib.kdn_diag_scan_varlen_fwd_ex(4, 2, 3000, 64, 64, kdn.KDN_F32, FAKE, FAKE, FAKE, FAKE,
                                               FAKE, FAKE, FAKE, 1.0, None, None, FAKE, None, None,
                                               ctypes.byref(opts), None, ctypes.byref(n), None) \
            == kdn.KDN_OK
    R = kdn.kdn_diag_varlen_plan(4, 2, 3000, 64, 64)[1]
    assert n1.value - n2.value >= 4 * 5 * 2 * (2 + 2 * R) * 64 * 64


def test_varlen_bwd_validation_and_workspace():
    n = ctypes.c_size_t(0)

    def call(N=3, H=2, T=40, dk=64, dv=64, dt=kdn.KDN_BF16, cu=FAKE, q=FAKE, beta=FAKE, dbeta=FAKE,
             d_o=FAKE, dA=FAKE, I0=None, mu0=None, dI0=None, dmu0=None, dq=FAKE, nb=n, ws=None):
        return lib.kdn_diag_scan_varlen_bwd(N, H, T, dk, dv, dt, cu, q, FAKE, FAKE, beta, FAKE, FAKE,
                                            1.0, I0, mu0, d_o, None, None, dq, FAKE, FAKE, dbeta, FAKE,
                                            dA, FAKE, dI0, dmu0, ws,
                                            None if nb is None else ctypes.byref(nb), None)

    assert call() == kdn.KDN_OK
    # frame scalars (16 B a token row) and checkpoints: every sequence of a
    # head holds ceil(len / 16) + 1 slots of 2 d_k d_v floats, at most
    # ceil(T / 16) + 2 N in all
    ckpt = 4 * 2 * (3 + 2 * 3) * 2 * 64 * 64
    assert n.value >= 16 * 2 * 40 + ckpt and n.value % 256 == 0
    full = n.value
    assert call(beta=None, dbeta=None) == kdn.KDN_OK and n.value > full  # Palimpsa-M: dbeta partials
    assert call(beta=None, dbeta=FAKE) == kdn.KDN_EINVAL
    assert call(dbeta=None) == kdn.KDN_EINVAL
    assert call(N=-1) == kdn.KDN_EINVAL
    assert call(dt=7) == kdn.KDN_EINVAL
    assert call(dk=32) == kdn.KDN_EUNSUPPORTED
    assert call(dv=24) == kdn.KDN_EUNSUPPORTED
    assert call(cu=None) == kdn.KDN_EINVAL
    assert call(cu=FAKE + 4) == kdn.KDN_EINVAL
    assert call(q=None) == kdn.KDN_EINVAL
    assert call(d_o=None) == kdn.KDN_EINVAL
    assert call(dA=None) == kdn.KDN_EINVAL
    assert call(dq=MIS) == kdn.KDN_EINVAL
    assert call(dI0=FAKE) == kdn.KDN_EINVAL                  # dI0 needs I0
    assert call(dmu0=FAKE) == kdn.KDN_EINVAL
    assert call(I0=FAKE, mu0=FAKE, dI0=FAKE, dmu0=FAKE) == kdn.KDN_OK
    assert call(I0=MIS) == kdn.KDN_EINVAL
    # no sequences: only the finishing sums (dA = 0, dI_prior = 0) are written
    assert call(N=0, cu=None, q=None, d_o=None, dq=None) == kdn.KDN_OK and 0 < n.value <= 256
    assert call(nb=None, ws=None) == kdn.KDN_EWORKSPACE
    small = ctypes.c_size_t(full - 1)
    assert call(nb=small, ws=FAKE) == kdn.KDN_EWORKSPACE

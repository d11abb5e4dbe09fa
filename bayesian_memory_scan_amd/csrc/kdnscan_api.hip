// kdnscan_api.hip -- the C ABI: argument validation, planning, workspace
// layout and kernel dispatch.  Validation completes before any HIP call.
#include "kdn_params.h"

#include <atomic>
#include <cmath>

namespace kdn {
namespace {
thread_local hipError_t g_last_error = hipSuccess;
}
void note_hip_error(hipError_t e) { g_last_error = e; }
}  // namespace kdn

namespace {

using namespace kdn;

// One dispatch covers at most 2^32 - 1 work-items (the dispatch packet's grid
// size is 32 bits).  Per-head and per-block launches use at most 512 threads
// per workgroup; element-wise passes walk with a grid stride and always fit.
constexpr int64_t kMaxItems = 4294967295;
constexpr int64_t kMaxGroupThreads = 512;
bool grid_fits(int64_t groups, int64_t threads = kMaxGroupThreads) {
    return groups >= 0 && groups <= kMaxItems / threads;
}
constexpr int32_t kMaxSegments = 64;

struct Plan {
    int32_t chunk;
    int32_t nchunks;
    int32_t S;
    int32_t R;   // sub-segments per segment for the composite pass (diagonal scan)
};

// Chunking and segment count of the diagonal scan; `request` is the
// caller's segment count (0: automatic).
Plan plan_scan(int64_t BH, int64_t T, int64_t dv, int32_t request) {
    Plan pl;
    pl.chunk = diag_chunk();
    pl.nchunks = static_cast<int32_t>((T + pl.chunk - 1) / pl.chunk);
    const int64_t ci = dv < 64 ? dv : 64;
    const int64_t units = BH * (dv / ci);
    int64_t S = 1;
    if (request > 0) {
        S = request;
    } else if (units > 0 && units < kNumCU && pl.nchunks >= 16) {
        S = (kNumCU + units - 1) / units;
        if (S > pl.nchunks / 8) S = pl.nchunks / 8;
    }
    if (S > kMaxSegments) S = kMaxSegments;
    if (S > pl.nchunks) S = pl.nchunks;
    if (S < 1) S = 1;
    pl.S = static_cast<int32_t>(S);
    // composites: about eight work units of 32 value columns per CU (one
    // wave each for fp32 inputs, two for bf16: a J wave's and an X wave's
    // share), at least 4 chunks per sub-segment
    int64_t R = 1;
    if (pl.S > 1 && BH > 0) {
        const int64_t units = BH * (pl.S - 1) * (dv > 32 ? dv / 32 : 1);
        R = 8 * kNumCU / units;
        const int64_t per_seg = pl.nchunks / pl.S;
        if (R > per_seg / 4) R = per_seg / 4;
        if (R < 1) R = 1;
    }
    pl.R = static_cast<int32_t>(R);
    return pl;
}

// Segments of the isotropic mean scan: about two one-wave workgroups per
// SIMD, at least four 16-token chunks per segment (or the caller's request).
Plan plan_iso(int64_t BH, int64_t T, int64_t dv, int32_t request) {
    Plan pl;
    pl.chunk = iso_chunk();
    pl.nchunks = static_cast<int32_t>((T + pl.chunk - 1) / pl.chunk);
    int64_t S = 1;
    if (request > 0) {
        S = request;
    } else if (BH > 0) {
        const int64_t units = BH * iso_tiles(dv);
        S = (8 * kNumCU + units - 1) / units;
        if (S > pl.nchunks / 4) S = pl.nchunks / 4;
    }
    if (S > kMaxSegments) S = kMaxSegments;
    if (S > pl.nchunks) S = pl.nchunks;
    if (S < 1) S = 1;
    pl.S = static_cast<int32_t>(S);
    return pl;
}

// Packed batch: the segment length of a split sequence and the sub-segments
// of each composite.  A sequence is split when it is longer than its fair
// share of the chip, ceil(H total_T tiles / CUs) tokens rounded up to a
// multiple of 256, and than kVarlenMinSeg; the request is 0 (automatic) or
// 1 (never split).  comps bounds the composite segments: a split sequence
// of len tokens has ceil(len / seg) - 1 <= len / seg of them, so all
// sequences together at most total_T / seg.  Sub-segments: about eight
// one-wave units (32 value columns) per CU over that bound, at least four
// chunks each.
constexpr int64_t kVarlenMinSeg = 512;
struct VarlenPlan {
    int64_t seg;     // 0: no sequence is split
    int32_t R;
    int64_t comps;   // capacity of the composite tables
    int64_t items;   // capacity of the item tables
    int64_t thr = 0; // sequences longer than thr are split (thr >= seg)
};
// Composite tables and sub-segments of a plan whose segment length is set.
static void plan_tables(VarlenPlan& v, int64_t N, int64_t H, int64_t total_T, int64_t dv) {
    v.comps = total_T / v.seg;
    v.items = N + v.comps;
    const int64_t units = v.comps * H * (dv > 32 ? dv / 32 : 1);
    int64_t R = 8 * kNumCU / units;
    if (R > v.seg / (4 * diag_chunk())) R = v.seg / (4 * diag_chunk());
    if (R < 1) R = 1;
    v.R = static_cast<int32_t>(R);
}

VarlenPlan plan_varlen(int64_t N, int64_t H, int64_t total_T, int64_t dv, int32_t request) {
    VarlenPlan v{0, 1, 0, N};
    if (request == 1 || N == 0 || H == 0) return v;
    const int64_t ntile = dv / varlen_cols(dv);
    const int64_t fair = (H * total_T * ntile + kNumCU - 1) / kNumCU;
    int64_t L = (fair + 255) / 256 * 256;
    if (L < kVarlenMinSeg) L = kVarlenMinSeg;
    if (total_T <= L) return v;
    v.seg = L;
    v.thr = L;
    plan_tables(v, N, H, total_T, dv);
    return v;
}

// The gradient's plan: the same split rule (sequences longer than a fair
// share), but the split sequences are cut into half-share segments.  Their
// checkpoint pass carries the adjoint composites at about three times the
// plain pass's cost per token, one workgroup per CU, so with fair-share
// segments a single long sequence fills only part of the chip for the
// whole pass; half-share segments give it twice the workgroups for half as
// long.  The reverse pass stays bound by the total work per CU.
VarlenPlan plan_varlen_bwd(int64_t N, int64_t H, int64_t total_T, int64_t dv) {
    VarlenPlan v = plan_varlen(N, H, total_T, dv, 0);
    if (v.seg >= 2 * kVarlenMinSeg) {
        v.seg = (v.seg / 2 + 255) / 256 * 256;
        plan_tables(v, N, H, total_T, dv);
    }
    return v;
}

// Workspace of a packed batch's forward scan, in this order.
struct VarlenWs {
    size_t scal, order, items, recs, seqcomp, comptab, nwork, comp, sub, gsub, total;
};
VarlenWs varlen_workspace(int64_t N, int64_t H, int64_t total_T, int64_t dk, int64_t dv,
                          const VarlenPlan& v) {
    VarlenWs w{};
    const size_t f = sizeof(float);
    w.scal = align_up(16 * static_cast<size_t>(H) * total_T, 256);
    w.order = align_up(4 * static_cast<size_t>(N), 256);
    w.items = align_up(4 * static_cast<size_t>(v.items), 256);          // each of item_seq, item_seg
    w.recs = align_up(sizeof(VarlenItemRec) * static_cast<size_t>(v.items), 256);
    w.seqcomp = align_up(4 * static_cast<size_t>(N), 256);
    w.comptab = v.comps > 0 ? align_up(4 * static_cast<size_t>(v.comps), 256) : 0;   // each of 3
    w.nwork = 256;
    const size_t units = static_cast<size_t>(v.comps) * H;
    w.comp = v.comps > 0 ? align_up(f * units * 2 * dk * dv, 256) : 0;
    w.sub = v.comps > 0 ? align_up(f * units * v.R * 2 * dk * dv, 256) : 0;
    w.gsub = v.comps > 0 ? align_up(f * units * v.R, 256) : 0;
    w.total = w.scal + w.order + 2 * w.items + w.recs + w.seqcomp + 3 * w.comptab + w.nwork + w.comp + w.sub + w.gsub;
    return w;
}

size_t scan_workspace_bytes(int64_t BH, int64_t dk, int64_t dv, const Plan& pl) {
    if (pl.S <= 1) return 0;
    const size_t comp = align_up(sizeof(float) * static_cast<size_t>(BH) * pl.S * 2 * dk * dv, 256);
    const size_t gdec = align_up(sizeof(float) * static_cast<size_t>(BH) * pl.S, 256);
    return comp + gdec;
}

// Diagonal scan: carry-in states + sub-segment composites and decays.
struct DiagWs {
    size_t scal, comp, sub, gsub, total;
};
DiagWs diag_workspace(int64_t BH, int64_t T, int64_t dk, int64_t dv, const Plan& pl) {
    DiagWs w{};
    w.scal = align_up(16 * static_cast<size_t>(BH) * T, 256);
    if (pl.S > 1) {
        const size_t nsub = static_cast<size_t>(BH) * (pl.S - 1) * pl.R;
        w.comp = align_up(sizeof(float) * static_cast<size_t>(BH) * pl.S * 2 * dk * dv, 256);
        w.sub = align_up(sizeof(float) * nsub * 2 * dk * dv, 256);
        w.gsub = align_up(sizeof(float) * nsub, 256);
    }
    w.total = w.scal + w.comp + w.sub + w.gsub;
    return w;
}

bool finite_positive(float x) { return std::isfinite(x) && x > 0.0f; }

bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

// Workspace protocol; returns KDN_OK to proceed, 1 for "query answered".
int workspace_check(void* workspace, size_t* workspace_bytes, size_t need) {
    if (workspace == nullptr && workspace_bytes != nullptr) {
        *workspace_bytes = need;
        return 1;
    }
    if (need == 0) return KDN_OK;
    if (workspace == nullptr || workspace_bytes == nullptr || *workspace_bytes < need) {
        if (workspace_bytes) *workspace_bytes = need;
        return KDN_EWORKSPACE;
    }
    if (!aligned16(workspace)) return KDN_EINVAL;
    return KDN_OK;
}

// Options of an extended call: a NULL pointer is the zero struct.  Checks
// what the call can check (segment request, echo buffer) before any HIP call.
bool opts_ok(const kdn_scan_opts* o) {
    if (o == nullptr) return true;
    if (o->segments < 0 || o->echo_capacity < 0) return false;
    if (o->bounds_echo != nullptr && (reinterpret_cast<uintptr_t>(o->bounds_echo) & 7u) != 0) return false;
    return true;
}
int32_t opt_segments(const kdn_scan_opts* o) { return o ? o->segments : 0; }
void apply_opts(DiagParams& p, const kdn_scan_opts* o) {
    if (o == nullptr) return;
    if (o->bounds_echo) {
        p.echo = o->bounds_echo;
        p.echo_cap = o->echo_capacity;
    }
    p.main_begin = o->main_begin;
    p.main_end = o->main_end;
}
void report_echo(kdn_scan_opts* o, int64_t records) {
    if (o) o->echo_words = records * KDN_ECHO_WORDS;
}

// Guard against overflow: B*H*T*D must stay < 2^62 (int64 element counts)
// and T below 2^31 (chunk and block counts are int32).
bool sizes_fit(int64_t B, int64_t H, int64_t T, int64_t D) {
    if (T > 2147483647) return false;
    const double n = static_cast<double>(B) * static_cast<double>(H) * static_cast<double>(T > 0 ? T : 1) *
                     static_cast<double>(D);
    return n < 4.0e18;
}

// The no-allocation entry's scratch: one array per GPU, reserved when the
// code object is loaded.  Host code must not use the array's name as a
// device address (it is a host-side stand-in): scratch_on_current_device
// returns the device address, looked up once per device with that device
// current and kept.
constexpr size_t kScratchBytes = KDN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        note_hip_error(e);
        return KDN_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return KDN_EUNSUPPORTED;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        // threads racing here look up the same address; any of them may store it
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            note_hip_error(e);
            return KDN_EHIP;
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return KDN_OK;
}

// The diagonal forward call.  fixed_scratch: the no-allocation entry, whose
// workspace is this GPU's scratch array (sub-segments reduced to fit it).
int diag_fwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v, kdn_dtype in_dtype,
             const void* q, const void* k, const void* v, const void* beta, const void* d,
             const float* A, float I_prior, const float* I0, const float* mu0,
             float* o, float* I_T, float* mu_T, kdn_scan_opts* opts,
             void* workspace, size_t* workspace_bytes, void* stream, bool fixed_scratch) {
    if (B < 0 || H < 0 || T < 0 || !opts_ok(opts)) return KDN_EINVAL;
    if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDN_EUNSUPPORTED;
    if (!finite_positive(I_prior)) return KDN_EINVAL;
    if (!sizes_fit(B, H, T, d_k > d_v ? d_k : d_v)) return KDN_EINVAL;
    const int64_t BH = B * H;
    if (BH > 0 && !ok_ptr(A)) return KDN_EINVAL;
    if (BH > 0 && T > 0) {
        if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_opt(beta) || !ok_ptr(d) || !ok_ptr(o))
            return KDN_EINVAL;
    }
    if (!ok_opt(I0) || !ok_opt(mu0) || !ok_opt(I_T) || !ok_opt(mu_T)) return KDN_EINVAL;

    Plan pl = plan_scan(BH, T, d_v, opt_segments(opts));
    const int64_t ntile = d_v / (d_v < 64 ? d_v : 64);
    if (!grid_fits(BH * pl.S * ntile)) return KDN_EINVAL;
    // composite pass: one wave per (head, sub-segment, column tile of 16 or 32)
    if (pl.S > 1 && !grid_fits(BH * (pl.S - 1) * pl.R * (d_v / 16), kWave)) return KDN_EINVAL;
    DiagWs dw = diag_workspace(BH, T, d_k, d_v, pl);
    size_t scratch_cap = 0;
    if (fixed_scratch) {
        while (dw.total > kScratchBytes && pl.S > 1 && pl.R > 1) {
            --pl.R;
            dw = diag_workspace(BH, T, d_k, d_v, pl);
        }
        if (dw.total > kScratchBytes) return KDN_ESCRATCH;
        if (BH > 0 && dw.total > 0) {
            const int rc = scratch_on_current_device(&workspace);
            if (rc != KDN_OK) return rc;
            scratch_cap = kScratchBytes;
            workspace_bytes = &scratch_cap;
        }
    }
    report_echo(opts, T > 0 ? BH * pl.S * ntile + (pl.S > 1 ? BH * (pl.S - 1) * pl.R * comp_tiles(d_k, d_v, in_dtype == KDN_BF16) : 0) : 0);
    const size_t need = dw.total;
    const int wc = workspace_check(workspace, workspace_bytes, need);
    if (wc == 1) return KDN_OK;
    if (wc != KDN_OK) return wc;
    if (BH == 0) return KDN_OK;

    DiagParams p{};
    p.q = q; p.k = k; p.v = v; p.beta = beta; p.d = d;
    p.A = A; p.I0 = I0; p.mu0 = mu0;
    p.o = o; p.I_T = I_T; p.mu_T = mu_T;
    char* ws = static_cast<char*>(workspace);
    p.scal = reinterpret_cast<float4*>(ws);
    if (pl.S > 1) {
        p.comp = reinterpret_cast<float*>(ws + dw.scal);
        p.sub = reinterpret_cast<float*>(ws + dw.scal + dw.comp);
        p.gsub = reinterpret_cast<float*>(ws + dw.scal + dw.comp + dw.sub);
    }
    p.H = H; p.T = T; p.dv = d_v; p.I_prior = I_prior;
    p.S = pl.S; p.nchunks = pl.nchunks;
    apply_opts(p, opts);
    (void)hipGetLastError();  // launch status below must reflect this call only
    return diag_scan_launch(p, B, d_k, in_dtype == KDN_BF16, pl.R, static_cast<hipStream_t>(stream));
}


}  // namespace

extern "C" {

const char* kdn_status_string(int status) {
    switch (status) {
        case KDN_OK: return "ok";
        case KDN_EINVAL: return "invalid argument (size, NULL pointer, alignment or I_prior)";
        case KDN_EUNSUPPORTED: return "unsupported configuration (d_k and d_v must be 16, 32, 64 or 128)";
        case KDN_EWORKSPACE: return "workspace missing or too small";
        case KDN_EHIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* kdn_last_hip_error(void) {
    return hipGetErrorString(g_last_error);
}

int kdn_diag_plan(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v, int32_t segments,
                  int32_t* chunk, int32_t* segments_out, int32_t* subsegments,
                  int64_t* seg_bounds, int32_t max_segments) {
    if (B < 0 || H < 0 || T < 0 || segments < 0) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDN_EUNSUPPORTED;
    if (!sizes_fit(B, H, T, d_k > d_v ? d_k : d_v)) return KDN_EINVAL;
    const Plan pl = plan_scan(B * H, T, d_v, segments);
    if (chunk) *chunk = pl.chunk;
    if (segments_out) *segments_out = pl.S;
    if (subsegments) *subsegments = pl.R;
    if (seg_bounds) {
        if (max_segments < pl.S) return KDN_EINVAL;
        for (int32_t s = 0; s <= pl.S; ++s) {
            const int64_t c = static_cast<int64_t>(s) * pl.nchunks / pl.S;
            const int64_t t = c * pl.chunk;
            seg_bounds[s] = t < T ? t : T;
        }
    }
    return KDN_OK;
}

int kdn_diag_scan_fwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                      kdn_dtype in_dtype,
                      const void* q, const void* k, const void* v,
                      const void* beta, const void* d,
                      const float* A, float I_prior,
                      const float* I0, const float* mu0,
                      float* o, float* I_T, float* mu_T,
                      void* workspace, size_t* workspace_bytes, void* stream) {
    return diag_fwd(B, H, T, d_k, d_v, in_dtype, q, k, v, beta, d, A, I_prior, I0, mu0, o, I_T, mu_T,
                    nullptr, workspace, workspace_bytes, stream, false);
}

int kdn_diag_scan_fwd_ex(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                         kdn_dtype in_dtype,
                         const void* q, const void* k, const void* v,
                         const void* beta, const void* d,
                         const float* A, float I_prior,
                         const float* I0, const float* mu0,
                         float* o, float* I_T, float* mu_T, kdn_scan_opts* opts,
                         void* workspace, size_t* workspace_bytes, void* stream) {
    return diag_fwd(B, H, T, d_k, d_v, in_dtype, q, k, v, beta, d, A, I_prior, I0, mu0, o, I_T, mu_T,
                    opts, workspace, workspace_bytes, stream, false);
}

int kdn_diag_scan_fwd_noalloc(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                              kdn_dtype in_dtype,
                              const void* q, const void* k, const void* v,
                              const void* beta, const void* d,
                              const float* A, float I_prior,
                              const float* I0, const float* mu0,
                              float* o, float* I_T, float* mu_T, void* stream) {
    return diag_fwd(B, H, T, d_k, d_v, in_dtype, q, k, v, beta, d, A, I_prior, I0, mu0, o, I_T, mu_T,
                    nullptr, nullptr, nullptr, stream, true);
}

int kdn_diag_scan_varlen_fwd(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                             kdn_dtype in_dtype, const int64_t* cu_seqlens,
                             const void* q, const void* k, const void* v,
                             const void* beta, const void* d,
                             const float* A, float I_prior,
                             const float* I0, const float* mu0,
                             float* o, float* I_T, float* mu_T,
                             void* workspace, size_t* workspace_bytes, void* stream) {
    return kdn_diag_scan_varlen_fwd_ex(N, H, total_T, d_k, d_v, in_dtype, cu_seqlens, q, k, v, beta, d, A,
                                       I_prior, I0, mu0, o, I_T, mu_T, nullptr, workspace,
                                       workspace_bytes, stream);
}

int kdn_diag_scan_varlen_fwd_ex(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                                kdn_dtype in_dtype, const int64_t* cu_seqlens,
                                const void* q, const void* k, const void* v,
                                const void* beta, const void* d,
                                const float* A, float I_prior,
                                const float* I0, const float* mu0,
                                float* o, float* I_T, float* mu_T, kdn_scan_opts* opts,
                                void* workspace, size_t* workspace_bytes, void* stream) {
    if (N < 0 || H < 0 || total_T < 0 || N >= 2147483647 || !opts_ok(opts)) return KDN_EINVAL;
    if (opt_segments(opts) > 1) return KDN_EINVAL;
    if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDN_EUNSUPPORTED;
    if (!finite_positive(I_prior)) return KDN_EINVAL;
    if (!sizes_fit(1, H, total_T, d_k > d_v ? d_k : d_v) || !sizes_fit(N, H, 1, d_k * d_v)) return KDN_EINVAL;
    const bool work = N > 0 && H > 0;
    const VarlenPlan vp = plan_varlen(N, H, total_T, d_v, opt_segments(opts));
    if (vp.items >= 2147483647) return KDN_EINVAL;
    if (work && (cu_seqlens == nullptr || (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) != 0))
        return KDN_EINVAL;
    if (work && !ok_ptr(A)) return KDN_EINVAL;
    if (H > 0 && total_T > 0) {
        if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_opt(beta) || !ok_ptr(d) || !ok_ptr(o))
            return KDN_EINVAL;
    }
    if (!ok_opt(I0) || !ok_opt(mu0) || !ok_opt(I_T) || !ok_opt(mu_T)) return KDN_EINVAL;
    const int64_t main_grid = varlen_main_grid(vp.items, H, d_v);
    const int64_t comp_grid = vp.comps * H * vp.R * comp_tiles(d_k, d_v, in_dtype == KDN_BF16);
    if (!grid_fits(main_grid) || !grid_fits(comp_grid)) return KDN_EINVAL;
    report_echo(opts, work ? main_grid + comp_grid : 0);
    const VarlenWs w = varlen_workspace(N, H, total_T, d_k, d_v, vp);
    const size_t need = work ? w.total : 0;
    const int wc = workspace_check(workspace, workspace_bytes, need);
    if (wc == 1) return KDN_OK;
    if (wc != KDN_OK) return wc;
    if (!work) return KDN_OK;

    DiagParams p{};
    p.q = q; p.k = k; p.v = v; p.beta = beta; p.d = d;
    p.A = A; p.I0 = I0; p.mu0 = mu0;
    p.o = o; p.I_T = I_T; p.mu_T = mu_T;
    char* ws = static_cast<char*>(workspace);
    p.scal = reinterpret_cast<float4*>(ws);
    ws += w.scal;
    p.seq_order = reinterpret_cast<int32_t*>(ws);
    ws += w.order;
    p.item_seq = reinterpret_cast<int32_t*>(ws);
    ws += w.items;
    p.item_seg = reinterpret_cast<int32_t*>(ws);
    ws += w.items;
    p.items = reinterpret_cast<VarlenItemRec*>(ws);
    ws += w.recs;
    p.seq_comp = reinterpret_cast<int32_t*>(ws);
    ws += w.seqcomp;
    if (vp.comps > 0) {
        p.comp_seq = reinterpret_cast<int32_t*>(ws);
        p.comp_seg = reinterpret_cast<int32_t*>(ws + w.comptab);
        p.split_seq = reinterpret_cast<int32_t*>(ws + 2 * w.comptab);
        ws += 3 * w.comptab;
    }
    p.nwork = reinterpret_cast<int32_t*>(ws);
    ws += w.nwork;
    if (vp.comps > 0) {
        p.comp = reinterpret_cast<float*>(ws);
        p.sub = reinterpret_cast<float*>(ws + w.comp);
        p.gsub = reinterpret_cast<float*>(ws + w.comp + w.sub);
    }
    p.H = H; p.T = total_T; p.dv = d_v; p.I_prior = I_prior;
    p.S = 1; p.nchunks = 0;
    p.cu_seqlens = cu_seqlens; p.nseq = static_cast<int32_t>(N);
    p.vl_seg = vp.seg; p.vl_thr = vp.thr; p.vl_items = vp.items; p.vl_comps = vp.comps;
    apply_opts(p, opts);
    (void)hipGetLastError();  // launch status below must reflect this call only
    return diag_varlen_launch(p, d_k, in_dtype == KDN_BF16, vp.R, static_cast<hipStream_t>(stream));
}

int kdn_diag_varlen_plan(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                         int32_t segments, int64_t* seg_tokens, int32_t* subsegments,
                         int64_t* max_items, int64_t* max_composites) {
    if (N < 0 || H < 0 || total_T < 0 || N >= 2147483647) return KDN_EINVAL;
    if (segments < 0 || segments > 1) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDN_EUNSUPPORTED;
    const VarlenPlan vp = plan_varlen(N, H, total_T, d_v, segments);
    if (seg_tokens) *seg_tokens = vp.seg;
    if (subsegments) *subsegments = vp.R;
    if (max_items) *max_items = vp.items;
    if (max_composites) *max_composites = vp.comps;
    return KDN_OK;
}

int kdn_diag_noise_scan_fwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                            kdn_dtype in_dtype,
                            const void* q, const void* k, const void* v, const void* beta,
                            const float* a, const float* p,
                            const float* lambda0, const float* mu0,
                            float* o, float* lambda_T, float* mu_T, void* stream) {
    if (B < 0 || H < 0 || T < 0) return KDN_EINVAL;
    if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDN_EUNSUPPORTED;
    if (!sizes_fit(B, H, T, d_k > d_v ? d_k : d_v)) return KDN_EINVAL;
    const int64_t BH = B * H;
    if (BH > 0 && T > 0) {
        if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(beta) || !ok_ptr(a) || !ok_ptr(p) ||
            !ok_ptr(o))
            return KDN_EINVAL;
    }
    if (!ok_opt(lambda0) || !ok_opt(mu0) || !ok_opt(lambda_T) || !ok_opt(mu_T)) return KDN_EINVAL;
    const int64_t ntile = d_v / (d_v < 64 ? d_v : 64);
    if (!grid_fits(BH * ntile)) return KDN_EINVAL;
    if (BH == 0) return KDN_OK;
    NoiseParams np{};
    np.q = q; np.k = k; np.v = v; np.beta = beta; np.a = a; np.p = p;
    np.lam0 = lambda0; np.mu0 = mu0; np.o = o; np.lam_T = lambda_T; np.mu_T = mu_T;
    np.H = H; np.T = T; np.dv = d_v;
    (void)hipGetLastError();  // launch status below must reflect this call only
    return noise_launch(np, B, d_k, in_dtype == KDN_BF16, static_cast<hipStream_t>(stream));
}

int kdn_diag_scan_bwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                      kdn_dtype in_dtype,
                      const void* q, const void* k, const void* v,
                      const void* beta, const void* d,
                      const float* A, float I_prior,
                      const float* I0, const float* mu0,
                      const float* d_o, const float* d_I_T, const float* d_mu_T,
                      float* dq, float* dk, float* dv, float* dbeta, float* dd,
                      float* dA, float* dI_prior, float* dI0, float* dmu0,
                      void* workspace, size_t* workspace_bytes, void* stream) {
    return kdn_diag_scan_bwd_ex(B, H, T, d_k, d_v, in_dtype, q, k, v, beta, d, A, I_prior, I0, mu0, d_o,
                                d_I_T, d_mu_T, dq, dk, dv, dbeta, dd, dA, dI_prior, dI0, dmu0, nullptr,
                                workspace, workspace_bytes, stream);
}

int kdn_diag_scan_bwd_ex(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                         kdn_dtype in_dtype,
                         const void* q, const void* k, const void* v,
                         const void* beta, const void* d,
                         const float* A, float I_prior,
                         const float* I0, const float* mu0,
                         const float* d_o, const float* d_I_T, const float* d_mu_T,
                         float* dq, float* dk, float* dv, float* dbeta, float* dd,
                         float* dA, float* dI_prior, float* dI0, float* dmu0, kdn_scan_opts* opts,
                         void* workspace, size_t* workspace_bytes, void* stream) {
    if (B < 0 || H < 0 || T < 0 || !opts_ok(opts)) return KDN_EINVAL;
    // the gradient takes the segment request only
    if (opts && (opts->bounds_echo || opts->main_begin || opts->main_end)) return KDN_EINVAL;
    if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v) || d_k < 64) return KDN_EUNSUPPORTED;
    if (!finite_positive(I_prior)) return KDN_EINVAL;
    if (!sizes_fit(B, H, T, d_k > d_v ? d_k : d_v)) return KDN_EINVAL;
    const int64_t BH = B * H;
    if (H > 0 && !ok_ptr(dA)) return KDN_EINVAL;
    if (BH > 0 && !ok_ptr(A)) return KDN_EINVAL;
    if (BH > 0 && T > 0) {
        if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_opt(beta) || !ok_ptr(d) || !ok_ptr(d_o))
            return KDN_EINVAL;
        if (!ok_ptr(dq) || !ok_ptr(dk) || !ok_ptr(dv) || !ok_ptr(dd)) return KDN_EINVAL;
        // Palimpsa-M gating (beta == NULL) has no beta to differentiate
        if (beta ? !ok_ptr(dbeta) : dbeta != nullptr) return KDN_EINVAL;
    }
    if (!ok_opt(I0) || !ok_opt(mu0) || !ok_opt(d_I_T) || !ok_opt(d_mu_T)) return KDN_EINVAL;
    if (!ok_opt(dI_prior) || !ok_opt(dI0) || !ok_opt(dmu0)) return KDN_EINVAL;
    if ((dI0 && !I0) || (dmu0 && !mu0)) return KDN_EINVAL;

    const int64_t ci = d_v < 64 ? d_v : 64;
    const int64_t ntile = d_v / ci;
    const int64_t nch = (T + diag_chunk() - 1) / diag_chunk();
    // Rows too few to fill the chip are cut into segments, planned as the
    // forward scan plans them (same segment bounds, so the forward composites
    // give each segment's starting state).
    const Plan pl = plan_scan(BH, T, d_v, opt_segments(opts));
    const int64_t S = pl.S;
    if (!grid_fits(BH * S * ntile)) return KDN_EINVAL;
    report_echo(opts, 0);
    const size_t f = sizeof(float);
    const size_t b_scal = align_up(16 * static_cast<size_t>(BH) * T, 256);
    const size_t b_ckpt = align_up(f * static_cast<size_t>(BH) * (nch + 1) * 2 * d_k * d_v, 256);
    const size_t b_rows = ntile > 1 ? align_up(f * static_cast<size_t>(ntile) * BH * T * d_k, 256) : 0;
    const size_t b_tok = align_up(f * static_cast<size_t>(ntile) * BH * T, 256);
    const size_t b_dip0 = align_up(f * static_cast<size_t>(ntile) * BH, 256);
    const int32_t split = bwd_token_split(BH, T);
    const size_t b_head = align_up(f * 2 * static_cast<size_t>(BH) * split, 256);
    const size_t b_db = beta ? 0 : b_tok;
    // segments: forward composites (carry-ins, sub-segment composites), the
    // adjoint composites and carried adjoints, and the segments' decays
    const DiagWs dw = diag_workspace(BH, T, d_k, d_v, pl);
    const size_t b_seg = S > 1 ? align_up(f * static_cast<size_t>(BH) * S * 2 * d_k * d_v, 256) : 0;
    const size_t b_adjg = S > 1 ? align_up(f * static_cast<size_t>(BH) * S, 256) : 0;
    const size_t b_fwd = S > 1 ? dw.comp + dw.sub + dw.gsub : 0;
    const size_t need = b_scal + b_ckpt + 2 * b_rows + 2 * b_tok + b_dip0 + b_head + b_db + b_fwd +
                        2 * b_seg + b_adjg;
    const int wc = workspace_check(workspace, workspace_bytes, need);
    if (wc == 1) return KDN_OK;
    if (wc != KDN_OK) return wc;
    if (H == 0) return KDN_OK;

    char* ws = static_cast<char*>(workspace);
    float4* scal = nullptr;
    BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.beta = beta; p.d = d;
    p.A = A; p.I0 = I0; p.mu0 = mu0;
    p.dout = d_o; p.dI_T = d_I_T; p.dmu_T = d_mu_T;
    p.dv_out = dv; p.dbeta = dbeta; p.dd = dd; p.dA = dA; p.dI_prior = dI_prior;
    p.dI0 = dI0; p.dmu0 = dmu0; p.dq = dq; p.dk = dk;
    if (BH > 0) {
        scal = reinterpret_cast<float4*>(ws);
        p.scal = scal;
        ws += b_scal;
        p.ckpt = reinterpret_cast<float*>(ws);
        ws += b_ckpt;
        if (ntile > 1) {
            p.part_dq = reinterpret_cast<float*>(ws);
            p.part_dk = reinterpret_cast<float*>(ws + b_rows);
            ws += 2 * b_rows;
        } else {
            p.part_dq = dq;
            p.part_dk = dk;
        }
        p.part_da = reinterpret_cast<float*>(ws);
        p.part_dip = reinterpret_cast<float*>(ws + b_tok);
        ws += 2 * b_tok;
        p.part_dip0 = reinterpret_cast<float*>(ws);
        ws += b_dip0;
        p.part_head = reinterpret_cast<float*>(ws);
        ws += b_head;
        if (!beta) p.part_db = reinterpret_cast<float*>(ws);
        ws += b_db;
    }
    p.BH = BH; p.H = H; p.T = T; p.dv = d_v; p.I_prior = I_prior;
    p.nchunks = static_cast<int32_t>(nch); p.ntile = static_cast<int32_t>(ntile);
    p.nruns = BH; p.tok_split = split;
    p.S = static_cast<int32_t>(S);

    DiagParams prep{};
    prep.k = k; prep.v = v; prep.beta = beta; prep.d = d; prep.A = A; prep.scal = scal;
    prep.I0 = I0; prep.mu0 = mu0;
    prep.H = H; prep.T = T; prep.dv = d_v; prep.I_prior = I_prior;
    prep.S = 1; prep.nchunks = static_cast<int32_t>(nch);
    if (BH > 0 && S > 1) {
        prep.S = static_cast<int32_t>(S);
        prep.comp = reinterpret_cast<float*>(ws);
        prep.sub = reinterpret_cast<float*>(ws + dw.comp);
        prep.gsub = reinterpret_cast<float*>(ws + dw.comp + dw.sub);
        ws += b_fwd;
        p.comp = prep.comp;
        p.adj = reinterpret_cast<float*>(ws);
        p.lam = reinterpret_cast<float*>(ws + b_seg);
        p.adjg = reinterpret_cast<float*>(ws + 2 * b_seg);
    }
    (void)hipGetLastError();  // launch status below must reflect this call only
    return diag_bwd_launch(p, prep, B, d_k, in_dtype == KDN_BF16, pl.R, static_cast<hipStream_t>(stream));
}

int kdn_diag_scan_varlen_bwd(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                             kdn_dtype in_dtype, const int64_t* cu_seqlens,
                             const void* q, const void* k, const void* v,
                             const void* beta, const void* d,
                             const float* A, float I_prior,
                             const float* I0, const float* mu0,
                             const float* d_o, const float* d_I_T, const float* d_mu_T,
                             float* dq, float* dk, float* dv, float* dbeta, float* dd,
                             float* dA, float* dI_prior, float* dI0, float* dmu0,
                             void* workspace, size_t* workspace_bytes, void* stream) {
    if (N < 0 || H < 0 || total_T < 0 || N >= 2147483647) return KDN_EINVAL;
    if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v) || d_k < 64) return KDN_EUNSUPPORTED;
    if (!finite_positive(I_prior)) return KDN_EINVAL;
    if (!sizes_fit(1, H, total_T, d_k > d_v ? d_k : d_v)) return KDN_EINVAL;
    if (!sizes_fit(N, H, 1, d_k * d_v)) return KDN_EINVAL;
    if (H > 0 && !ok_ptr(dA)) return KDN_EINVAL;
    const bool work = N > 0 && H > 0;
    if (work) {
        if (!ok_ptr(A) || !ok_ptr(cu_seqlens)) return KDN_EINVAL;
        if (total_T > 0) {
            if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_opt(beta) || !ok_ptr(d) || !ok_ptr(d_o))
                return KDN_EINVAL;
            if (!ok_ptr(dq) || !ok_ptr(dk) || !ok_ptr(dv) || !ok_ptr(dd)) return KDN_EINVAL;
            if (beta ? !ok_ptr(dbeta) : dbeta != nullptr) return KDN_EINVAL;
        }
    }
    if (!ok_opt(I0) || !ok_opt(mu0) || !ok_opt(d_I_T) || !ok_opt(d_mu_T)) return KDN_EINVAL;
    if (!ok_opt(dI_prior) || !ok_opt(dI0) || !ok_opt(dmu0)) return KDN_EINVAL;
    if ((dI0 && !I0) || (dmu0 && !mu0)) return KDN_EINVAL;

    const int64_t ci = d_v < 64 ? d_v : 64;
    const int64_t ntile = d_v / ci;
    const int64_t C = diag_chunk();
    // checkpoint slots per (head, column tile): every sequence holds
    // ceil(len / C) + 1, at most total_T / C + 2 N in all
    const int64_t ck_stride = (total_T + C - 1) / C + 2 * N;
    if (!grid_fits(((N * H + 7) / 8 * 8) * ntile)) return KDN_EINVAL;
    const size_t f = sizeof(float);
    const size_t rows = static_cast<size_t>(H) * total_T;
    const size_t b_scal = align_up(16 * rows, 256);
    const size_t b_order = align_up(4 * static_cast<size_t>(N), 256);
    const size_t b_ckoff = align_up(8 * static_cast<size_t>(N), 256);
    const size_t b_ckpt = align_up(f * static_cast<size_t>(H) * ck_stride * 2 * d_k * d_v, 256);
    const size_t b_rows = ntile > 1 ? align_up(f * static_cast<size_t>(ntile) * rows * d_k, 256) : 0;
    const size_t b_tok = align_up(f * static_cast<size_t>(ntile) * rows, 256);
    const size_t b_dip0 = align_up(f * static_cast<size_t>(ntile) * N * H, 256);
    const int32_t split = bwd_token_split(H, work ? total_T : 0);
    const size_t b_head = align_up(f * 2 * static_cast<size_t>(H) * split, 256);
    const size_t b_db = beta ? 0 : b_tok;
    // sequences longer than a fair share run in segments (the forward plan of
    // kdn_diag_varlen_plan): its tables and composites, plus per item the
    // adjoint composite and carried adjoint (adj, lam) and the decay (adjg)
    const VarlenPlan vp = work ? plan_varlen_bwd(N, H, total_T, d_v) : VarlenPlan{0, 1, 0, N};
    if (vp.items >= 2147483647 || !grid_fits((vp.items * H + 7) / 8 * 8 * ntile)) return KDN_EINVAL;
    const VarlenWs vw = varlen_workspace(N, H, total_T, d_k, d_v, vp);
    const size_t b_item = align_up(f * static_cast<size_t>(vp.items) * H * 2 * d_k * d_v, 256);
    const size_t b_itemg = align_up(f * static_cast<size_t>(vp.items) * H, 256);
    const size_t b_split = vp.seg > 0 ? 2 * vw.items + vw.recs + 2 * vw.seqcomp + 3 * vw.comptab + vw.nwork +
                                            vw.comp + vw.sub + vw.gsub + 2 * b_item + b_itemg
                                      : 0;
    const size_t need = work ? b_scal + b_order + b_ckoff + b_ckpt + 2 * b_rows + 2 * b_tok + b_dip0 + b_head + b_db +
                                   b_split
                             : b_head;
    const int wc = workspace_check(workspace, workspace_bytes, need);
    if (wc == 1) return KDN_OK;
    if (wc != KDN_OK) return wc;
    if (H == 0) return KDN_OK;

    char* ws = static_cast<char*>(workspace);
    BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.beta = beta; p.d = d;
    p.A = A; p.I0 = I0; p.mu0 = mu0;
    p.dout = d_o; p.dI_T = d_I_T; p.dmu_T = d_mu_T;
    p.dv_out = dv; p.dbeta = dbeta; p.dd = dd; p.dA = dA; p.dI_prior = dI_prior;
    p.dI0 = dI0; p.dmu0 = dmu0; p.dq = dq; p.dk = dk;
    p.BH = H; p.H = H; p.T = work ? total_T : 0; p.dv = d_v; p.I_prior = I_prior;
    p.nchunks = 0; p.ntile = static_cast<int32_t>(ntile);
    p.cu_seqlens = cu_seqlens; p.nseq = static_cast<int32_t>(N);
    p.nruns = N * H; p.ck_stride = ck_stride; p.tok_split = split; p.S = 1;
    DiagParams prep{};
    if (work) {
        float4* scal = reinterpret_cast<float4*>(ws);
        p.scal = scal;
        ws += b_scal;
        p.seq_order = reinterpret_cast<int32_t*>(ws);
        ws += b_order;
        p.seq_ckoff = reinterpret_cast<int64_t*>(ws);
        ws += b_ckoff;
        p.ckpt = reinterpret_cast<float*>(ws);
        ws += b_ckpt;
        if (ntile > 1) {
            p.part_dq = reinterpret_cast<float*>(ws);
            p.part_dk = reinterpret_cast<float*>(ws + b_rows);
            ws += 2 * b_rows;
        } else {
            p.part_dq = dq;
            p.part_dk = dk;
        }
        p.part_da = reinterpret_cast<float*>(ws);
        p.part_dip = reinterpret_cast<float*>(ws + b_tok);
        ws += 2 * b_tok;
        p.part_dip0 = reinterpret_cast<float*>(ws);
        ws += b_dip0;
        if (!beta) p.part_db = reinterpret_cast<float*>(ws + b_head);
        prep.d = d; prep.A = A; prep.scal = scal;
        prep.H = H; prep.T = total_T; prep.dv = d_v; prep.I_prior = I_prior;
        prep.S = 1; prep.cu_seqlens = cu_seqlens; prep.nseq = static_cast<int32_t>(N);
        if (vp.seg > 0) {
            char* w = ws + b_head + b_db;
            auto take = [&](size_t n) { char* x = w; w += n; return x; };
            prep.k = k; prep.v = v; prep.beta = beta; prep.I0 = I0; prep.mu0 = mu0;
            prep.seq_order = p.seq_order;
            prep.item_seq = reinterpret_cast<int32_t*>(take(vw.items));
            prep.item_seg = reinterpret_cast<int32_t*>(take(vw.items));
            prep.items = reinterpret_cast<VarlenItemRec*>(take(vw.recs));
            prep.seq_comp = reinterpret_cast<int32_t*>(take(vw.seqcomp));
            prep.seq_item = reinterpret_cast<int32_t*>(take(vw.seqcomp));
            if (vp.comps > 0) {
                prep.comp_seq = reinterpret_cast<int32_t*>(take(vw.comptab));
                prep.comp_seg = reinterpret_cast<int32_t*>(take(vw.comptab));
                prep.split_seq = reinterpret_cast<int32_t*>(take(vw.comptab));
            }
            prep.nwork = reinterpret_cast<int32_t*>(take(vw.nwork));
            if (vp.comps > 0) {
                prep.comp = reinterpret_cast<float*>(take(vw.comp));
                prep.sub = reinterpret_cast<float*>(take(vw.sub));
                prep.gsub = reinterpret_cast<float*>(take(vw.gsub));
            }
            prep.vl_seg = vp.seg; prep.vl_thr = vp.thr; prep.vl_items = vp.items; prep.vl_comps = vp.comps;
            p.item_seq = prep.item_seq; p.item_seg = prep.item_seg; p.seq_item = prep.seq_item;
            p.seq_comp = prep.seq_comp; p.split_seq = prep.split_seq; p.nwork = prep.nwork;
            p.comp = prep.comp;
            p.vl_seg = vp.seg; p.vl_thr = vp.thr; p.vl_items = vp.items; p.vl_comps = vp.comps;
            p.adj = reinterpret_cast<float*>(take(b_item));
            p.lam = reinterpret_cast<float*>(take(b_item));
            p.adjg = reinterpret_cast<float*>(take(b_itemg));
        }
    } else {
        // nothing to run but the finishing sums: dA = 0, dI_prior = 0
        p.nseq = 0;
        p.ntile = 0;
    }
    p.part_head = reinterpret_cast<float*>(ws);
    (void)hipGetLastError();  // launch status below must reflect this call only
    return diag_varlen_bwd_launch(p, prep, d_k, in_dtype == KDN_BF16, vp.R, static_cast<hipStream_t>(stream));
}

int kdn_mobius_precision_scan(int64_t B, int64_t H, int64_t T,
                              const float* a, const float* p, const float* Lambda,
                              const float* lambda0, float* lambda_out,
                              int64_t d_k, int64_t d_v,
                              const float* q, const float* k, const float* v,
                              const float* mu0, float* o, float* mu_T,
                              void* workspace, size_t* workspace_bytes, void* stream) {
    return kdn_mobius_precision_scan_ex(B, H, T, a, p, Lambda, lambda0, lambda_out, d_k, d_v, q, k, v, mu0,
                                        o, mu_T, nullptr, workspace, workspace_bytes, stream);
}

int kdn_mobius_precision_scan_ex(int64_t B, int64_t H, int64_t T,
                                 const float* a, const float* p, const float* Lambda,
                                 const float* lambda0, float* lambda_out,
                                 int64_t d_k, int64_t d_v,
                                 const float* q, const float* k, const float* v,
                                 const float* mu0, float* o, float* mu_T, kdn_scan_opts* opts,
                                 void* workspace, size_t* workspace_bytes, void* stream) {
    if (B < 0 || H < 0 || T < 0 || !opts_ok(opts)) return KDN_EINVAL;
    const bool mean = !(d_k == 0 && d_v == 0);
    if (mean && (!head_size_ok(d_k) || !head_size_ok(d_v))) return KDN_EUNSUPPORTED;
    if (!sizes_fit(B, H, T, mean ? (d_k > d_v ? d_k : d_v) : 1)) return KDN_EINVAL;
    const int64_t BH = B * H;
    if (BH > 0 && T > 0) {
        if (!ok_ptr(a) || !ok_ptr(p) || !ok_ptr(Lambda)) return KDN_EINVAL;
        if (mean && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(o))) return KDN_EINVAL;
    }
    if (!ok_opt(lambda0) || !ok_opt(lambda_out) || !ok_opt(mu0) || !ok_opt(mu_T)) return KDN_EINVAL;

    const int64_t blk = mob_block();
    const int64_t nblk = (T + blk - 1) / blk;
    if (!grid_fits(BH * nblk)) return KDN_EINVAL;
    const size_t b_blk = align_up(sizeof(float) * static_cast<size_t>(BH) * nblk * 4, 256);
    size_t need = (BH > 0 && T > 0) ? b_blk : 0;
    Plan pl{};
    size_t b_gate = 0;
    report_echo(opts, 0);
    if (mean) {
        pl = plan_iso(BH, T, d_v, opt_segments(opts));
        if (!grid_fits(BH * pl.S * iso_tiles(d_v), kWave)) return KDN_EINVAL;
        if (T > 0) report_echo(opts, BH * pl.S * iso_tiles(d_v) * (pl.S > 1 ? 2 : 1));
        b_gate = align_up(sizeof(float) * static_cast<size_t>(BH) * T, 256);
        need += 2 * b_gate + scan_workspace_bytes(BH, d_k, d_v, pl);
    }
    const int wc = workspace_check(workspace, workspace_bytes, need);
    if (wc == 1) return KDN_OK;
    if (wc != KDN_OK) return wc;
    if (BH == 0) return KDN_OK;

    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    MobParams mp{};
    mp.a = a; mp.p = p; mp.Lam = Lambda; mp.lambda0 = lambda0; mp.lambda_out = lambda_out;
    mp.T = T; mp.nblk = static_cast<int32_t>(nblk);
    if (T > 0) {
        mp.blk = reinterpret_cast<float*>(ws);
        ws += b_blk;
    }
    if (mean && T > 0) {
        mp.F = reinterpret_cast<float*>(ws);
        mp.G = reinterpret_cast<float*>(ws + b_gate);
        ws += 2 * b_gate;
    }
    (void)hipGetLastError();  // launch status below must reflect this call only
    int rc = mobius_launch(mp, BH, st);
    if (rc != KDN_OK || !mean) return rc;

    DiagParams dp{};
    dp.q = q; dp.k = k; dp.v = v;
    dp.F = mp.F; dp.G = mp.G;
    dp.mu0 = mu0; dp.o = o; dp.mu_T = mu_T;
    if (pl.S > 1) {
        dp.comp = reinterpret_cast<float*>(ws);
        dp.gdec = reinterpret_cast<float*>(ws + align_up(sizeof(float) * static_cast<size_t>(BH) * pl.S * 2 * d_k * d_v, 256));
    }
    dp.H = H; dp.T = T; dp.dv = d_v; dp.I_prior = 1.0f;
    dp.S = pl.S; dp.nchunks = pl.nchunks;
    apply_opts(dp, opts);
    return iso_mean_launch(dp, B, d_k, st);
}

int kdn_decode_step(int64_t B, int64_t H, int64_t d_k, int64_t d_v, kdn_dtype in_dtype,
                    const void* q, const void* k, const void* v,
                    const void* beta, const void* d,
                    const float* A, float I_prior,
                    float* I, float* mu, float* o, void* stream) {
    if (B < 0 || H < 0) return KDN_EINVAL;
    if (in_dtype != KDN_F32 && in_dtype != KDN_BF16) return KDN_EINVAL;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return KDN_EUNSUPPORTED;
    if (!finite_positive(I_prior)) return KDN_EINVAL;
    if (!sizes_fit(B, H, 1, d_k * d_v)) return KDN_EINVAL;
    const int64_t BH = B * H;
    if (!grid_fits(BH)) return KDN_EINVAL;
    if (BH == 0) return KDN_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_opt(beta) || !ok_ptr(d) || !ok_ptr(A) ||
        !ok_ptr(I) || !ok_ptr(mu) || !ok_ptr(o))
        return KDN_EINVAL;
    DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.beta = beta; p.d = d; p.A = A;
    p.I = I; p.mu = mu; p.o = o; p.H = H; p.I_prior = I_prior;
    (void)hipGetLastError();  // launch status below must reflect this call only
    return decode_launch(p, B, d_k, d_v, in_dtype == KDN_BF16, static_cast<hipStream_t>(stream));
}

}  // extern "C"

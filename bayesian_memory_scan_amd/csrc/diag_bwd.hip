// diag_bwd.hip -- gradient of the diagonal-precision memory scan: finishing
// passes and launchers, and the kernels of diag_bwd_kernels.h for whole rows
// and packed batches (rows cut into segments: diag_bwd_seg.hip).
#include "diag_bwd_kernels.h"

#include <mutex>

namespace kdn {

// ---------------------------------------------------------------------------
// Finishing passes: sum the column tiles' partials (fixed order: the result
// does not depend on timing).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_diag_bwd_rows(BwdParams p, int64_t n4) {
    const int64_t stride4 = n4;   // float4s per tile slice
    const float4* a = reinterpret_cast<const float4*>(p.part_dq);
    const float4* b = reinterpret_cast<const float4*>(p.part_dk);
    for (int64_t e = elem_first(); e < n4; e += elem_stride()) {
        float4 sq = a[e], sk = b[e];
        for (int t = 1; t < p.ntile; ++t) {
            const float4 x = a[t * stride4 + e], y = b[t * stride4 + e];
            sq.x += x.x; sq.y += x.y; sq.z += x.z; sq.w += x.w;
            sk.x += y.x; sk.y += y.y; sk.z += y.z; sk.w += y.w;
        }
        reinterpret_cast<float4*>(p.dq)[e] = sq;
        reinterpret_cast<float4*>(p.dk)[e] = sk;
    }
}

// Token ranges of the finishing sums: about two workgroups per CU, each range
// at least 1024 tokens.
int32_t bwd_token_split(int64_t rows, int64_t T) {
    const int64_t want = rows > 0 ? (2 * kNumCU + rows - 1) / rows : 1;
    const int64_t most = (T + 1023) / 1024;
    const int64_t s = want < most ? want : most;
    return s < 1 ? 1 : static_cast<int32_t>(s);
}

// One workgroup per token range r of row bh: dd_t = -A alpha_t dalpha_t, and
// the range's sums of the dA terms (-d_t alpha_t dalpha_t) and the dI_prior
// terms; range 0 also takes the row's starting-state terms.
template <bool BF16>
__global__ __launch_bounds__(256) void k_diag_bwd_tokens(BwdParams p) {
    const int64_t bh = blockIdx.x / p.tok_split;
    const int32_t r = static_cast<int32_t>(blockIdx.x % p.tok_split);
    const int64_t per = (p.T + p.tok_split - 1) / p.tok_split;
    const int64_t t0 = r * per;
    const int64_t t1 = t0 + per < p.T ? t0 + per : p.T;
    const int tid = threadIdx.x;
    const float A = p.A[bh % p.H];
    const int64_t n = p.BH * p.T;
    float sa = 0.0f, si = 0.0f;
    for (int64_t t = t0 + tid; t < t1; t += 256) {
        const int64_t x = bh * p.T + t;
        float da = 0.0f, di = 0.0f;
        for (int tl = 0; tl < p.ntile; ++tl) {
            da += p.part_da[tl * n + x];
            di += p.part_dip[tl * n + x];
        }
        const float alpha = fast_exp(-p.scal[x].w);
        const float d = BF16 ? bf16_at(static_cast<const uint16_t*>(p.d), x) : static_cast<const float*>(p.d)[x];
        float db = 0.0f;   // Palimpsa-M gating: the input-gate share of d_t
        if (!p.beta) {
            for (int tl = 0; tl < p.ntile; ++tl) db += p.part_db[tl * n + x];
        }
        p.dd[x] = fmaf(-A * alpha, da, db);
        sa = fmaf(-d * alpha, da, sa);
        si += di;
    }
    // packed batch: row bh is head bh, whose runs (sequence s, head bh) each
    // have a starting state
    if (p.cu_seqlens && r == 0) {
        for (int64_t sq = tid; sq < p.nseq; sq += 256)
            for (int tl = 0; tl < p.ntile; ++tl) si += p.part_dip0[tl * p.nruns + sq * p.H + bh];
    }
    __shared__ float red[2][256];
    red[0][tid] = sa;
    red[1][tid] = si;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) {
            red[0][tid] += red[0][tid + h];
            red[1][tid] += red[1][tid + h];
        }
        __syncthreads();
    }
    if (tid == 0) {
        float i0 = 0.0f;
        if (!p.cu_seqlens && r == 0)
            for (int tl = 0; tl < p.ntile; ++tl) i0 += p.part_dip0[tl * p.nruns + bh];
        p.part_head[2 * blockIdx.x] = red[0][0];
        p.part_head[2 * blockIdx.x + 1] = red[1][0] + i0;
    }
}

// dA[h] = sum over the batch and token ranges of the range sums; dI_prior =
// sum over all.
__global__ __launch_bounds__(256) void k_diag_bwd_heads(BwdParams p) {
    const int tid = threadIdx.x;
    const int64_t B = p.H > 0 ? p.BH / p.H : 0;
    const int64_t R = p.tok_split;
    for (int64_t h = tid; h < p.H; h += 256) {
        float s = 0.0f;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t r = 0; r < R; ++r) s += p.part_head[2 * ((b * p.H + h) * R + r)];
        p.dA[h] = s;
    }
    if (!p.dI_prior) return;
    __shared__ float red[256];
    float s = 0.0f;
    for (int64_t x = tid; x < p.BH * R; x += 256) s += p.part_head[2 * x + 1];
    red[tid] = s;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) p.dI_prior[0] = red[0];
}

// reverse == false: the checkpoint pass only (a packed batch whose split
// sequences run through diag_bwd_seg_launch)
template <int DK, int DV, bool BF16>
static int launch_bwd_shape(const BwdParams& p, hipStream_t st, bool reverse = true) {
    using Sh = BwdShape<DK, DV>;
    // a packed batch: whole groups of 8 runs (see bwd_run)
    const int64_t g = p.cu_seqlens ? (static_cast<int64_t>(p.nseq) * p.H + 7) / 8 * 8 * Sh::NTILE
                                   : p.BH * Sh::NTILE;
    if (g == 0) return KDN_OK;
    const dim3 grid(static_cast<uint32_t>(g));
    if (p.T > 0) hipLaunchKernelGGL((k_diag_bwd_ckpt<DK, DV, BF16, false>), grid, dim3(Sh::NTH), 0, st, p);
    if (reverse) hipLaunchKernelGGL((k_diag_bwd<DK, DV, BF16, false>), grid, dim3(Sh::NTH), 0, st, p);
    return launch_status();
}

template <int DK, bool BF16>
static int launch_bwd_dv(const BwdParams& p, int64_t dv, hipStream_t st, bool reverse = true) {
    switch (dv) {
        case 16: return launch_bwd_shape<DK, 16, BF16>(p, st, reverse);
        case 32: return launch_bwd_shape<DK, 32, BF16>(p, st, reverse);
        case 64: return launch_bwd_shape<DK, 64, BF16>(p, st, reverse);
        case 128: return launch_bwd_shape<DK, 128, BF16>(p, st, reverse);
        default: return KDN_EUNSUPPORTED;
    }
}

// Packed batch: the sequences' longest-first order (rank counting, as the
// forward's plan; past 16384 sequences, index order) and the first checkpoint
// slot of each sequence, an exclusive prefix sum of ceil(len / 16) + 1 slots
// (the states before its chunks and its final state).  One workgroup.
__global__ __launch_bounds__(kPlanThreads) void k_varlen_bwd_plan(BwdParams p) {
    __shared__ int64_t lens[kPlanLds];
    __shared__ int64_t part[kPlanThreads];
    const int32_t n = p.nseq;
    const int tid = threadIdx.x;
    plan_longest_first(p.cu_seqlens, n, p.T, p.seq_order, lens);
    // thread tid owns sequences [s0, s1); lens stays as staged above
    const int32_t per = (n + kPlanThreads - 1) / kPlanThreads;
    const int32_t s0 = tid * per < n ? tid * per : n;
    const int32_t s1 = s0 + per < n ? s0 + per : n;
    auto slots = [&](int32_t s) {
        const int64_t len = n <= kPlanLds ? lens[s] : clamped_length(p.cu_seqlens, p.T, s);
        return (len + kBwdChunk - 1) / kBwdChunk + 1;
    };
    int64_t sum = 0;
    for (int32_t s = s0; s < s1; ++s) sum += slots(s);
    // inclusive prefix over the threads' sums (Hillis-Steele in LDS)
    part[tid] = sum;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {
        const int64_t v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t off = part[tid] - sum;
    for (int32_t s = s0; s < s1; ++s) {
        p.seq_ckoff[s] = off;
        off += slots(s);
    }
}

// Enqueue the whole gradient: frame scalars, segment starting states (rows
// cut into segments), checkpoints, reverse pass, and the finishing sums.
// Arguments were validated by the caller.
int diag_bwd_launch(const BwdParams& p, const DiagParams& prep, int64_t B, int64_t dk, bool bf16,
                    int32_t R, hipStream_t st) {
    if (p.BH > 0) {
        if (p.T > 0) {
            const int rc = diag_prep_launch(prep, B, bf16, false, st);
            if (rc != KDN_OK) return rc;
        }
        if (p.S > 1) {
            // each segment's starting state: the forward scan's composites and carry
            const int rc = diag_comp_launch(prep, B, dk, bf16, R, st);
            if (rc != KDN_OK) return rc;
        }
        int rc;
        if (p.S > 1) rc = diag_bwd_seg_launch(p, dk, bf16, st);
        else if (dk == 64) rc = bf16 ? launch_bwd_dv<64, true>(p, p.dv, st) : launch_bwd_dv<64, false>(p, p.dv, st);
        else rc = bf16 ? launch_bwd_dv<128, true>(p, p.dv, st) : launch_bwd_dv<128, false>(p, p.dv, st);
        if (rc != KDN_OK) return rc;
        if (p.ntile > 1 && p.T > 0) {
            const int64_t n4 = p.BH * p.T * dk / 4;
            hipLaunchKernelGGL(k_diag_bwd_rows, dim3(elem_groups(n4)), dim3(256), 0,
                               st, p, n4);
        }
        const dim3 tgrid(static_cast<uint32_t>(p.BH * p.tok_split));
        if (bf16) hipLaunchKernelGGL(k_diag_bwd_tokens<true>, tgrid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL(k_diag_bwd_tokens<false>, tgrid, dim3(256), 0, st, p);
    }
    if (p.H > 0) hipLaunchKernelGGL(k_diag_bwd_heads, dim3(1), dim3(256), 0, st, p);
    return launch_status();
}

// A second stream per device, with the events of one fork and one join.  A
// packed batch's two checkpoint passes write disjoint runs' checkpoints: the
// split sequences' pass (with adjoint composites) holds one workgroup per CU
// on their items alone, so the whole sequences' pass runs beside it on this
// stream, and the reverse pass waits for both.  Created on first use (default
// priority, no implicit ordering with the null stream) and kept until the
// process ends; g_side_mu makes a call's fork-and-join one unit between host
// threads, so that no other call re-records the events in between.
namespace {
constexpr int kSideDevices = 64;
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool made = false, failed = false;
};
std::mutex g_side_mu;
SideStream g_side[kSideDevices];

// The current device's side stream (g_side_mu held), or nullptr where none
// could be made; a failed creation is not retried and leaves no pending error.
SideStream* side_stream() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSideDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    SideStream& sd = g_side[dev];
    if (!sd.made && !sd.failed) {
        if (hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&sd.join, hipEventDisableTiming) == hipSuccess) {
            sd.made = true;
        } else {
            sd.failed = true;
            (void)hipGetLastError();
        }
    }
    return sd.made ? &sd : nullptr;
}

// The stream may fork: not under graph capture, where the caller's graph
// would have to take in the side stream's work.
bool may_fork(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return cs == hipStreamCaptureStatusNone;
}
}  // namespace

// The gradient over a packed variable-length batch: the plan, the frame
// scalars per sequence-aligned chunk, then the same kernels with (sequence,
// head) runs, or (item, head) runs of the segmented kernels where sequences
// can be longer than a fair share; the finishing sums run over the H rows of
// the token axis.
int diag_varlen_bwd_launch(const BwdParams& p, const DiagParams& prep, int64_t dk, bool bf16,
                           int32_t R, hipStream_t st) {
    if (p.H == 0) return KDN_OK;
    if (p.nseq > 0) {
        // sequences longer than a fair share run in segments: the forward
        // plan (items, composite segments), then after the frame scalars the
        // forward composites and carries give the segments' starting states
        if (p.vl_seg > 0) varlen_plan_launch(prep, R, st);
        hipLaunchKernelGGL(k_varlen_bwd_plan, dim3(1), dim3(kPlanThreads), 0, st, p);
        int rc = diag_prep_varlen_launch(prep, bf16, false, st);
        if (rc != KDN_OK) return rc;
        if (p.vl_seg > 0) {
            if (prep.vl_comps > 0 && (rc = diag_varlen_comp_launch(prep, dk, bf16, R, st)) != KDN_OK) return rc;
            // whole sequences' checkpoints (the plain pass, on the side
            // stream where there is one), then the split sequences' with
            // their adjoint composites, the carry, and the reverse pass over
            // every item once both checkpoint passes are done
            std::lock_guard<std::mutex> lk(g_side_mu);
            SideStream* sd = may_fork(st) ? side_stream() : nullptr;
            hipStream_t ck = st;
            if (sd != nullptr) {
                hipError_t e = hipEventRecord(sd->fork, st);
                if (e == hipSuccess) e = hipStreamWaitEvent(sd->s, sd->fork, 0);
                if (e != hipSuccess) {
                    note_hip_error(e);
                    return KDN_EHIP;
                }
                ck = sd->s;
            }
            rc = dk == 64 ? (bf16 ? launch_bwd_dv<64, true>(p, p.dv, ck, false) : launch_bwd_dv<64, false>(p, p.dv, ck, false))
                          : (bf16 ? launch_bwd_dv<128, true>(p, p.dv, ck, false) : launch_bwd_dv<128, false>(p, p.dv, ck, false));
            if (rc != KDN_OK) return rc;
            if (sd != nullptr) {
                const hipError_t e = hipEventRecord(sd->join, sd->s);
                if (e != hipSuccess) {
                    note_hip_error(e);
                    return KDN_EHIP;
                }
            }
            rc = diag_bwd_seg_launch(p, dk, bf16, st, sd != nullptr ? sd->join : nullptr);
        } else if (dk == 64) {
            rc = bf16 ? launch_bwd_dv<64, true>(p, p.dv, st) : launch_bwd_dv<64, false>(p, p.dv, st);
        } else {
            rc = bf16 ? launch_bwd_dv<128, true>(p, p.dv, st) : launch_bwd_dv<128, false>(p, p.dv, st);
        }
        if (rc != KDN_OK) return rc;
    }
    if (p.T > 0) {
        if (p.ntile > 1) {
            const int64_t n4 = p.BH * p.T * dk / 4;
            hipLaunchKernelGGL(k_diag_bwd_rows, dim3(elem_groups(n4)), dim3(256), 0, st, p, n4);
        }
    }
    const dim3 tgrid(static_cast<uint32_t>(p.BH * p.tok_split));
    if (bf16) hipLaunchKernelGGL(k_diag_bwd_tokens<true>, tgrid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_diag_bwd_tokens<false>, tgrid, dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_diag_bwd_heads, dim3(1), dim3(256), 0, st, p);
    return launch_status();
}

}  // namespace kdn

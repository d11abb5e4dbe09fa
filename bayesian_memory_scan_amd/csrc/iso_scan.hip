// iso_scan.hip -- gated affine mean scan of the isotropic filter, chunked on
// the fp32 matrix cores.
//
// With the precisions known, the posterior mean is affine (KLA, "Riassunto
// Tecnico: Kalman Linear Attention", Metodologia 2) and gated by the
// precision ratios of Metodologia 3:
//   mu_t = F_t mu_{t-1} + G_t k_t v_t^T,      o_t = mu_t^T q_t.
// Over a chunk of 16 tokens with in-chunk log-decays b_t = sum_{u<=t} log F_u
// (so e^{b_t - b_s} <= 1 for s <= t):
//   O   = (Q K^T (.) D) V + diag(e^{b}) Q mu_start,   D[t][s] = e^{b_t - b_s} G_s [s <= t]
//   mu_end = e^{b_last} mu_start + (w (.) K)^T V,     w_s = G_s e^{b_last - b_s}
// Every product is a genuine contraction (mu is shared by the chunk), so it
// runs on v_mfma_f32_16x16x4f32.  Lane layout (checked on the device): A[i][k]
// in lane i + 16k, B[k][j] in lane j + 16k, D[i][j] in lane j + 16(i/4), reg i%4.
//
// A workgroup owns one (head, segment); wave w owns value columns
// [16w, 16w+16) and keeps its d_k x 16 slice of mu in MFMA accumulators.  The
// segment composite pass (COMPOSITE) runs only the state update from a zero
// state; segments are then combined in order by the shared carry pass.
#include "kdn_params.h"

namespace kdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kIsoChunk = 16;

template <int DK, int DV, bool COMPOSITE>
__global__ __launch_bounds__(DV / 16 * kWave) void k_iso(DiagParams p) {
    constexpr int C = kIsoChunk;
    constexpr int W = DV / 16;                 // waves: one per 16 value columns
    constexpr int NTH = W * kWave;
    constexpr int QR = DK + 2;                 // q, k row stride: conflict-free Q K^T / Q mu reads,
                                               // at most 2-way for the (w k)^T V reads
    constexpr int VR = DV + 16;                // row stride of v
    constexpr int KSTEPS = DK / 4;             // MFMA k-steps over d_k
    constexpr int MT = DK / 16;                // row tiles of mu

    struct Stage {
        float qr[COMPOSITE ? 1 : C][QR];       // q row-major [t][j]
        float kq[C][QR];                       // k row-major [s][j]
        float vr[C][VR];                       // v row-major [s][i]
        float4 sc[C];                          // b2_t, e^{b_t}, G_t, w_t
        float decay;                           // e^{b_last}
    };
    __shared__ Stage stg[2];
    __shared__ float st[COMPOSITE ? 1 : W][C][C];   // per-wave S^T [s][t]
    __shared__ float mu_s[COMPOSITE ? 1 : W][COMPOSITE ? 1 : DK][16];   // mu slice of each wave
    __shared__ float s_logsum;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = tid / kWave;
    const int g = lane / 16;
    const int c = lane % 16;
    const int64_t bh = blockIdx.x / p.S;
    const int seg = static_cast<int>(blockIdx.x % p.S) ;
    const int nseg_run = COMPOSITE ? p.S - 1 : p.S;
    if (seg >= nseg_run) return;               // whole workgroup exits together

    const int64_t c0 = static_cast<int64_t>(seg) * p.nchunks / p.S;
    const int64_t c1 = static_cast<int64_t>(seg + 1) * p.nchunks / p.S;
    const int64_t t_begin = c0 * C;
    const int64_t t_end = c1 * C < p.T ? c1 * C : p.T;

    const float* qh = static_cast<const float*>(p.q) + bh * p.T * DK;
    const float* kh = static_cast<const float*>(p.k) + bh * p.T * DK;
    const float* vh = static_cast<const float*>(p.v) + bh * p.T * DV;
    const float* Fh = p.F + bh * p.T;
    const float* Gh = p.G + bh * p.T;

    // ---- mu slice (rows all d_k, columns 16w..16w+15) in accumulator layout:
    //      macc[m][r] = mu[16m + 4g + r][16w + c] ----
    f32x4 macc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x = 0.0f;
            if constexpr (!COMPOSITE) {
                const int64_t off = static_cast<int64_t>(16 * m + 4 * g + r) * DV + 16 * w + c;
                if (p.S == 1) {
                    if (p.mu0) x = p.mu0[bh * DK * DV + off];
                } else {
                    x = p.comp[((bh * p.S + seg) * 2 + 1) * DK * DV + off];
                }
            }
            macc[m][r] = x;
        }
    }
    auto store_mu_slice = [&]() {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) mu_s[w][16 * m + 4 * g + r][c] = macc[m][r];
    };
    if constexpr (!COMPOSITE) store_mu_slice();

    // ---- staging ----
    constexpr int QV = C * DK / 4;             // float4 vectors of q (and k) per chunk
    constexpr int VV = C * DV / 4;
    constexpr int NQ = (QV + NTH - 1) / NTH;
    constexpr int NV = (VV + NTH - 1) / NTH;
    float4 rq[NQ], rk[NQ], rv[NV];
    float rF = 1.0f, rG = 0.0f;
    float logsum = 0.0f;   // wave 0 lanes < 16: sum of log2 F over the segment

    auto fetch = [&](int64_t t0, int L) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int e = tid + n * NTH;
            rk[n] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            rq[n] = rk[n];
            if (e < QV && e * 4 < L * DK) {
                rk[n] = *reinterpret_cast<const float4*>(kh + t0 * DK + 4 * e);
                if constexpr (!COMPOSITE) rq[n] = *reinterpret_cast<const float4*>(qh + t0 * DK + 4 * e);
            }
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int e = tid + n * NTH;
            rv[n] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (e < VV && e * 4 < L * DV) rv[n] = *reinterpret_cast<const float4*>(vh + t0 * DV + 4 * e);
        }
        if (tid < C) {
            rF = tid < L ? Fh[t0 + tid] : 1.0f;
            rG = tid < L ? Gh[t0 + tid] : 0.0f;
        }
    };

    auto commit = [&](int nb) {
        Stage& S = stg[nb];
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int e = tid + n * NTH;
            if (e < QV) {
                const int t = 4 * e / DK;
                const int j = 4 * e % DK;
                *reinterpret_cast<float2*>(&S.kq[t][j]) = make_float2(rk[n].x, rk[n].y);
                *reinterpret_cast<float2*>(&S.kq[t][j + 2]) = make_float2(rk[n].z, rk[n].w);
                if constexpr (!COMPOSITE) {
                    *reinterpret_cast<float2*>(&S.qr[t][j]) = make_float2(rq[n].x, rq[n].y);
                    *reinterpret_cast<float2*>(&S.qr[t][j + 2]) = make_float2(rq[n].z, rq[n].w);
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int e = tid + n * NTH;
            if (e < VV) *reinterpret_cast<float4*>(&S.vr[4 * e / DV][4 * e % DV]) = rv[n];
        }
        if (tid < C) {
            const float l2 = __log2f(rF);           // <= 0 (F in (0, 1])
            float b2 = l2;
#pragma unroll
            for (int o = 1; o < C; o <<= 1) {
                const float u = __shfl_up(b2, o, C);
                if (tid >= o) b2 += u;
            }
            const float blast = __shfl(b2, C - 1, C);
            S.sc[tid] = make_float4(b2, exp2f(b2), rG, rG * exp2f(blast - b2));
            if (tid == 0) S.decay = exp2f(blast);
            logsum += blast;
        }
    };

    const int64_t nch = (t_end - t_begin + C - 1) / C;
    auto chunk_len = [&](int64_t cc) -> int {
        const int64_t rem = t_end - (t_begin + cc * C);
        return static_cast<int>(rem < C ? rem : C);
    };

    if (nch > 0) {
        fetch(t_begin, chunk_len(0));
        commit(0);
    }
    __syncthreads();
    if (nch > 1) fetch(t_begin + C, chunk_len(1));

    for (int64_t ch = 0; ch < nch; ++ch) {
        const int b = static_cast<int>(ch & 1);
        const int L = chunk_len(ch);
        const int64_t t0 = t_begin + ch * C;
        const Stage& S = stg[b];

        if constexpr (!COMPOSITE) {
            // S = Q K^T, computed by every wave (no cross-wave exchange):
            // sacc[r] = S[t = 4g + r][s = c].  The q A-operands are kept for Q mu.
            float qa[KSTEPS];
            f32x4 sp[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) sp[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {   // four independent accumulation chains
                qa[kk] = S.qr[c][4 * kk + g];
                sp[kk & 3] = mfma4(qa[kk], S.kq[c][4 * kk + g], sp[kk & 3]);
            }
            const f32x4 sacc = (sp[0] + sp[1]) + (sp[2] + sp[3]);
            // A operand of (S (.) D) V wants A[t = c][s = 4kk + g]: transpose
            // the 16 x 16 tile through this wave's LDS scratch.
            *reinterpret_cast<float4*>(&st[w][c][4 * g]) = make_float4(sacc[0], sacc[1], sacc[2], sacc[3]);
            const float4 sct = S.sc[c];
            float av[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s_ = 4 * kk + g;
                const float4 scs = S.sc[s_];
                const float sv = st[w][s_][c];
                av[kk] = s_ <= c ? sv * exp2f(sct.x - scs.x) * scs.z : 0.0f;
            }
            f32x4 op[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) op[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                op[kk & 3] = mfma4(qa[kk] * sct.y, mu_s[w][4 * kk + g][c], op[kk & 3]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) op[kk] = mfma4(av[kk], S.vr[4 * kk + g][16 * w + c], op[kk]);
            const f32x4 oacc = (op[0] + op[1]) + (op[2] + op[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                if (t < L) p.o[(bh * p.T + t0 + t) * DV + 16 * w + c] = oacc[r];
            }
        }

        // state update: mu = e^{b_last} mu + (w (.) K)^T V
        {
            const float decay = S.decay;
            float bv[4], wk[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bv[kk] = S.vr[4 * kk + g][16 * w + c];
                wk[kk] = S.sc[4 * kk + g].w;
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                macc[m] *= decay;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    macc[m] = mfma4(S.kq[4 * kk + g][16 * m + c] * wk[kk], bv[kk], macc[m]);
            }
            if constexpr (!COMPOSITE) store_mu_slice();
        }

        if (ch + 1 < nch) commit(b ^ 1);
        __syncthreads();
        if (ch + 2 < nch) fetch(t0 + 2 * C, chunk_len(ch + 2));
    }

    if (tid == 0) s_logsum = logsum;
    __syncthreads();
    if constexpr (COMPOSITE) {
        float* slot = p.comp + ((bh * p.S + seg) * 2 + 1) * DK * DV;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                slot[static_cast<int64_t>(16 * m + 4 * g + r) * DV + 16 * w + c] = macc[m][r];
        if (tid == 0) p.gdec[bh * p.S + seg] = exp2f(s_logsum);
    } else if (seg == p.S - 1 && p.mu_T) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p.mu_T[(bh * DK + 16 * m + 4 * g + r) * DV + 16 * w + c] = macc[m][r];
    }
}

int iso_chunk() { return kIsoChunk; }

template <int DK, bool COMPOSITE>
static int iso_launch_dv(const DiagParams& p, int64_t dv, int64_t grid, hipStream_t st) {
    switch (dv) {
        case 16: hipLaunchKernelGGL((k_iso<DK, 16, COMPOSITE>), dim3(grid), dim3(64), 0, st, p); break;
        case 32: hipLaunchKernelGGL((k_iso<DK, 32, COMPOSITE>), dim3(grid), dim3(128), 0, st, p); break;
        case 64: hipLaunchKernelGGL((k_iso<DK, 64, COMPOSITE>), dim3(grid), dim3(256), 0, st, p); break;
        case 128: hipLaunchKernelGGL((k_iso<DK, 128, COMPOSITE>), dim3(grid), dim3(512), 0, st, p); break;
        default: return KDN_EUNSUPPORTED;
    }
    return launch_status();
}

template <bool COMPOSITE>
static int iso_launch(const DiagParams& p, int64_t dk, int64_t dv, int64_t grid, hipStream_t st) {
    switch (dk) {
        case 16: return iso_launch_dv<16, COMPOSITE>(p, dv, grid, st);
        case 32: return iso_launch_dv<32, COMPOSITE>(p, dv, grid, st);
        case 64: return iso_launch_dv<64, COMPOSITE>(p, dv, grid, st);
        case 128: return iso_launch_dv<128, COMPOSITE>(p, dv, grid, st);
        default: return KDN_EUNSUPPORTED;
    }
}

// Enqueue the gated mean scan; F, G were written by the Mobius pass.
int iso_mean_launch(const DiagParams& p, int64_t B, int64_t dk, hipStream_t st) {
    const int64_t BH = B * p.H;
    if (BH == 0) return KDN_OK;
    if (p.T == 0) return copy_state_launch(p, B, dk, true, st);   // mu_T = mu0
    const int64_t grid = BH * p.S;
    int rc;
    if (p.S > 1) {
        if ((rc = iso_launch<true>(p, dk, p.dv, grid, st)) != KDN_OK) return rc;
        if ((rc = diag_carry_launch(p, B, dk, true, st)) != KDN_OK) return rc;
    }
    return iso_launch<false>(p, dk, p.dv, grid, st);
}

}  // namespace kdn

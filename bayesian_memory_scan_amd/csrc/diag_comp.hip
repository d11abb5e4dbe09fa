// diag_comp.hip -- segment composites of the diagonal-precision scan on the
// fp32 matrix cores, and their ordered carry.
//
// With J = I - I_prior, the precision and information-mean updates of the
// diagonal scan (Palimpsa, "Learning to Remember, Learn, and Forget in
// Attention-Based Models", Metodologia 2, multiplied through by I_t) are the
// affine recurrences
//   J_t = alpha_t J_{t-1} + beta_t[i] k_t[j]^2,   eta_t = alpha_t eta_{t-1} + beta_t[i] v_t[i] k_t[j].
// Over a stretch of tokens starting from zero they give the composite
// (G, J, eta): G = prod alpha, and per 16-token chunk with in-chunk
// log-decays b_t = -sum_{u<=t} A d_u and weights w_s = e^{b_last - b_s} <= 1,
//   J   <- e^{b_last} J   + (w (.) K^2)^T B,      eta <- e^{b_last} eta + (w (.) K)^T (B (.) V),
// two genuine contractions over the chunk's tokens: v_mfma_f32_16x16x4f32.
// Composites combine in order, (G2, X2) o (G1, X1) = (G2 G1, G2 X1 + X2), the
// associativity that makes these updates scannable (KLA summary,
// Metodologia 2).
//
// A workgroup owns one sub-segment of one head; wave w owns value columns
// [16w, 16w+16) and all d_k rows, J and eta in MFMA accumulators.
#include "kdn_params.h"

#include <type_traits>

namespace kdn {

typedef float f32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4c mfma4c(float a, float b, f32x4c c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Token range of sub-segment r of segment s: the segment's chunks split in R.
__device__ __forceinline__ void sub_tokens(const DiagParams& p, int C, int R, int s, int r,
                                           int64_t& t0, int64_t& t1) {
    const int64_t c0 = static_cast<int64_t>(s) * p.nchunks / p.S;
    const int64_t c1 = static_cast<int64_t>(s + 1) * p.nchunks / p.S;
    const int64_t n = c1 - c0;
    const int64_t a = c0 + static_cast<int64_t>(r) * n / R;
    const int64_t b = c0 + static_cast<int64_t>(r + 1) * n / R;
    t0 = a * C;
    t1 = b * C < p.T ? b * C : p.T;
}

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(DV / 16 * kWave) void k_diag_comp(DiagParams p, int32_t R) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int C = 16;
    constexpr int W = DV / 16;
    constexpr int NTH = W * kWave;
    constexpr int KR = DK + 16;          // row strides: conflict-free MFMA operand reads
    constexpr int VR = DV + 16;
    constexpr int MT = DK / 16;
    constexpr int VW = BF16 ? 8 : 4;     // elements per 16-byte vector
    constexpr int NKV = (C * DK / VW + NTH - 1) / NTH;
    constexpr int NVV = (C * DV / VW + NTH - 1) / NTH;

    struct Stage {
        float k[C][KR];
        float k2[C][KR];
        float b[C][VR];
        float bv[C][VR];
        float w[C];
        float decay;
    };
    __shared__ Stage stg[2];
    __shared__ float s_logsum;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = tid / kWave;
    const int g = lane / 16;
    const int c = lane % 16;
    const int nsub = (p.S - 1) * R;
    const int64_t bh = blockIdx.x / nsub;
    const int sr = static_cast<int>(blockIdx.x % nsub);
    const int seg = sr / R;
    const int sub = sr % R;
    int64_t t_begin, t_end;
    sub_tokens(p, C, R, seg, sub, t_begin, t_end);

    const E* kh = static_cast<const E*>(p.k) + bh * p.T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * p.T * DV;
    // beta == NULL: Palimpsa-M gating, beta_t[i] = d_t
    const E* bth = p.beta ? static_cast<const E*>(p.beta) + bh * p.T * DV : nullptr;
    const E* dh = static_cast<const E*>(p.d) + bh * p.T;
    const float4* sch = p.scal + bh * p.T;

    f32x4c J[MT], X[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        J[m] = f32x4c{0.0f, 0.0f, 0.0f, 0.0f};
        X[m] = J[m];
    }

    uint4 rk[NKV], rb[NVV], rv[NVV];
    float rl = 0.0f;
    float logsum = 0.0f;   // wave 0 lanes < 16: sum of b_last over chunks (log of prod alpha)

    auto fetch = [&](int64_t t0, int L) {
#pragma unroll
        for (int n = 0; n < NKV; ++n) {
            const int e = tid + n * NTH;
            rk[n] = make_uint4(0u, 0u, 0u, 0u);
            if (e * VW < L * DK) rk[n] = ld16(kh + t0 * DK + static_cast<int64_t>(e) * VW);
        }
#pragma unroll
        for (int n = 0; n < NVV; ++n) {
            const int e = tid + n * NTH;
            rb[n] = make_uint4(0u, 0u, 0u, 0u);
            rv[n] = rb[n];
            if (e * VW < L * DV) {
                rb[n] = bth ? ld16(bth + t0 * DV + static_cast<int64_t>(e) * VW)
                            : splat16<BF16>(dh, t0 + e * VW / DV);
                rv[n] = ld16(vh + t0 * DV + static_cast<int64_t>(e) * VW);
            }
        }
        if (tid < C) rl = tid < L ? sch[t0 + tid].w : 0.0f;   // A d_t (0: padding)
    };

    auto commit = [&](int nb) {
        Stage& S = stg[nb];
#pragma unroll
        for (int n = 0; n < NKV; ++n) {
            const int e = tid + n * NTH;
            if (e * VW < C * DK) {
                const int t = e * VW / DK;
                const int j = e * VW % DK;
                float f[VW];
                widen<BF16>(rk[n], f);
#pragma unroll
                for (int u = 0; u < VW; ++u) {
                    S.k[t][j + u] = f[u];
                    S.k2[t][j + u] = f[u] * f[u];
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NVV; ++n) {
            const int e = tid + n * NTH;
            if (e * VW < C * DV) {
                const int t = e * VW / DV;
                const int i = e * VW % DV;
                float fb[VW], fv[VW];
                widen<BF16>(rb[n], fb);
                widen<BF16>(rv[n], fv);
#pragma unroll
                for (int u = 0; u < VW; ++u) {
                    S.b[t][i + u] = fb[u];
                    S.bv[t][i + u] = fb[u] * fv[u];
                }
            }
        }
        if (tid < C) {
            float b = -rl;
#pragma unroll
            for (int o = 1; o < C; o <<= 1) {
                const float u = __shfl_up(b, o, C);
                if (tid >= o) b += u;
            }
            const float blast = __shfl(b, C - 1, C);
            S.w[tid] = fast_exp(blast - b);
            if (tid == 0) S.decay = fast_exp(blast);
            logsum += blast;
        }
    };

    const int64_t nch = (t_end - t_begin + C - 1) / C;
    auto chunk_len = [&](int64_t ch) -> int {
        const int64_t rem = t_end - (t_begin + ch * C);
        return static_cast<int>(rem < C ? rem : C);
    };

    if (nch > 0) {
        fetch(t_begin, chunk_len(0));
        commit(0);
    }
    __syncthreads();
    if (nch > 1) fetch(t_begin + C, chunk_len(1));

    for (int64_t ch = 0; ch < nch; ++ch) {
        const int bsel = static_cast<int>(ch & 1);
        const Stage& S = stg[bsel];
        const float decay = S.decay;
        float wk[4], bj[4], be[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            wk[kk] = S.w[4 * kk + g];
            bj[kk] = S.b[4 * kk + g][16 * wv + c];
            be[kk] = S.bv[4 * kk + g][16 * wv + c];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            J[m] *= decay;
            X[m] *= decay;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                J[m] = mfma4c(S.k2[4 * kk + g][16 * m + c] * wk[kk], bj[kk], J[m]);
                X[m] = mfma4c(S.k[4 * kk + g][16 * m + c] * wk[kk], be[kk], X[m]);
            }
        }
        if (ch + 1 < nch) commit(bsel ^ 1);
        __syncthreads();
        if (ch + 2 < nch) fetch(t_begin + (ch + 2) * C, chunk_len(ch + 2));
    }

    if (tid == 0) s_logsum = logsum;
    __syncthreads();
    // J[m][r] = J[16m + 4g + r][16 wv + c]
    const int64_t slot = (bh * (p.S - 1) + seg) * R + sub;
    float* out = p.sub + slot * 2 * DK * DV;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t off = static_cast<int64_t>(16 * m + 4 * g + r) * DV + 16 * wv + c;
            out[off] = J[m][r];
            out[static_cast<int64_t>(DK) * DV + off] = X[m][r];
        }
    if (tid == 0) p.gsub[slot] = fast_exp(s_logsum);
}

// Ordered carry: sub-segment composites -> the starting (J, eta) of every
// main segment.  One thread per memory entry of every head.
__global__ __launch_bounds__(256) void k_diag_carry_sub(DiagParams p, int64_t dk, int64_t n_total, int32_t R) {
    const int64_t n_per_head = dk * p.dv;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= n_total) return;
    const int64_t bh = e / n_per_head;
    const int64_t r = e % n_per_head;
    const int64_t off = bh * n_per_head + r;
    const float m0 = p.mu0 ? p.mu0[off] : 0.0f;
    float J = 0.0f, eta;
    if (p.I0) {
        const float I0 = p.I0[off];
        J = I0 - p.I_prior;
        eta = I0 * m0;
    } else {
        eta = p.I_prior * m0;
    }
    for (int s = 0; s < p.S; ++s) {
        float* cin = p.comp + ((bh * p.S + s) * 2) * n_per_head;
        cin[r] = J;
        cin[n_per_head + r] = eta;
        if (s + 1 == p.S) break;
        for (int u = 0; u < R; ++u) {
            const int64_t slot = (bh * (p.S - 1) + s) * R + u;
            const float* sub = p.sub + slot * 2 * n_per_head;
            const float G = p.gsub[slot];
            J = __builtin_fmaf(G, J, sub[r]);
            eta = __builtin_fmaf(G, eta, sub[n_per_head + r]);
        }
    }
}

template <int DK, bool BF16>
static int comp_launch_dv(const DiagParams& p, int64_t dv, int64_t grid, int32_t R, hipStream_t st) {
    switch (dv) {
        case 16: hipLaunchKernelGGL((k_diag_comp<DK, 16, BF16>), dim3(grid), dim3(64), 0, st, p, R); break;
        case 32: hipLaunchKernelGGL((k_diag_comp<DK, 32, BF16>), dim3(grid), dim3(128), 0, st, p, R); break;
        case 64: hipLaunchKernelGGL((k_diag_comp<DK, 64, BF16>), dim3(grid), dim3(256), 0, st, p, R); break;
        case 128: hipLaunchKernelGGL((k_diag_comp<DK, 128, BF16>), dim3(grid), dim3(512), 0, st, p, R); break;
        default: return KDN_EUNSUPPORTED;
    }
    return launch_status();
}

template <bool BF16>
static int comp_launch(const DiagParams& p, int64_t dk, int64_t grid, int32_t R, hipStream_t st) {
    switch (dk) {
        case 16: return comp_launch_dv<16, BF16>(p, p.dv, grid, R, st);
        case 32: return comp_launch_dv<32, BF16>(p, p.dv, grid, R, st);
        case 64: return comp_launch_dv<64, BF16>(p, p.dv, grid, R, st);
        case 128: return comp_launch_dv<128, BF16>(p, p.dv, grid, R, st);
        default: return KDN_EUNSUPPORTED;
    }
}

// Composites of segments 0..S-2 in R sub-segments each, then the carry into
// every segment's starting state (p.comp).  Needs the per-token scalars.
int diag_comp_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st) {
    const int64_t BH = B * p.H;
    const int64_t grid = BH * (p.S - 1) * R;
    int rc = bf16 ? comp_launch<true>(p, dk, grid, R, st) : comp_launch<false>(p, dk, grid, R, st);
    if (rc != KDN_OK) return rc;
    const int64_t n = BH * dk * p.dv;
    hipLaunchKernelGGL(k_diag_carry_sub, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st,
                       p, dk, n, R);
    return launch_status();
}

}  // namespace kdn

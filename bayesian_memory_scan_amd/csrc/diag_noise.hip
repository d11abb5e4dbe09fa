// diag_noise.hip -- Diagonal KDN with process noise, forward.
//
// Kalman Delta Networks abstract, "Diagonal KDN": each one-step posterior is
// projected onto the diagonal Gaussian family by online mean-field VI, and
// the Kalman gain weights each residual write.  Memory column i is a latent
// s_i in R^{d_k} observed through v_t[i] = k_t^T s_i + noise (precision
// beta_t[i]); the predict step decays by a_t and adds process noise p_t (KLA
// summary, Metodologia 1).  Per entry the kernel keeps a variance sig = 1/lambda
// and a mean mu.  Per token, for every column i:
//   sp   = a^2 sig + p,   mp = a mu                        (predict, per entry)
//   S_i  = sum_j k_j^2 sp_j + 1/beta_i,  r_i = v_i - sum_j k_j mp_j
//   mu   = mp + sp k_j r_i / S_i                           (residual write)
//   sig  = sp / (1 + beta_i k_j^2 sp)                      (diagonal of the
//                                                           posterior precision)
//   o_t[i] = sum_j q_j mu_j
// The precision 1/sig follows the Mobius map l -> ((1 + w p) l + w a^2) / (p l + a^2),
// w = beta k^2.
//
// Work decomposition as in the diagonal scan: a workgroup owns one head and
// one tile of value columns for the whole sequence; lane <-> value column i,
// JP key rows per lane in VGPRs; tokens staged 16 at a time through LDS
// (double-buffered, widened to fp32); key-side values reach the fmacs as DPP
// row broadcasts.  The two sums over j per (token, column) are the only
// coupling between entries: each row group's partial sums meet in a
// double-buffered LDS slot behind one barrier per token.
#include "kdn_lane.h"
#include "kdn_params.h"

namespace kdn {

constexpr int kNoiseChunk = 16;

template <int DK, int CI, int W, bool BF16>
__global__ __launch_bounds__(W * kWave) void k_diag_noise(NoiseParams p) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int C = kNoiseChunk;
    constexpr int NTH = W * kWave;
    constexpr int P = NTH / CI;          // row groups per workgroup
    constexpr int JP = DK / P;           // key rows per lane
    constexpr int VW = BF16 ? 8 : 4;
    constexpr int VK = C * DK / VW;
    constexpr int VB = C * CI / VW;
    constexpr int NVK = (VK + NTH - 1) / NTH;
    constexpr int NVB = (VB + NTH - 1) / NTH;
    static_assert(NTH % CI == 0 && DK % P == 0, "tile shape");
    static_assert(JP == 4 || JP == 8 || JP == 16, "key rows per lane: one DPP row");
    static_assert(CI >= 16, "a DPP row must stay inside one row group");

    struct Stage {
        float k[C][DK];
        float k2[C][DK];
        float q[C][DK];
        float2 bv[C][CI];   // (beta_i, v_i)
        float4 sc[C];       // (a^2, p, a, -)
    };
    __shared__ Stage stg[2];
    __shared__ float opart[2][C][P][CI];
    __shared__ float2 red[2][P][CI];   // per-token partial (sum k^2 sp, sum k mp) of each row group

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int col = tid % CI;
    const int rg = tid / CI;
    const int j0 = rg * JP;
    const int jl = j0 + (lane & (JP - 1));
    const int ntile = static_cast<int>(p.dv / CI);
    const int64_t wg = xcd_local_id();
    const int tile = static_cast<int>(wg % ntile);
    const int64_t bh = wg / ntile;
    const int i = tile * CI + col;
    const int64_t T = p.T;

    const E* qh = static_cast<const E*>(p.q) + bh * T * DK;
    const E* kh = static_cast<const E*>(p.k) + bh * T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * T * p.dv + tile * CI;
    const E* bth = static_cast<const E*>(p.beta) + bh * T * p.dv + tile * CI;
    const float* ah = p.a + bh * T;
    const float* ph = p.p + bh * T;

    float sig[JP], mu[JP];   // variance 1/lambda and mean of each entry
#pragma unroll
    for (int r = 0; r < JP; ++r) {
        const int64_t off = (bh * DK + j0 + r) * p.dv + i;
        sig[r] = p.lam0 ? 1.0f / p.lam0[off] : 1.0f;
        mu[r] = p.mu0 ? p.mu0[off] : 0.0f;
    }

    uint4 rk[NVK], rq[NVK], rb[NVB], rv[NVB];
    float2 rap = make_float2(1.0f, 0.0f);

    auto fetch = [&](int64_t t0, int L) {
#pragma unroll
        for (int n = 0; n < NVK; ++n) {
            const int vi = tid + n * NTH;
            if (vi < VK && vi * VW < L * DK) {
                rk[n] = ld16(kh + t0 * DK + static_cast<int64_t>(vi) * VW);
                rq[n] = ld16(qh + t0 * DK + static_cast<int64_t>(vi) * VW);
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int cv = vi % (CI / VW);
            if (vi < VB && row < L) {
                const int64_t off = (t0 + row) * p.dv + cv * VW;
                rb[n] = ld16(bth + off);
                rv[n] = ld16(vh + off);
            }
        }
        if (tid < L) rap = make_float2(ah[t0 + tid], ph[t0 + tid]);
    };

    auto commit = [&](int nb, int L) {
        Stage& S = stg[nb];
#pragma unroll
        for (int n = 0; n < NVK; ++n) {
            const int vi = tid + n * NTH;
            if (vi < VK && vi * VW < L * DK) {
                const int row = vi * VW / DK;
                const int c0 = vi * VW % DK;
                float f[VW];
                widen<BF16>(rk[n], f);
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    S.k[row][c0 + e] = f[e];
                    S.k2[row][c0 + e] = f[e] * f[e];
                }
                widen<BF16>(rq[n], f);
#pragma unroll
                for (int e = 0; e < VW; ++e) S.q[row][c0 + e] = f[e];
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int c0 = (vi % (CI / VW)) * VW;
            if (vi < VB && row < L) {
                float fv[VW], fb[VW];
                widen<BF16>(rv[n], fv);
                widen<BF16>(rb[n], fb);
#pragma unroll
                for (int e = 0; e < VW; ++e) S.bv[row][c0 + e] = make_float2(fb[e], fv[e]);
            }
        }
        if (tid < L) S.sc[tid] = make_float4(rap.x * rap.x, rap.y, rap.x, 0.0f);
    };

    const int64_t nch = (T + C - 1) / C;
    auto chunk_len = [&](int64_t c) -> int {
        const int64_t rem = T - c * C;
        return static_cast<int>(rem < C ? rem : C);
    };

    if (nch > 0) {
        fetch(0, chunk_len(0));
        commit(0, chunk_len(0));
    }
    __syncthreads();
    if (nch > 1) fetch(C, chunk_len(1));

    for (int64_t c = 0; c < nch; ++c) {
        const int b = static_cast<int>(c & 1);
        const int L = chunk_len(c);
        const int64_t t0 = c * C;
        const Stage& S = stg[b];

        float4 sc = S.sc[0];
        float2 bvv = S.bv[0][col];
        float vk = S.k[0][jl], vk2 = S.k2[0][jl], vq = S.q[0][jl];
        for (int tt = 0; tt < L; ++tt) {
            const int tn = tt + 1 < L ? tt + 1 : tt;
            const float4 sc_n = S.sc[tn];
            const float2 bvv_n = S.bv[tn][col];
            const float vk_n = S.k[tn][jl], vk2_n = S.k2[tn][jl], vq_n = S.q[tn][jl];

            // predict, and this row group's share of the two sums over j
            float ps[2] = {0.0f, 0.0f}, pm[2] = {0.0f, 0.0f};
            float sp[JP];
#pragma unroll
            for (int r = 0; r < JP; ++r) {
                sp[r] = fmaf(sc.x, sig[r], sc.y);
                mu[r] *= sc.z;
            }
            Unroll<0, JP>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                fmac_bcast<r>(ps[r & 1], vk2, sp[r]);   // sum_j k_j^2 sp_j
                fmac_bcast<r>(pm[r & 1], vk, mu[r]);    // sum_j k_j mp_j
            });
            red[tt & 1][rg][col] = make_float2(ps[0] + ps[1], pm[0] + pm[1]);
            __syncthreads();
            float Ssum = fast_rcp(bvv.x), pred = 0.0f;
#pragma unroll
            for (int g = 0; g < P; ++g) {
                const float2 x = red[tt & 1][g][col];
                Ssum += x.x;
                pred += x.y;
            }
            // residual write with the Kalman gain, and the projected variance
            const float gain = (bvv.y - pred) * fast_rcp(Ssum);
            Unroll<0, JP>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                fmac_bcast<r>(mu[r], vk, sp[r] * gain);
                const float den = fmaf(bcast<r>(vk2) * bvv.x, sp[r], 1.0f);
                sig[r] = sp[r] * fast_rcp(den);
            });
            float m[JP];
#pragma unroll
            for (int r = 0; r < JP; ++r) m[r] = mu[r];
            float acc[4];
            Unroll<0, 4>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                acc[r] = bcast<r>(vq) * m[r];
            });
            Unroll<4, JP>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                fmac_bcast<r>(acc[r & 3], vq, m[r]);
            });
            opart[b][tt][rg][col] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            sc = sc_n;
            bvv = bvv_n;
            vk = vk_n;
            vk2 = vk2_n;
            vq = vq_n;
        }

        if (c + 1 < nch) commit(b ^ 1, chunk_len(c + 1));
        __syncthreads();
        for (int e = tid; e < L * CI; e += NTH) {
            const int tt = e / CI;
            const int cc = e % CI;
            float sum = 0.0f;
#pragma unroll
            for (int g = 0; g < P; ++g) sum += opart[b][tt][g][cc];
            p.o[(bh * T + t0 + tt) * p.dv + tile * CI + cc] = sum;
        }
        if (c + 2 < nch) fetch(t0 + 2 * C, chunk_len(c + 2));
    }

#pragma unroll
    for (int r = 0; r < JP; ++r) {
        const int64_t off = (bh * DK + j0 + r) * p.dv + i;
        if (p.lam_T) p.lam_T[off] = 1.0f / sig[r];
        if (p.mu_T) p.mu_T[off] = mu[r];
    }
}

constexpr int noise_waves(int DK, int CI) {
    const int w = DK * CI / (kWave * 16);
    return w < 1 ? 1 : w;
}

template <int DK, int CI, bool BF16>
static void noise_one(const NoiseParams& p, int64_t grid, hipStream_t st) {
    constexpr int W = noise_waves(DK, CI);
    hipLaunchKernelGGL((k_diag_noise<DK, CI, W, BF16>), dim3(static_cast<uint32_t>(grid)),
                       dim3(W * kWave), 0, st, p);
}

template <int DK, bool BF16>
static int noise_dk(const NoiseParams& p, int CI, int64_t grid, hipStream_t st) {
    switch (CI) {
        case 16: noise_one<DK, 16, BF16>(p, grid, st); break;
        case 32: noise_one<DK, 32, BF16>(p, grid, st); break;
        case 64: noise_one<DK, 64, BF16>(p, grid, st); break;
        default: return KDN_EUNSUPPORTED;
    }
    return KDN_OK;
}

template <bool BF16>
static int noise_main(const NoiseParams& p, int64_t dk, int CI, int64_t grid, hipStream_t st) {
    switch (dk) {
        case 16: return noise_dk<16, BF16>(p, CI, grid, st);
        case 32: return noise_dk<32, BF16>(p, CI, grid, st);
        case 64: return noise_dk<64, BF16>(p, CI, grid, st);
        case 128: return noise_dk<128, BF16>(p, CI, grid, st);
        default: return KDN_EUNSUPPORTED;
    }
}

// T == 0: the final state is the starting state.
__global__ __launch_bounds__(256) void k_noise_copy(NoiseParams p, int64_t n) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= n) return;
    if (p.lam_T) p.lam_T[e] = p.lam0 ? p.lam0[e] : 1.0f;
    if (p.mu_T) p.mu_T[e] = p.mu0 ? p.mu0[e] : 0.0f;
}

int noise_launch(const NoiseParams& p, int64_t B, int64_t dk, bool bf16, hipStream_t st) {
    const int64_t BH = B * p.H;
    if (BH == 0) return KDN_OK;
    if (p.T == 0) {
        const int64_t n = BH * dk * p.dv;
        hipLaunchKernelGGL(k_noise_copy, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st, p, n);
        return launch_status();
    }
    const int CI = p.dv < 64 ? static_cast<int>(p.dv) : 64;
    const int64_t grid = BH * (p.dv / CI);
    const int rc = bf16 ? noise_main<true>(p, dk, CI, grid, st) : noise_main<false>(p, dk, CI, grid, st);
    if (rc != KDN_OK) return rc;
    return launch_status();
}

}  // namespace kdn

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
// Work decomposition: a workgroup owns one head and one tile of value
// columns for the whole sequence.  Every wave holds all d_k rows of its
// columns, so the two sums over j close inside the wave and need no barrier:
//   * lane = rg * CPW + cw: RG = d_k/16 row groups of 16 rows, CPW = 64/RG
//     columns per wave; each lane keeps 16 rows of one column in VGPRs;
//   * the sums over a column's row groups run on permlane32/permlane16 swaps
//     and one DPP rotate (lane bits log2(CPW)..5), two values at once;
//   * tokens are staged 16 at a time through LDS (double-buffered, widened to
//     fp32, k^2 precomputed); a lane reads its 16 rows of k, k^2 and q as
//     broadcast ds_read_b128, so every fmac has plain VGPR operands;
//   * the read-out sum lands in every lane of the column; the row group 0
//     lanes write it to an LDS row that the workgroup stores once per chunk.
#include "kdn_lane.h"
#include "kdn_params.h"

namespace kdn {

constexpr int kNoiseChunk = 16;
constexpr int kNoiseRows = 16;        // key rows per lane
constexpr int kDppRowRor8 = 0x128;    // row_ror:8, lane l <-> l ^ 8 inside a row of 16

// Sum over the RG row groups of a column (lane bits above the column index).
// Two values at once: on return every lane holds both totals.
template <int RG>
__device__ __forceinline__ void group_sum2(float& a, float& b) {
    if constexpr (RG > 1) {
        float x = swap32_add(a, b);                 // lanes 0-31: a, 32-63: b, over bit 5
        if constexpr (RG >= 4) x = swap16_add(x, x);   // bit 4
        if constexpr (RG >= 8) x += dpp<kDppRowRor8>(x);   // bit 3
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    }
}

template <int RG>
__device__ __forceinline__ float group_sum1(float x) {
    if constexpr (RG > 1) {
        x = swap32_add(x, x);
        if constexpr (RG >= 4) x = swap16_add(x, x);
        if constexpr (RG >= 8) x += dpp<kDppRowRor8>(x);
    }
    return x;
}

template <int DK, int W, bool BF16>
__global__ __launch_bounds__(W * kWave) void k_diag_noise(NoiseParams p) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int C = kNoiseChunk;
    constexpr int JP = kNoiseRows;
    constexpr int RG = DK / JP;          // row groups of a column
    constexpr int CPW = kWave / RG;      // columns per wave
    constexpr int CI = W * CPW;          // columns per workgroup
    constexpr int NTH = W * kWave;
    constexpr int VW = BF16 ? 8 : 4;
    constexpr int VK = C * DK / VW;
    constexpr int VB = C * CI / VW;
    constexpr int NVK = (VK + NTH - 1) / NTH;
    constexpr int NVB = (VB + NTH - 1) / NTH;
    static_assert(DK % JP == 0 && CPW * RG == kWave, "tile shape");

    struct Stage {
        float4 k[C][DK / 4];
        float4 k2[C][DK / 4];
        float4 q[C][DK / 4];
        float2 bv[C][CI];   // (beta_i, v_i)
        float4 sc[C];       // (a^2, p, a, -)
    };
    __shared__ Stage stg[2];
    __shared__ float orow[2][C][CI];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = tid / kWave;
    const int rg = lane / CPW;
    const int col = w * CPW + lane % CPW;     // column within the tile
    const int ntile = static_cast<int>((p.dv + CI - 1) / CI);
    const int64_t wg = xcd_local_id();
    const int tile = static_cast<int>(wg % ntile);
    const int64_t bh = wg / ntile;
    const int i = tile * CI + col;
    const bool live = i < p.dv;               // d_v smaller than a wave's columns
    const int64_t T = p.T;

    const E* qh = static_cast<const E*>(p.q) + bh * T * DK;
    const E* kh = static_cast<const E*>(p.k) + bh * T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * T * p.dv + tile * CI;
    const E* bth = static_cast<const E*>(p.beta) + bh * T * p.dv + tile * CI;
    const float* ah = p.a + bh * T;
    const float* ph = p.p + bh * T;
    const int ncol = p.dv - tile * CI < CI ? static_cast<int>(p.dv - tile * CI) : CI;

    // variance 1/lambda and frame-scaled mean of this lane's 16 rows of column i
    float sig[JP], mt[JP];
#pragma unroll
    for (int r = 0; r < JP; ++r) {
        const int64_t off = (bh * DK + rg * JP + r) * p.dv + i;
        sig[r] = live && p.lam0 ? 1.0f / p.lam0[off] : 1.0f;
        mt[r] = live && p.mu0 ? p.mu0[off] : 0.0f;
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
            if (vi < VB && row < L && cv * VW < ncol) {
                const int64_t off = (t0 + row) * p.dv + cv * VW;
                rb[n] = ld16(bth + off);
                rv[n] = ld16(vh + off);
            }
        }
        if (tid < L) rap = make_float2(ah[t0 + tid], ph[t0 + tid]);
    };

    auto commit = [&](int nb, int L) {
        Stage& S = stg[nb];
        float* const kf = reinterpret_cast<float*>(S.k);
        float* const k2f = reinterpret_cast<float*>(S.k2);
        float* const qf = reinterpret_cast<float*>(S.q);
#pragma unroll
        for (int n = 0; n < NVK; ++n) {
            const int vi = tid + n * NTH;
            if (vi < VK && vi * VW < L * DK) {
                float f[VW];
                widen<BF16>(rk[n], f);
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    kf[vi * VW + e] = f[e];
                    k2f[vi * VW + e] = f[e] * f[e];
                }
                widen<BF16>(rq[n], f);
#pragma unroll
                for (int e = 0; e < VW; ++e) qf[vi * VW + e] = f[e];
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int c0 = (vi % (CI / VW)) * VW;
            if (vi < VB && row < L && c0 < ncol) {
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

    // The mean is carried in a decayed frame, mu = Am * mt with Am the product
    // of a since the frame start, so the predict step costs one multiply per
    // token instead of one per entry.  A frame restarts (mt *= Am, Am = 1)
    // when Am falls below 2^-32; Am is the same in every lane.
    float Am = 1.0f;
    for (int64_t c = 0; c < nch; ++c) {
        const int b = static_cast<int>(c & 1);
        const int L = chunk_len(c);
        const int64_t t0 = c * C;
        const Stage& S = stg[b];

        // One token, all in registers of this wave: predict, the two sums
        // over j, the residual write, the projected variance, the read-out.
        auto token = [&](int tt) __attribute__((always_inline)) {
            const float4 sc = S.sc[tt];
            const float2 bvv = S.bv[tt][col];
            float kr[JP], k2r[JP], qr[JP];
#pragma unroll
            for (int u = 0; u < JP / 4; ++u) {
                const float4 x = S.k[tt][rg * (JP / 4) + u];
                const float4 y = S.k2[tt][rg * (JP / 4) + u];
                const float4 z = S.q[tt][rg * (JP / 4) + u];
                kr[4 * u] = x.x; kr[4 * u + 1] = x.y; kr[4 * u + 2] = x.z; kr[4 * u + 3] = x.w;
                k2r[4 * u] = y.x; k2r[4 * u + 1] = y.y; k2r[4 * u + 2] = y.z; k2r[4 * u + 3] = y.w;
                qr[4 * u] = z.x; qr[4 * u + 1] = z.y; qr[4 * u + 2] = z.z; qr[4 * u + 3] = z.w;
            }
            Am *= sc.z;
            if (Am < 0x1p-32f) {
#pragma unroll
                for (int r = 0; r < JP; ++r) mt[r] *= Am;
                Am = 1.0f;
            }
            float sp[JP], ps[2] = {0.0f, 0.0f}, pm[2] = {0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < JP; ++r) {
                sp[r] = fmaf(sc.x, sig[r], sc.y);
                ps[r & 1] = fmaf(k2r[r], sp[r], ps[r & 1]);   // sum_j k_j^2 sp_j
                pm[r & 1] = fmaf(kr[r], mt[r], pm[r & 1]);    // sum_j k_j mp_j / Am
            }
            float Sp = ps[0] + ps[1], Pm = pm[0] + pm[1];
            group_sum2<RG>(Sp, Pm);
            // residual write with the Kalman gain (in the frame), and the
            // projected variance
            const float gain = (bvv.y - Am * Pm) * fast_rcp((Sp + fast_rcp(bvv.x)) * Am);
            float acc[2] = {0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < JP; ++r) {
                mt[r] = fmaf(kr[r], sp[r] * gain, mt[r]);
                const float den = fmaf(k2r[r] * bvv.x, sp[r], 1.0f);
                sig[r] = sp[r] * fast_rcp(den);
                acc[r & 1] = fmaf(qr[r], mt[r], acc[r & 1]);
            }
            const float o_t = group_sum1<RG>(acc[0] + acc[1]);
            if (rg == 0) orow[b][tt][col] = Am * o_t;
        };

        if (L == C) {
            Unroll<0, C>::run([&](auto u) { token(decltype(u)::value); });
        } else {
            for (int tt = 0; tt < L; ++tt) token(tt);
        }

        if (c + 1 < nch) commit(b ^ 1, chunk_len(c + 1));
        __syncthreads();
        for (int e = tid; e < L * CI; e += NTH) {
            const int tt = e / CI;
            const int cc = e % CI;
            if (cc < ncol) p.o[(bh * T + t0 + tt) * p.dv + tile * CI + cc] = orow[b][tt][cc];
        }
        if (c + 2 < nch) fetch(t0 + 2 * C, chunk_len(c + 2));
    }

    if (live) {
#pragma unroll
        for (int r = 0; r < JP; ++r) {
            const int64_t off = (bh * DK + rg * JP + r) * p.dv + i;
            if (p.lam_T) p.lam_T[off] = 1.0f / sig[r];
            if (p.mu_T) p.mu_T[off] = Am * mt[r];
        }
    }
}

// Waves per workgroup: 64 value columns per workgroup where d_v allows.
constexpr int noise_waves(int DK, int64_t dv) {
    const int cpw = kWave / (DK / kNoiseRows);
    const int64_t cols = dv < 64 ? dv : 64;
    const int64_t w = (cols + cpw - 1) / cpw;
    return static_cast<int>(w < 1 ? 1 : w);
}

template <int DK, int W, bool BF16>
static void noise_one(const NoiseParams& p, int64_t BH, hipStream_t st) {
    constexpr int CI = W * (kWave / (DK / kNoiseRows));
    const int64_t grid = BH * ((p.dv + CI - 1) / CI);
    hipLaunchKernelGGL((k_diag_noise<DK, W, BF16>), dim3(static_cast<uint32_t>(grid)), dim3(W * kWave), 0, st, p);
}

// W runs up to d_k / 16 (64 columns of d_k / 16 row groups each).
template <int DK, bool BF16>
static int noise_dk(const NoiseParams& p, int64_t BH, hipStream_t st) {
    constexpr int WMAX = DK / kNoiseRows;
    const int w = noise_waves(DK, p.dv);
    if (w == 1) noise_one<DK, 1, BF16>(p, BH, st);
    else if (w == 2 && WMAX >= 2) noise_one<DK, (WMAX >= 2 ? 2 : 1), BF16>(p, BH, st);
    else if (w == 4 && WMAX >= 4) noise_one<DK, (WMAX >= 4 ? 4 : 1), BF16>(p, BH, st);
    else if (w == 8 && WMAX >= 8) noise_one<DK, (WMAX >= 8 ? 8 : 1), BF16>(p, BH, st);
    else return KDN_EUNSUPPORTED;
    return KDN_OK;
}

template <bool BF16>
static int noise_main(const NoiseParams& p, int64_t dk, int64_t BH, hipStream_t st) {
    switch (dk) {
        case 16: return noise_dk<16, BF16>(p, BH, st);
        case 32: return noise_dk<32, BF16>(p, BH, st);
        case 64: return noise_dk<64, BF16>(p, BH, st);
        case 128: return noise_dk<128, BF16>(p, BH, st);
        default: return KDN_EUNSUPPORTED;
    }
}

// T == 0: the final state is the starting state.
__global__ __launch_bounds__(256) void k_noise_copy(NoiseParams p, int64_t n) {
    for (int64_t e = elem_first(); e < n; e += elem_stride()) {
        if (p.lam_T) p.lam_T[e] = p.lam0 ? p.lam0[e] : 1.0f;
        if (p.mu_T) p.mu_T[e] = p.mu0 ? p.mu0[e] : 0.0f;
    }
}

int noise_launch(const NoiseParams& p, int64_t B, int64_t dk, bool bf16, hipStream_t st) {
    const int64_t BH = B * p.H;
    if (BH == 0) return KDN_OK;
    if (p.T == 0) {
        const int64_t n = BH * dk * p.dv;
        hipLaunchKernelGGL(k_noise_copy, dim3(elem_groups(n)), dim3(256), 0, st, p, n);
        return launch_status();
    }
    const int rc = bf16 ? noise_main<true>(p, dk, BH, st) : noise_main<false>(p, dk, BH, st);
    if (rc != KDN_OK) return rc;
    return launch_status();
}

}  // namespace kdn

// diag_scan.hip -- diagonal-precision memory scan, forward.
//
// Recurrence (Palimpsa, "Learning to Remember, Learn, and Forget in
// Attention-Based Models", Metodologia 1-2), per head and memory entry [j][i]:
//   alpha_t = exp(-A d_t)
//   I_t  = alpha_t I_{t-1} + (1 - alpha_t) I_prior + beta_t[i] k_t[j]^2
//   mu_t = alpha_t (I_{t-1}/I_t) mu_{t-1} + beta_t[i] v_t[i] k_t[j] / I_t
//   o_t[i] = sum_j q_t[j] mu_t[j][i]      (query read-out, KLA Metodologia 1)
//
// The kernels carry the information-form mean eta = I (.) mu instead of mu:
// multiplying the mu update by I_t gives eta_t = alpha_t eta_{t-1} +
// beta_t[i] v_t[i] k_t[j], which is affine like the precision update (the KLA
// summary, Metodologia 2, makes the same observation for its information
// mean).  mu_t = eta_t / I_t is formed only where it is read.
//
// Work decomposition (one GPU):
//   * a workgroup owns one head (b,h), one tile of CI value columns and one
//     sequence segment; lane <-> value column i, and each lane keeps JP key
//     rows j of (I, eta) in VGPRs for the whole segment;
//   * tokens are staged C at a time into LDS (double-buffered, converted to
//     fp32, k^2 precomputed) while the next chunk's global loads are in
//     flight; per-token partial read-outs from the P row groups are summed
//     through LDS once per chunk;
//   * long sequences are cut into S segments: a composite pass computes, from
//     a zero state, each segment's decay product and (J, eta) contribution
//     (J = I - I_prior obeys J_t = alpha_t J_{t-1} + beta k^2); a carry pass
//     combines them in order, (G2, X2) o (G1, X1) = (G2 G1, G2 X1 + X2), into
//     every segment's starting state; the main pass then runs all segments
//     in parallel.  The association is the one that makes the precision and
//     information-mean updates scannable (KLA Metodologia 2).
#include "kdn_params.h"

#include <type_traits>

namespace kdn {


// Kernel modes.  DIAG: diagonal precision (I, eta) with read-out.  ISO: the
// gated affine mean of the isotropic filter, mu_t = F_t mu_{t-1} + G_t k v^T
// (KLA Metodologia 2-3), with read-out.  The _COMP variants compute segment
// composites from a zero state, without read-out.
enum Mode { DIAG = 0, DIAG_COMP = 1, ISO = 2, ISO_COMP = 3 };

// Token bounds of segment `seg`: whole chunks [seg*n/S, (seg+1)*n/S).
__device__ __forceinline__ void segment_tokens(const DiagParams& p, int C, int seg,
                                               int64_t& t0, int64_t& t1) {
    const int64_t c0 = static_cast<int64_t>(seg) * p.nchunks / p.S;
    const int64_t c1 = static_cast<int64_t>(seg + 1) * p.nchunks / p.S;
    t0 = c0 * C;
    t1 = c1 * C < p.T ? c1 * C : p.T;
}

template <int DK, int CI, int W, int C, bool BF16, int MODE>
__global__ __launch_bounds__(W * kWave) void k_diag(DiagParams p) {
    constexpr bool COMPOSITE = (MODE & 1) != 0;
    constexpr bool ISO_M = MODE >= ISO;
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int NTH = W * kWave;
    constexpr int P = NTH / CI;          // row groups per workgroup
    constexpr int JP = DK / P;           // key rows per lane
    constexpr int VW = BF16 ? 8 : 4;     // elements per 16-byte vector
    constexpr int VK = C * DK / VW;      // vectors of k (and q) per chunk
    constexpr int VB = C * CI / VW;      // vectors of beta (and v) per chunk
    constexpr int NVK = (VK + NTH - 1) / NTH;
    constexpr int NVB = (VB + NTH - 1) / NTH;
    static_assert(NTH % CI == 0 && DK % P == 0 && JP % 4 == 0, "tile shape");
    static_assert(C <= NTH, "one thread per token for the gates");
    static_assert(!(ISO_M && BF16), "isotropic inputs are fp32");

    __shared__ float s_k[2][C][DK];
    __shared__ float s_k2[2][ISO_M ? 1 : C][DK];
    __shared__ float s_q[2][COMPOSITE ? 1 : C][DK];
    __shared__ float s_b[2][ISO_M ? 1 : C][CI];
    __shared__ float s_v[2][C][CI];
    __shared__ float s_a[2][C];
    __shared__ float s_c[2][C];
    __shared__ float s_o[2][COMPOSITE ? 1 : C][P][CI];

    const int tid = threadIdx.x;
    const int col = tid % CI;
    const int rg = tid / CI;
    const int j0 = rg * JP;
    const int ntile = static_cast<int>(p.dv / CI);
    const int nseg = COMPOSITE ? p.S - 1 : p.S;
    int64_t wg = blockIdx.x;
    const int tile = static_cast<int>(wg % ntile);
    wg /= ntile;
    const int seg = static_cast<int>(wg % nseg);
    const int64_t bh = wg / nseg;
    const int h = static_cast<int>(bh % p.H);
    const int i = tile * CI + col;

    int64_t t_begin, t_end;
    segment_tokens(p, C, seg, t_begin, t_end);

    const float A = ISO_M ? 0.0f : p.A[h];
    const float I_prior = p.I_prior;
    const E* qh = static_cast<const E*>(p.q) + bh * p.T * DK;
    const E* kh = static_cast<const E*>(p.k) + bh * p.T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * p.T * p.dv + tile * CI;
    const E* bth = ISO_M ? nullptr : static_cast<const E*>(p.beta) + bh * p.T * p.dv + tile * CI;
    const E* dh = ISO_M ? nullptr : static_cast<const E*>(p.d) + bh * p.T;
    const float* Fh = ISO_M ? p.F + bh * p.T : nullptr;
    const float* Gh = ISO_M ? p.G + bh * p.T : nullptr;

    // ---- state, JP key rows per lane: I (J in DIAG_COMP; unused in ISO) and eta
    //      (the information mean in DIAG, the mean itself in ISO) ----
    float I[JP], eta[JP];
    float gprod = 1.0f;
    if constexpr (COMPOSITE) {
#pragma unroll
        for (int r = 0; r < JP; ++r) { I[r] = 0.0f; eta[r] = 0.0f; }
    } else {
        if (p.S == 1) {
#pragma unroll
            for (int r = 0; r < JP; ++r) {
                const int64_t off = (bh * DK + j0 + r) * p.dv + i;
                const float m0 = p.mu0 ? p.mu0[off] : 0.0f;
                if constexpr (ISO_M) {
                    I[r] = 1.0f;
                    eta[r] = m0;
                } else {
                    const float I0 = p.I0 ? p.I0[off] : I_prior;
                    I[r] = I0;
                    eta[r] = I0 * m0;
                }
            }
        } else {
            const float* cin = p.comp + ((bh * p.S + seg) * 2) * DK * p.dv;
#pragma unroll
            for (int r = 0; r < JP; ++r) {
                const int64_t off = static_cast<int64_t>(j0 + r) * p.dv + i;
                I[r] = ISO_M ? 1.0f : I_prior + cin[off];
                eta[r] = cin[static_cast<int64_t>(DK) * p.dv + off];
            }
        }
    }

    // ---- chunk staging: global -> registers -> LDS (fp32) ----
    uint4 rk[NVK], rq[NVK], rb[NVB], rv[NVB];
    float rd = 0.0f, rg2 = 0.0f;

    auto fetch = [&](int64_t t0, int L) {
#pragma unroll
        for (int n = 0; n < NVK; ++n) {
            const int vi = tid + n * NTH;
            if (vi < VK && vi * VW < L * DK) {
                rk[n] = ld16(kh + t0 * DK + static_cast<int64_t>(vi) * VW);
                if constexpr (!COMPOSITE) rq[n] = ld16(qh + t0 * DK + static_cast<int64_t>(vi) * VW);
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int cv = vi % (CI / VW);
            if (vi < VB && row < L) {
                const int64_t off = (t0 + row) * p.dv + cv * VW;
                if constexpr (!ISO_M) rb[n] = ld16(bth + off);
                rv[n] = ld16(vh + off);
            }
        }
        if (tid < L) {
            if constexpr (ISO_M) {
                rd = Fh[t0 + tid];
                rg2 = Gh[t0 + tid];
            } else if constexpr (BF16) {
                rd = bf16_at(reinterpret_cast<const uint16_t*>(dh), t0 + tid);
            } else {
                rd = reinterpret_cast<const float*>(dh)[t0 + tid];
            }
        }
    };

    auto commit = [&](int nb, int L) {
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
                    s_k[nb][row][c0 + e] = f[e];
                    if constexpr (!ISO_M) s_k2[nb][row][c0 + e] = f[e] * f[e];
                }
                if constexpr (!COMPOSITE) {
                    widen<BF16>(rq[n], f);
#pragma unroll
                    for (int e = 0; e < VW; ++e) s_q[nb][row][c0 + e] = f[e];
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int c0 = (vi % (CI / VW)) * VW;
            if (vi < VB && row < L) {
                float f[VW];
                if constexpr (!ISO_M) {
                    widen<BF16>(rb[n], f);
#pragma unroll
                    for (int e = 0; e < VW; ++e) s_b[nb][row][c0 + e] = f[e];
                }
                widen<BF16>(rv[n], f);
#pragma unroll
                for (int e = 0; e < VW; ++e) s_v[nb][row][c0 + e] = f[e];
            }
        }
        if (tid < L) {
            if constexpr (ISO_M) {
                s_a[nb][tid] = rd;    // F_t
                s_c[nb][tid] = rg2;   // G_t
            } else {
                const float alpha = fast_exp(-A * rd);
                s_a[nb][tid] = alpha;
                s_c[nb][tid] = (1.0f - alpha) * I_prior;
            }
        }
    };

    const int64_t nch = (t_end - t_begin + C - 1) / C;
    auto chunk_len = [&](int64_t c) -> int {
        const int64_t rem = t_end - (t_begin + c * C);
        return static_cast<int>(rem < C ? rem : C);
    };

    if (nch > 0) {
        fetch(t_begin, chunk_len(0));
        commit(0, chunk_len(0));
    }
    __syncthreads();
    if (nch > 1) fetch(t_begin + C, chunk_len(1));

    for (int64_t c = 0; c < nch; ++c) {
        const int b = static_cast<int>(c & 1);
        const int L = chunk_len(c);
        const int64_t t0 = t_begin + c * C;

        for (int tt = 0; tt < L; ++tt) {
            const float a = s_a[b][tt];
            const float cc = s_c[b][tt];
            float bi = 0.0f, bvi;
            if constexpr (ISO_M) {
                bvi = cc * s_v[b][tt][col];          // G_t v_t[i]
            } else {
                bi = s_b[b][tt][col];
                bvi = bi * s_v[b][tt][col];          // beta_t[i] v_t[i]
            }
            float acc = 0.0f;
#pragma unroll
            for (int jj = 0; jj < JP; jj += 4) {
                const float4 kk = *reinterpret_cast<const float4*>(&s_k[b][tt][j0 + jj]);
                const float kv[4] = {kk.x, kk.y, kk.z, kk.w};
                float k2v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (!ISO_M) {
                    const float4 k2 = *reinterpret_cast<const float4*>(&s_k2[b][tt][j0 + jj]);
                    k2v[0] = k2.x; k2v[1] = k2.y; k2v[2] = k2.z; k2v[3] = k2.w;
                }
                float qv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (!COMPOSITE) {
                    const float4 qq = *reinterpret_cast<const float4*>(&s_q[b][tt][j0 + jj]);
                    qv[0] = qq.x; qv[1] = qq.y; qv[2] = qq.z; qv[3] = qq.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (MODE == DIAG) {
                        const float w = __builtin_fmaf(bi, k2v[e], cc);
                        I[jj + e] = __builtin_fmaf(a, I[jj + e], w);
                        eta[jj + e] = __builtin_fmaf(a, eta[jj + e], bvi * kv[e]);
                        const float m = eta[jj + e] * fast_rcp(I[jj + e]);
                        acc = __builtin_fmaf(qv[e], m, acc);
                    } else if constexpr (MODE == DIAG_COMP) {
                        I[jj + e] = __builtin_fmaf(a, I[jj + e], bi * k2v[e]);
                        eta[jj + e] = __builtin_fmaf(a, eta[jj + e], bvi * kv[e]);
                    } else if constexpr (MODE == ISO) {
                        eta[jj + e] = __builtin_fmaf(a, eta[jj + e], bvi * kv[e]);
                        acc = __builtin_fmaf(qv[e], eta[jj + e], acc);
                    } else {
                        eta[jj + e] = __builtin_fmaf(a, eta[jj + e], bvi * kv[e]);
                    }
                }
            }
            if constexpr (COMPOSITE) gprod *= a;
            else s_o[b][tt][rg][col] = acc;
        }

        if (c + 1 < nch) commit(b ^ 1, chunk_len(c + 1));
        __syncthreads();
        if constexpr (!COMPOSITE) {
            for (int e = tid; e < L * CI; e += NTH) {
                const int tt = e / CI;
                const int cc = e % CI;
                float sum = 0.0f;
#pragma unroll
                for (int g = 0; g < P; ++g) sum += s_o[b][tt][g][cc];
                p.o[(bh * p.T + t0 + tt) * p.dv + tile * CI + cc] = sum;
            }
        }
        if (c + 2 < nch) fetch(t0 + 2 * C, chunk_len(c + 2));
    }

    if constexpr (COMPOSITE) {
        float* cj = p.comp + ((bh * p.S + seg) * 2) * DK * p.dv;
#pragma unroll
        for (int r = 0; r < JP; ++r) {
            const int64_t off = static_cast<int64_t>(j0 + r) * p.dv + i;
            cj[off] = I[r];
            cj[static_cast<int64_t>(DK) * p.dv + off] = eta[r];
        }
        if (tid == 0 && tile == 0) p.gdec[bh * p.S + seg] = gprod;
    } else if (seg == p.S - 1) {
#pragma unroll
        for (int r = 0; r < JP; ++r) {
            const int64_t off = (bh * DK + j0 + r) * p.dv + i;
            if constexpr (ISO_M) {
                if (p.mu_T) p.mu_T[off] = eta[r];
            } else {
                if (p.I_T) p.I_T[off] = I[r];
                if (p.mu_T) p.mu_T[off] = eta[r] / I[r];
            }
        }
    }
}

// Carry pass: in order over segments, turn each segment's composite into the
// state it starts from.  One thread per memory entry of every head.
__global__ __launch_bounds__(256) void k_diag_carry(DiagParams p, int64_t dk, int64_t n_total, int iso) {
    const int64_t n_per_head = dk * p.dv;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= n_total) return;
    const int64_t bh = e / n_per_head;
    const int64_t r = e % n_per_head;
    const int64_t off = bh * n_per_head + r;
    const float m0 = p.mu0 ? p.mu0[off] : 0.0f;
    float J = 0.0f, eta;
    if (iso) {
        eta = m0;
    } else if (p.I0) {
        const float I0 = p.I0[off];
        J = I0 - p.I_prior;
        eta = I0 * m0;
    } else {
        eta = p.I_prior * m0;
    }
    for (int s = 0; s < p.S; ++s) {
        float* slot = p.comp + ((bh * p.S + s) * 2) * n_per_head;
        float Js = 0.0f, es = 0.0f, G = 1.0f;
        if (s + 1 < p.S) {
            Js = slot[r];
            es = slot[n_per_head + r];
            G = p.gdec[bh * p.S + s];
        }
        slot[r] = J;
        slot[n_per_head + r] = eta;
        J = __builtin_fmaf(G, J, Js);
        eta = __builtin_fmaf(G, eta, es);
    }
}

// T == 0: the final state is the starting state.
__global__ __launch_bounds__(256) void k_diag_copy_state(DiagParams p, int64_t n, int iso) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= n) return;
    const float m0 = p.mu0 ? p.mu0[e] : 0.0f;
    if (!iso && p.I_T) p.I_T[e] = p.I0 ? p.I0[e] : p.I_prior;
    if (p.mu_T) p.mu_T[e] = m0;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

constexpr int kDiagChunk = 16;

// Workgroup width for a (DK, CI) tile: enough waves that each lane keeps
// 16 key rows when the tile is large, never fewer than one wave.
constexpr int diag_waves(int DK, int CI) {
    const int w = DK * CI / (kWave * 16);
    return w < 1 ? 1 : w;
}

template <int DK, int CI, bool BF16, int MODE>
static void launch_one(const DiagParams& p, int64_t grid, hipStream_t st) {
    constexpr int W = diag_waves(DK, CI);
    hipLaunchKernelGGL((k_diag<DK, CI, W, kDiagChunk, BF16, MODE>), dim3(static_cast<uint32_t>(grid)),
                       dim3(W * kWave), 0, st, p);
}

template <int DK, bool BF16, int MODE>
static int launch_dk(const DiagParams& p, int CI, int64_t grid, hipStream_t st) {
    switch (CI) {
        case 16: launch_one<DK, 16, BF16, MODE>(p, grid, st); break;
        case 32: launch_one<DK, 32, BF16, MODE>(p, grid, st); break;
        case 64: launch_one<DK, 64, BF16, MODE>(p, grid, st); break;
        default: return KDN_EUNSUPPORTED;
    }
    return KDN_OK;
}

template <bool BF16, int MODE>
static int launch_mode(const DiagParams& p, int64_t dk, int CI, int64_t grid, hipStream_t st) {
    switch (dk) {
        case 16: return launch_dk<16, BF16, MODE>(p, CI, grid, st);
        case 32: return launch_dk<32, BF16, MODE>(p, CI, grid, st);
        case 64: return launch_dk<64, BF16, MODE>(p, CI, grid, st);
        case 128: return launch_dk<128, BF16, MODE>(p, CI, grid, st);
        default: return KDN_EUNSUPPORTED;
    }
}

int diag_chunk() { return kDiagChunk; }

// Enqueue a whole segmented scan (diagonal precision, or the isotropic gated
// mean when iso is set).  Arguments were validated by the caller; comp/gdec
// point into a workspace of the size the planner reported when S > 1.
int diag_scan_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, bool iso, hipStream_t st) {
    const int64_t BH = B * p.H;
    if (BH == 0) return KDN_OK;
    if (p.T == 0) {
        const int64_t n = BH * dk * p.dv;
        hipLaunchKernelGGL(k_diag_copy_state, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st,
                           p, n, iso ? 1 : 0);
        return launch_status();
    }
    const int CI = p.dv < 64 ? static_cast<int>(p.dv) : 64;
    const int64_t ntile = p.dv / CI;
    int rc = KDN_OK;
    if (p.S > 1) {
        const int64_t g1 = BH * (p.S - 1) * ntile;
        if (iso) rc = launch_mode<false, ISO_COMP>(p, dk, CI, g1, st);
        else rc = bf16 ? launch_mode<true, DIAG_COMP>(p, dk, CI, g1, st)
                       : launch_mode<false, DIAG_COMP>(p, dk, CI, g1, st);
        if (rc != KDN_OK) return rc;
        if ((rc = launch_status()) != KDN_OK) return rc;
        const int64_t n = BH * dk * p.dv;
        hipLaunchKernelGGL(k_diag_carry, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, st,
                           p, dk, n, iso ? 1 : 0);
        if ((rc = launch_status()) != KDN_OK) return rc;
    }
    const int64_t g2 = BH * p.S * ntile;
    if (iso) rc = launch_mode<false, ISO>(p, dk, CI, g2, st);
    else rc = bf16 ? launch_mode<true, DIAG>(p, dk, CI, g2, st) : launch_mode<false, DIAG>(p, dk, CI, g2, st);
    if (rc != KDN_OK) return rc;
    return launch_status();
}

}  // namespace kdn

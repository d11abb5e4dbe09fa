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
//     rows j of (I, eta) in VGPRs for the whole segment, in a scaled frame
//     (below) so both updates are plain accumulations;
//   * tokens are staged C at a time into LDS (double-buffered, converted to
//     fp32, k^2 precomputed) while the next chunk's global loads are in
//     flight; the per-token frame scalars come from a small prep kernel; the
//     key-side values of a lane's rows reach the fmacs as DPP row broadcasts;
//     per-token partial read-outs of the P row groups are summed through LDS
//     once per chunk;
//   * long sequences are cut into S segments whose starting states come from
//     segment composites computed on the matrix cores and carried in order
//     (diag_comp.hip); all segments then run in parallel.
#include "kdn_lane.h"
#include "kdn_params.h"

namespace kdn {

// Scaled frame.  Between renormalisations the kernel keeps I~ = s_t I_t and
// eta~ = s_t eta_t, where s_t = prod(1/alpha) since the frame's start token.
// Per token and entry that turns both updates into accumulations:
//   I~  += beta_i s_t k_j^2 + (1 - alpha_t) I_prior s_t,   eta~ += beta_i v_i s_t k_j,
// and mu = eta~ / I~ needs no scale at all.  A frame starts at every chunk's
// first token and wherever s would pass e^kFrameLog; at a start the state is
// multiplied by rho_t = alpha_t / s_{t-1} and s restarts at 1.
constexpr float kFrameLog = 30.0f;

template <int DK, int CI, int W, int C, bool BF16>
__global__ __launch_bounds__(W * kWave) void k_diag(DiagParams p) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int NTH = W * kWave;
    constexpr int P = NTH / CI;          // row groups per workgroup
    constexpr int JP = DK / P;           // key rows per lane
    constexpr int VW = BF16 ? 8 : 4;     // elements per 16-byte vector
    constexpr int VK = C * DK / VW;      // vectors of k (and q) per chunk
    constexpr int VB = C * CI / VW;      // vectors of beta (and v) per chunk
    constexpr int NVK = (VK + NTH - 1) / NTH;
    constexpr int NVB = (VB + NTH - 1) / NTH;
    static_assert(NTH % CI == 0 && DK % P == 0, "tile shape");
    static_assert(JP == 4 || JP == 8 || JP == 16, "key rows per lane: one DPP row");
    static_assert(CI >= 16, "a DPP row must stay inside one row group");
    static_assert(C == 16, "per-token scalars are scanned across 16 lanes");
    // k^2 is staged next to k where the LDS allows it; a workgroup of fewer
    // than 8 waves must leave room for a second one on its CU (80 KB), and
    // then squares k per token instead (one multiply per token and lane).
    constexpr int kLdsK2 = 2 * (3 * C * DK + 2 * C * CI) * 4 + 2 * C * P * CI * 4;
    constexpr bool K2 = W >= 8 || kLdsK2 <= 80 * 1024;

    struct Stage {
        float k[C][DK];
        float k2[K2 ? C : 1][DK];
        float q[C][DK];
        float2 bv[C][CI];   // (beta_i, v_i)
    };
    __shared__ Stage stg[2];
    __shared__ float opart[2][C][P][CI];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int col = tid % CI;
    const int rg = tid / CI;
    const int j0 = rg * JP;
    const int jl = j0 + (lane & (JP - 1));   // the key row this lane holds for broadcasts
    const int ntile = static_cast<int>(p.dv / CI);
    // Packed variable-length batch: workgroups go out in blockIdx order, so
    // runs are numbered to follow the plan's longest-first order (the longest
    // sequences start first, the short ones fill in behind), in groups of
    // 8 runs x ntile tiles where a run's tiles are 8 blocks apart and so land
    // on the same XCD (blocks are dealt to the 8 XCDs round-robin).
    // Otherwise XCD-local ids.
    int64_t wg;
    int tile;
    if (p.cu_seqlens) {
        const int64_t b = blockIdx.x;
        const int64_t within = b % (8 * ntile);
        tile = static_cast<int>(within / 8);
        wg = b / (8 * ntile) * 8 + within % 8;
    } else {
        wg = xcd_local_id();
        tile = static_cast<int>(wg % ntile);
        wg /= ntile;
    }
    const int i = tile * CI + col;
    // bh: head of the token inputs; sb: slot of this run's starting/final
    // state; cin: its carried-in starting state, or NULL for the run's own;
    // last: the run ends its sequence and writes the final state
    int seg;
    int32_t sq = -1;
    int64_t bh, sb, t_begin, t_end;
    const float* cin = nullptr;
    bool last;
    if (p.cu_seqlens) {
        // one segment (the whole sequence unless it is split) of one head
        VarlenItem it;
        if (!varlen_item(p, wg, it)) return;   // past the plan's items
        bh = it.bh;
        sb = it.sb;
        sq = it.sq;
        seg = it.seg;
        t_begin = it.t_begin;
        t_end = it.t_end;
        last = it.last;
        if (it.carry >= 0) cin = p.comp + ((it.carry * p.H + bh) * 2) * DK * p.dv;
    } else {
        seg = static_cast<int>(wg % p.S);
        bh = wg / p.S;
        sb = bh;
        segment_tokens(p, C, seg, t_begin, t_end);
        last = seg == p.S - 1;
        if (p.S > 1) cin = p.comp + ((bh * p.S + seg) * 2) * DK * p.dv;
    }
    if (tid == 0) echo_bounds(p, blockIdx.x, 1, sb, seg, tile, t_begin, t_end, sq);

    const float I_prior = p.I_prior;
    const E* qh = static_cast<const E*>(p.q) + bh * p.T * DK;
    const E* kh = static_cast<const E*>(p.k) + bh * p.T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * p.T * p.dv + tile * CI;
    // beta == NULL: Palimpsa-M gating, beta_t[i] = d_t
    const E* bth = p.beta ? static_cast<const E*>(p.beta) + bh * p.T * p.dv + tile * CI : nullptr;
    const E* dh = static_cast<const E*>(p.d) + bh * p.T;

    // ---- state, JP key rows per lane, in the scaled frame with s = 1 at the
    //      segment start: I~ and the information mean eta~ ----
    float I[JP], eta[JP];
    if (!cin) {
#pragma unroll
        for (int r = 0; r < JP; ++r) {
            const int64_t off = (sb * DK + j0 + r) * p.dv + i;
            const float m0 = p.mu0 ? p.mu0[off] : 0.0f;
            const float I0 = p.I0 ? p.I0[off] : I_prior;
            I[r] = I0;
            eta[r] = I0 * m0;
        }
    } else {
#pragma unroll
        for (int r = 0; r < JP; ++r) {
            const int64_t off = static_cast<int64_t>(j0 + r) * p.dv + i;
            I[r] = I_prior + cin[off];
            eta[r] = cin[static_cast<int64_t>(DK) * p.dv + off];
        }
    }

    // ---- chunk staging: global -> registers -> LDS (fp32) ----
    uint4 rk[NVK], rq[NVK], rb[NVB], rv[NVB];
    float s_prev = 1.0f;   // scale of the last token of the previous chunk (uniform)
    const float4* sch = p.scal + bh * p.T;
    // The per-token frame scalars (rho, dP, s, -) are read through the scalar
    // cache: their addresses are uniform, so they land in SGPRs and feed the
    // VALU as scalar operands with no LDS staging and no readfirstlane.
    typedef __attribute__((address_space(4))) const float scalar_f32;
    auto frame_scalars = [&](int64_t t0) { return (scalar_f32*)(uintptr_t)(sch + t0); };

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
                rb[n] = bth ? ld16(bth + off) : splat16<BF16>(dh, t0 + row);
                rv[n] = ld16(vh + off);
            }
        }
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
                    if constexpr (K2) S.k2[row][c0 + e] = f[e] * f[e];
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
        const Stage& S = stg[b];
        const float inv_sp = 1.0f / s_prev;   // a chunk's first token restarts the frame

        scalar_f32* const cs = frame_scalars(t0);
        // One token: frame change, state update, read-out partial.  bvv, vk,
        // vk2, vq are the token's operands from the stage.
        auto token = [&](int tt, const float2 bvv, const float vk, const float vk2,
                         const float vq) __attribute__((always_inline)) {
            const float s_t = cs[4 * tt + 2];
            const uint32_t rho_bits = tt == 0 ? __builtin_amdgcn_readfirstlane(__float_as_uint(cs[0] * inv_sp))
                                              : __float_as_uint(cs[4 * tt]);
            if (rho_bits != 0x3f800000u) {
                const float rho = __uint_as_float(rho_bits);
#pragma unroll
                for (int r = 0; r < JP; ++r) {
                    I[r] *= rho;
                    eta[r] *= rho;
                }
            }
            const float bs = bvv.x * s_t;            // beta_i s_t
            const float bvs = bs * bvv.y;            // beta_i v_i s_t
            Unroll<0, JP>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                fmac_bcast<r>(I[r], vk2, bs);
            });
            const float dP = cs[4 * tt + 1];
#pragma unroll
            for (int r = 0; r < JP; ++r) I[r] += dP;
            Unroll<0, JP>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                fmac_bcast<r>(eta[r], vk, bvs);
            });
            float m[JP];
#pragma unroll
            for (int r = 0; r < JP; ++r) m[r] = eta[r] * fast_rcp(I[r]);
            // four read-out accumulators, each started by a broadcast multiply
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
        };

        if (L == C) {
            // a whole chunk: unrolled, so every stage offset is a constant and
            // the compiler schedules the operand reads ahead by itself
            Unroll<0, C>::run([&](auto u) {
                constexpr int tt = decltype(u)::value;
                const float vk = S.k[tt][jl];
                float vk2;
                if constexpr (K2) vk2 = S.k2[tt][jl];
                else vk2 = dpp_src(vk * vk);
                token(tt, S.bv[tt][col], vk, vk2, S.q[tt][jl]);
            });
        } else {
            // the ragged last chunk, software-pipelined over tokens: the next
            // token's LDS operands are loaded while the current one computes
            float2 bvv = S.bv[0][col];
            float vk = S.k[0][jl], vk2, vq = S.q[0][jl];
            if constexpr (K2) vk2 = S.k2[0][jl];
            else vk2 = dpp_src(vk * vk);
            for (int tt = 0; tt < L; ++tt) {
                const int tn = tt + 1 < L ? tt + 1 : tt;
                const float2 bvv_n = S.bv[tn][col];
                const float vk_n = S.k[tn][jl], vq_n = S.q[tn][jl];
                float vk2_n;
                if constexpr (K2) vk2_n = S.k2[tn][jl];
                else vk2_n = dpp_src(vk_n * vk_n);
                token(tt, bvv, vk, vk2, vq);
                bvv = bvv_n;
                vk = vk_n;
                vk2 = vk2_n;
                vq = vq_n;
            }
        }

        s_prev = cs[4 * (L - 1) + 2];
        if (c + 1 < nch) commit(b ^ 1, chunk_len(c + 1));
        __syncthreads();
        for (int e = tid; e < L * CI; e += NTH) {
            const int tt = e / CI;
            const int cc = e % CI;
            float sum = 0.0f;
#pragma unroll
            for (int g = 0; g < P; ++g) sum += opart[b][tt][g][cc];
            p.o[(bh * p.T + t0 + tt) * p.dv + tile * CI + cc] = sum;
        }
        if (c + 2 < nch) fetch(t0 + 2 * C, chunk_len(c + 2));
    }

    // back from the scaled frame: true state = scaled state / s_last
    const float s_last = s_prev;
    if (last) {
#pragma unroll
        for (int r = 0; r < JP; ++r) {
            const int64_t off = (sb * DK + j0 + r) * p.dv + i;
            if (p.I_T) p.I_T[off] = I[r] / s_last;
            if (p.mu_T) p.mu_T[off] = eta[r] / I[r];
        }
    }
}

// The scan for 64-column tiles, with a block of RB key rows x 2 value columns
// per lane and every multiplicand in a VGPR.  A wave holds 2*RB key rows:
// lanes 0-31 the first RB, lanes 32-63 the next RB, lane l % 32 the column
// pair (2c, 2c+1).  At d_k = 128, RB = 4 gives 16-wave workgroups, four waves
// per SIMD: a 64-column tile of a head is all the work one workgroup has.
//
// Frames.  The precision is kept in true units: with the decay alpha_t and
// the prior increment P_t = (1 - alpha_t) I_prior from the frame-scalar pass,
//   I = fma(I, alpha_t, P_t),   I = fma(k_j^2, beta_i, I)
// costs the same two instructions as an update in a scaled frame, and needs
// no rescale when a frame restarts.  The information mean is kept scaled,
// eta~ = s_t eta (s_t as in k_diag), so its update is one fmac with s_t k_j
// staged; the read-out divides by s_t through the staged query q_j / s_t.
// The eta frame restarts at every chunk's first token; a chunk with no other
// restart (the usual case: s stays below e^kFrameLog for 16 tokens) applies
// that rescale before its tokens and runs them unrolled with no per-token
// branch, any other chunk checks every token.
//
// Read-out.  sum_j q_j mu_j over a lane's key rows is taken four rows at a
// time with one reciprocal: for rows a, b, c, d of a column,
//   q_a e_a / I_a + q_b e_b / I_b = (q_a e_a I_b + q_b e_b I_a) / (I_a I_b) = n_ab / d_ab,
//   n_ab / d_ab + n_cd / d_cd = (n_ab d_cd + n_cd d_ab) / (d_ab d_cd),
// 14 full-rate instructions and one v_rcp_f32 per four entries in place of
// four reciprocals, four multiplies and four fmacs (measured on gfx950, the
// reciprocal issues at about a quarter of the full rate).  The products of
// four precisions must stay in range, so the grouped form runs only where
//   * every precision of the wave is at least 2^-24 (checked once: I never
//     falls below min(I_0, I_prior)), and
//   * every precision stays below 2^24 through the chunk: checked per chunk
//     from the wave's largest precision at the chunk start plus the largest
//     growth 16 tokens can bring, I_prior + 16 max(beta) max(k^2), with the
//     maxima running over every token staged so far;
// and a token whose grouped read-out is not finite (a numerator past the
// fp32 range) is read out again one reciprocal per entry.  Elsewhere the
// read-out takes one reciprocal per entry.
//   * The two row blocks of a column are summed by one v_permlane32_swap;
//     the waves' partial read-outs go through LDS once per chunk, single-
//     buffered (with a second barrier) when 16 waves' worth would not fit
//     next to the stage.
template <int DK, int RB, int C, bool BF16>
__global__ __launch_bounds__(DK / (2 * RB) * kWave) void k_diag_blk(DiagParams p) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int CI = 64;
    constexpr int W = DK / (2 * RB);     // waves: 2*RB key rows each
    constexpr int NTH = W * kWave;
    constexpr int P = W;                 // row groups of the read-out: one per wave
    // Partial read-outs double-buffered (no second barrier per chunk) only
    // where two workgroups still fit in a CU's 160 KB of LDS: at d_k = 64 a
    // second buffer would leave one 8-wave workgroup per CU, half the waves.
    constexpr int kStageBytes = (3 * C * DK + 2 * C * CI + 4 * C + 4) * 4;
    constexpr int kPartBytes = C * P * CI * 4;
    constexpr int NOB = W <= 8 && 2 * (2 * kStageBytes + 2 * kPartBytes) <= 160 * 1024 ? 2 : 1;
    constexpr int VW = BF16 ? 8 : 4;
    constexpr int VK = C * DK / VW;
    constexpr int VB = C * CI / VW;
    // staging jobs of a chunk: VK vectors of k, VK of q, VB of (beta, v), dealt
    // to threads in that order, NJS per thread
    constexpr int NJ = 2 * VK + VB;
    constexpr int NJS = (NJ + NTH - 1) / NTH;
    static_assert(RB == 4 || RB == 8, "key rows per lane: whole groups of four");
    static_assert(DK % (2 * RB) == 0 && NTH <= 1024, "tile shape");
    static_assert(C == 16, "per-token scalars come in 16-token chunks");
    constexpr float kQuadHi = 16777216.0f;          // 2^24
    constexpr float kQuadLo = 1.0f / 16777216.0f;   // 2^-24

    struct Stage {
        float ks[C][DK];    // s_t k_t[j]
        float k2[C][DK];    // k_t[j]^2
        float q[C][DK];     // q_t[j] / s_t
        float2 bv[C][CI];   // (beta_i, beta_i v_i)
        float4 ap[C];       // (alpha_t, (1 - alpha_t) I_prior, rho_t of the eta frame, -)
        uint32_t restarts;  // bit t: token t restarts the eta frame (rho_t != 1)
    };
    static_assert(sizeof(Stage) == kStageBytes, "stage size used to choose the partial buffers");
    __shared__ Stage stg[2];
    __shared__ float opart[NOB][C][P][CI];
    // running maxima of k^2 and beta over every token staged so far, as the
    // bits of non-negative floats (which order like the floats)
    __shared__ uint32_t run_max[2];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = tid / kWave;
    const int half = lane / 32;          // which RB-row block of the wave's 2*RB rows
    const int cp = lane % 32;            // column pair
    const int j0 = wv * 2 * RB + half * RB;
    const int ocol = 2 * cp + half;      // the column whose read-out partial this lane ends with
    const int ntile = static_cast<int>(p.dv / CI);
    // Packed variable-length batch: runs follow the plan's longest-first
    // order in groups of 8 runs x ntile tiles, a run's tiles 8 blocks apart
    // (so on one XCD), as in k_diag.  Otherwise XCD-local ids.
    int64_t wg;
    int tile;
    if (p.cu_seqlens) {
        const int64_t blk = blockIdx.x;
        const int64_t within = blk % (8 * ntile);
        tile = static_cast<int>(within / 8);
        wg = blk / (8 * ntile) * 8 + within % 8;
    } else {
        wg = xcd_local_id();
        tile = static_cast<int>(wg % ntile);
        wg /= ntile;
    }
    const int i0 = tile * CI + 2 * cp;
    // bh: head of the token inputs; sb: slot of this run's starting/final
    // state; cin: its carried-in starting state, or NULL for the run's own;
    // last: the run ends its sequence and writes the final state
    int seg;
    int32_t sq = -1;
    int64_t bh, sb, t_begin, t_end;
    const float* cin = nullptr;
    bool last;
    if (p.cu_seqlens) {
        VarlenItem it;
        if (!varlen_item(p, wg, it)) return;   // past the plan's items
        bh = it.bh;
        sb = it.sb;
        sq = it.sq;
        seg = it.seg;
        t_begin = it.t_begin;
        t_end = it.t_end;
        last = it.last;
        if (it.carry >= 0) cin = p.comp + ((it.carry * p.H + bh) * 2) * DK * p.dv;
    } else {
        seg = static_cast<int>(wg % p.S);
        bh = wg / p.S;
        sb = bh;
        segment_tokens(p, C, seg, t_begin, t_end);
        last = seg == p.S - 1;
        if (p.S > 1) cin = p.comp + ((bh * p.S + seg) * 2) * DK * p.dv;
    }
    if (tid == 0) echo_bounds(p, blockIdx.x, 1, sb, seg, tile, t_begin, t_end, sq);

    const float I_prior = p.I_prior;
    const E* qh = static_cast<const E*>(p.q) + bh * p.T * DK;
    const E* kh = static_cast<const E*>(p.k) + bh * p.T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * p.T * p.dv + tile * CI;
    const E* bth = p.beta ? static_cast<const E*>(p.beta) + bh * p.T * p.dv + tile * CI : nullptr;
    const E* dh = static_cast<const E*>(p.d) + bh * p.T;

    // I in true units, eta~ = s eta with s = 1 at the segment start
    float I[RB][2], eta[RB][2];
    if (!cin) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t off = (sb * DK + j0 + r) * p.dv + i0;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float m0 = p.mu0 ? p.mu0[off + c] : 0.0f;
                const float I0 = p.I0 ? p.I0[off + c] : I_prior;
                I[r][c] = I0;
                eta[r][c] = I0 * m0;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t off = static_cast<int64_t>(j0 + r) * p.dv + i0;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                I[r][c] = I_prior + cin[off + c];
                eta[r][c] = cin[static_cast<int64_t>(DK) * p.dv + off + c];
            }
        }
    }
    // I never falls below min(I_0, I_prior): the grouped read-out's lower
    // bound holds for the whole run if it holds now
    bool quad_ok;
    {
        float lo = I_prior;
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c) lo = fminf(lo, I[r][c]);
        quad_ok = __builtin_amdgcn_ballot_w64(!(lo >= kQuadLo)) == 0;
    }

    // A thread's staging jobs: job j < VK is vector j of the chunk's k (its
    // s k and k^2), VK <= j < 2 VK vector j - VK of q (q / s), then (beta, v)
    // vectors; the jobs spread over 10 of the 16 waves at d_k = 128, so no
    // wave carries much staging into the chunk's barrier.
    uint4 ra[NJS], rb2[NJS];      // raw vectors (k, q or beta; v)
    float rs[NJS];                // s of the job's token (k and q jobs)
    // frame scalars (rho, P, s, A d) of token tid of the chunk (tid < C), and
    // for tid 0 the scale of the token before the chunk (1 at the run start)
    float4 rsc = make_float4(1.0f, 0.0f, 1.0f, 0.0f);
    float rsp = 1.0f;
    const float4* sch = p.scal + bh * p.T;
    // the running maxima as this wave last read them
    float seen_k = 0.0f, seen_b = 0.0f;

    auto fetch = [&](int64_t t0, int L) {
#pragma unroll
        for (int n = 0; n < NJS; ++n) {
            const int j = tid + n * NTH;
            if (j < VK) {
                if (j * VW < L * DK) {
                    ra[n] = ld16(kh + t0 * DK + static_cast<int64_t>(j) * VW);
                    rs[n] = sch[t0 + j * VW / DK].z;
                }
            } else if (j < 2 * VK) {
                const int vi = j - VK;
                if (vi * VW < L * DK) {
                    ra[n] = ld16(qh + t0 * DK + static_cast<int64_t>(vi) * VW);
                    rs[n] = sch[t0 + vi * VW / DK].z;
                }
            } else if (j < NJ) {
                const int vi = j - 2 * VK;
                const int row = vi / (CI / VW);
                const int cv = vi % (CI / VW);
                if (row < L) {
                    const int64_t off = (t0 + row) * p.dv + cv * VW;
                    ra[n] = bth ? ld16(bth + off) : splat16<BF16>(dh, t0 + row);
                    rb2[n] = ld16(vh + off);
                }
            }
        }
        if (tid < L) rsc = sch[t0 + tid];
        if (tid == 0) rsp = t0 > t_begin ? sch[t0 - 1].z : 1.0f;
    };

    auto commit = [&](int nb, int L) {
        Stage& S = stg[nb];
        float mk = 0.0f, mb = 0.0f;
#pragma unroll
        for (int n = 0; n < NJS; ++n) {
            const int j = tid + n * NTH;
            float f[VW];
            if (j < VK) {
                if (j * VW < L * DK) {
                    const int row = j * VW / DK;
                    const int c0 = j * VW % DK;
                    widen<BF16>(ra[n], f);
                    float ks[VW], k2[VW];
#pragma unroll
                    for (int e = 0; e < VW; ++e) {
                        ks[e] = f[e] * rs[n];
                        k2[e] = f[e] * f[e];
                        mk = fmaxf(mk, k2[e]);
                    }
                    store_run<VW>(&S.ks[row][c0], ks);
                    store_run<VW>(&S.k2[row][c0], k2);
                }
            } else if (j < 2 * VK) {
                const int vi = j - VK;
                if (vi * VW < L * DK) {
                    const int row = vi * VW / DK;
                    const int c0 = vi * VW % DK;
                    const float inv_s = fast_rcp(rs[n]);
                    widen<BF16>(ra[n], f);
#pragma unroll
                    for (int e = 0; e < VW; ++e) f[e] *= inv_s;
                    store_run<VW>(&S.q[row][c0], f);
                }
            } else if (j < NJ) {
                const int vi = j - 2 * VK;
                const int row = vi / (CI / VW);
                const int c0 = (vi % (CI / VW)) * VW;
                if (row < L) {
                    float fv[VW], bv[2 * VW];
                    widen<BF16>(ra[n], f);
                    widen<BF16>(rb2[n], fv);
#pragma unroll
                    for (int e = 0; e < VW; ++e) {
                        bv[2 * e] = f[e];
                        bv[2 * e + 1] = f[e] * fv[e];
                        mb = fmaxf(mb, f[e]);
                    }
                    store_run<2 * VW>(reinterpret_cast<float*>(&S.bv[row][c0]), bv);
                }
            }
        }
        // raise the running maxima only where this lane saw more (rarely,
        // once the first chunks are in)
        if (mk > seen_k) atomicMax(&run_max[0], __float_as_uint(mk));
        if (mb > seen_b) atomicMax(&run_max[1], __float_as_uint(mb));
        // per-token (alpha, P, rho): a chunk's first token restarts the eta
        // frame from the previous token's scale
        if (wv == 0) {
            const float rho = tid == 0 ? rsc.x / rsp : rsc.x;
            if (tid < L) S.ap[tid] = make_float4(fast_exp(-rsc.w), rsc.y, rho, 0.0f);
            const uint64_t m = __builtin_amdgcn_ballot_w64(tid < L && rho != 1.0f);
            if (tid == 0) S.restarts = static_cast<uint32_t>(m);
        }
    };

    const int64_t nch = (t_end - t_begin + C - 1) / C;
    auto chunk_len = [&](int64_t c) -> int {
        const int64_t rem = t_end - (t_begin + c * C);
        return static_cast<int>(rem < C ? rem : C);
    };

    if (tid < 2) run_max[tid] = 0u;
    __syncthreads();
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
        const Stage& S = stg[b];
        // A token's operands: RB key rows of s k, k^2 and q / s (shared by
        // half a wave), the lane's (beta, beta v) column pair and the token's
        // (alpha, P).
        struct Ops {
            float4 k[RB / 4], k2[RB / 4], q[RB / 4];
            float4 bv;
            float4 ap;
        };
        auto load_ops = [&](int tt) __attribute__((always_inline)) {
            Ops o;
            const float4* kp = reinterpret_cast<const float4*>(&S.ks[tt][j0]);
            const float4* k2p = reinterpret_cast<const float4*>(&S.k2[tt][j0]);
            const float4* qp = reinterpret_cast<const float4*>(&S.q[tt][j0]);
#pragma unroll
            for (int h = 0; h < RB / 4; ++h) {
                o.k[h] = kp[h];
                o.k2[h] = k2p[h];
                o.q[h] = qp[h];
            }
            o.bv = *reinterpret_cast<const float4*>(&S.bv[tt][2 * cp]);
            o.ap = S.ap[tt];
            return o;
        };
        // The chunk's first operands are read with its flags, so that their
        // latency overlaps the flag reads and the range check below (not at
        // d_k = 64 in fp32, whose registers would then exceed 128 and halve
        // the workgroups per CU).
        constexpr bool kFirstEarly = BF16 || DK == 128;
        Ops op0{};
        if constexpr (kFirstEarly) op0 = load_ops(0);
        const uint32_t restarts = __builtin_amdgcn_readfirstlane(S.restarts);

        // Grouped read-out for this chunk: every precision of the wave stays
        // below 2^24 if the largest now, or I_prior, plus the chunk's largest
        // growth does.
        bool quad;
        {
            seen_k = __uint_as_float(run_max[0]);
            seen_b = __uint_as_float(run_max[1]);
            const float lim = kQuadHi - static_cast<float>(C) * seen_k * seen_b;
            float hi = I_prior;
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) hi = fmaxf(hi, I[r][cc]);
            quad = quad_ok && __builtin_amdgcn_ballot_w64(!(hi + I_prior <= lim)) == 0;
        }

        auto lane_of = [](const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; };
        // read-out of column cc over the lane's RB rows, four rows per reciprocal
        auto readout_quad = [&](const Ops& o, int cc) __attribute__((always_inline)) {
            float acc = 0.0f;
#pragma unroll
            for (int g = 0; g < RB; g += 4) {
                const float4 qv = o.q[g / 4];
                const float Ia = I[g][cc], Ib = I[g + 1][cc], Ic = I[g + 2][cc], Id = I[g + 3][cc];
                float nab = qv.x * (eta[g][cc] * Ib);
                nab = __builtin_fmaf(qv.y, eta[g + 1][cc] * Ia, nab);
                float ncd = qv.z * (eta[g + 2][cc] * Id);
                ncd = __builtin_fmaf(qv.w, eta[g + 3][cc] * Ic, ncd);
                const float dab = Ia * Ib;
                const float dcd = Ic * Id;
                const float num = __builtin_fmaf(ncd, dab, nab * dcd);
                const float rq = fast_rcp(dab * dcd);
                acc = g == 0 ? num * rq : __builtin_fmaf(num, rq, acc);
            }
            return acc;
        };
        // the same with one reciprocal per entry
        auto readout_direct = [&](const Ops& o, int cc) __attribute__((always_inline)) {
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float qq = lane_of(o.q[r / 4], r % 4);
                const float m = eta[r][cc] * fast_rcp(I[r][cc]);
                acc = r == 0 ? qq * m : __builtin_fmaf(qq, m, acc);
            }
            return acc;
        };
        // One token from its operands: eta frame restart, state update,
        // read-out partial.
        auto token = [&](int tt, const Ops& o, bool mid_restarts) __attribute__((always_inline)) {
            if (mid_restarts && ((restarts >> tt) & 1u)) {
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) eta[r][cc] *= o.ap.z;
            }
            const float bet[2] = {o.bv.x, o.bv.z};
            const float bvv[2] = {o.bv.y, o.bv.w};
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float kk = lane_of(o.k[r / 4], r % 4);
                const float k2 = lane_of(o.k2[r / 4], r % 4);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    I[r][cc] = __builtin_fmaf(k2, bet[cc], __builtin_fmaf(I[r][cc], o.ap.x, o.ap.y));
                    eta[r][cc] = __builtin_fmaf(kk, bvv[cc], eta[r][cc]);
                }
            }
            float x = 0.0f;
            bool done = false;
            if (quad) {
                x = swap32_add(readout_quad(o, 0), readout_quad(o, 1));
                done = __builtin_amdgcn_ballot_w64(!__builtin_isfinite(x)) == 0;
            }
            if (!done) x = swap32_add(readout_direct(o, 0), readout_direct(o, 1));
            opart[b % NOB][tt][wv][ocol] = x;
        };
        if (L == C && (restarts >> 1) == 0u) {
            // a whole chunk whose frame restarts at most at its first token
            // (the usual case): that rescale goes first, then the tokens run
            // unrolled and branch-free, each token's LDS operands loaded while
            // the previous token computes
            Ops cur;
            if constexpr (kFirstEarly) cur = op0;
            else cur = load_ops(0);
            if (restarts & 1u) {
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) eta[r][cc] *= cur.ap.z;
            }
            Unroll<0, C>::run([&](auto u) {
                constexpr int tt = decltype(u)::value;
                Ops nxt;
                if constexpr (tt + 1 < C) nxt = load_ops(tt + 1);
                token(tt, cur, false);
                if constexpr (tt + 1 < C) cur = nxt;
            });
        } else {
            if constexpr (kFirstEarly) token(0, op0, true);
            for (int tt = kFirstEarly ? 1 : 0; tt < L; ++tt) token(tt, load_ops(tt), true);
        }

        if (c + 1 < nch) commit(b ^ 1, chunk_len(c + 1));
        __syncthreads();
        for (int e = tid; e < L * CI; e += NTH) {
            const int tt = e / CI;
            const int cc = e % CI;
            float sum = 0.0f;
#pragma unroll
            for (int g = 0; g < P; ++g) sum += opart[b % NOB][tt][g][cc];
            p.o[(bh * p.T + t0 + tt) * p.dv + tile * CI + cc] = sum;
        }
        // one partial buffer: every sum is read before the next chunk writes it
        if (NOB == 1) __syncthreads();
        if (c + 2 < nch) fetch(t0 + 2 * C, chunk_len(c + 2));
    }

    if (last) {
        const float inv_s_last = t_end > t_begin ? 1.0f / sch[t_end - 1].z : 1.0f;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t off = (sb * DK + j0 + r) * p.dv + i0;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                if (p.I_T) p.I_T[off + cc] = I[r][cc];
                if (p.mu_T) p.mu_T[off + cc] = eta[r][cc] * inv_s_last / I[r][cc];
            }
        }
    }
}

// Per-token scalars of the scaled frame, one thread per 16-token chunk of a
// head, walking its tokens in order: alpha = exp(-A d), the frame cuts (a
// frame starts at the chunk's first token and wherever the log-growth since
// that token crosses a multiple of kFrameLog), s = product of 1/alpha since
// the frame start, rho = alpha / s_{t-1} at a start (for the chunk's first
// token only alpha: the main pass divides by the previous chunk's last s).
// Output (rho, dP, s, A d) per token, where the prior increment dP is
// (1 - alpha) I_prior s for a pass that keeps the precision in the scaled
// frame (TRUE_I false) and (1 - alpha) I_prior for one that keeps it in true
// units (TRUE_I true; 1 - alpha from expm1, exact to rounding at small A d).
// One chunk's walk: tokens [t0, t0 + L) of head bh, a chunk start.
template <bool BF16, bool TRUE_I>
__device__ __forceinline__ void prep_chunk(const DiagParams& p, int64_t bh, int64_t t0, int L) {
    const float A = p.A[bh % p.H];
    float cum = 0.0f, s = 1.0f;
    int fr_prev = 0;
    float4* out = p.scal + bh * p.T + t0;
    for (int k = 0; k < L; ++k) {
        const int64_t t = bh * p.T + t0 + k;
        const float d = BF16 ? bf16_at(static_cast<const uint16_t*>(p.d), t) : static_cast<const float*>(p.d)[t];
        const float ell = A * d;
        const float alpha = fast_exp(-ell);
        float rho;
        if (k == 0) {
            rho = alpha;
            s = 1.0f;
        } else {
            cum += ell;
            const int fr = static_cast<int>(cum * (1.0f / kFrameLog));
            if (fr != fr_prev) {
                rho = alpha / s;
                s = 1.0f;
            } else {
                rho = 1.0f;
                s *= fast_exp(ell);
            }
            fr_prev = fr;
        }
        const float dP = TRUE_I ? -expm1f(-ell) * p.I_prior : (1.0f - alpha) * p.I_prior * s;
        out[k] = make_float4(rho, dP, s, ell);
    }
}

template <bool BF16, bool TRUE_I>
__global__ __launch_bounds__(256) void k_diag_prep(DiagParams p, int64_t n_units, int32_t nch) {
    constexpr int C = kDiagChunkTokens;
    for (int64_t u = elem_first(); u < n_units; u += elem_stride()) {
        const int64_t bh = u / nch;
        const int64_t t0 = (u % nch) * C;
        prep_chunk<BF16, TRUE_I>(p, bh, t0, p.T - t0 < C ? static_cast<int>(p.T - t0) : C);
    }
}

// Packed variable-length batch: chunks start at every sequence's first token.
// One thread per (head, packed token); the threads at a chunk start walk it.
template <bool BF16, bool TRUE_I>
__global__ __launch_bounds__(256) void k_diag_prep_varlen(DiagParams p) {
    constexpr int C = kDiagChunkTokens;
    for (int64_t u = elem_first(); u < p.H * p.T; u += elem_stride()) {
        const int64_t h = u / p.T;
        const int64_t t = u % p.T;
        int64_t t_begin, t_end;
        const int32_t s = find_sequence(p, t);
        sequence_tokens(p, s, t_begin, t_end);
        if ((t - t_begin) % C != 0) continue;
        prep_chunk<BF16, TRUE_I>(p, h, t, t_end - t < C ? static_cast<int>(t_end - t) : C);
    }
}

// Carry pass: in order over segments, turn each segment's composite into the
// state it starts from.  One thread per memory entry of every head.  The
// composites of 8 segments are loaded together, so a long chain of segments
// costs one memory round trip per 8 (the isotropic pass touches only eta).
__device__ __forceinline__ void carry_entry(const DiagParams& p, int64_t dk, int64_t e, int iso) {
    constexpr int B8 = 8;
    const int64_t n_per_head = dk * p.dv;
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
    float* const base = p.comp + bh * p.S * 2 * n_per_head + r;
    for (int s0 = 0; s0 < p.S; s0 += B8) {
        float Js[B8], es[B8], G[B8];
#pragma unroll
        for (int u = 0; u < B8; ++u) {
            const int s = s0 + u;
            const bool has = s + 1 < p.S;     // the last segment's composite is never read
            Js[u] = has && !iso ? base[s * 2 * n_per_head] : 0.0f;
            es[u] = has ? base[(s * 2 + 1) * n_per_head] : 0.0f;
            G[u] = has ? p.gdec[bh * p.S + s] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < B8; ++u) {
            const int s = s0 + u;
            if (s < p.S) {
                if (!iso) base[s * 2 * n_per_head] = J;
                base[(s * 2 + 1) * n_per_head] = eta;
            }
            J = __builtin_fmaf(G[u], J, Js[u]);
            eta = __builtin_fmaf(G[u], eta, es[u]);
        }
    }
}

__global__ __launch_bounds__(256) void k_diag_carry(DiagParams p, int64_t dk, int64_t n_total, int iso) {
    for (int64_t e = elem_first(); e < n_total; e += elem_stride()) carry_entry(p, dk, e, iso);
}

// T == 0: the final state is the starting state.
__global__ __launch_bounds__(256) void k_diag_copy_state(DiagParams p, int64_t n, int iso) {
    for (int64_t e = elem_first(); e < n; e += elem_stride()) {
        const float m0 = p.mu0 ? p.mu0[e] : 0.0f;
        if (!iso && p.I_T) p.I_T[e] = p.I0 ? p.I0[e] : p.I_prior;
        if (p.mu_T) p.mu_T[e] = m0;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

constexpr int kDiagChunk = kDiagChunkTokens;

// Workgroup width for a (DK, CI) tile: enough waves that each lane keeps
// 16 key rows when the tile is large, never fewer than one wave.
constexpr int diag_waves(int DK, int CI) {
    const int w = DK * CI / (kWave * 16);
    return w < 1 ? 1 : w;
}

template <int DK, int CI, bool BF16>
static void launch_one(const DiagParams& p, int64_t grid, hipStream_t st) {
    constexpr int W = diag_waves(DK, CI);
    hipLaunchKernelGGL((k_diag<DK, CI, W, kDiagChunk, BF16>), dim3(static_cast<uint32_t>(grid)),
                       dim3(W * kWave), 0, st, p);
}

template <int DK, bool BF16>
static int launch_dk(const DiagParams& p, int CI, int64_t grid, hipStream_t st) {
    if (CI == 64) {
        constexpr int RB = DK >= 64 ? 4 : 8;
        hipLaunchKernelGGL((k_diag_blk<DK, RB, kDiagChunk, BF16>), dim3(static_cast<uint32_t>(grid)),
                           dim3(DK / (2 * RB) * kWave), 0, st, p);
        return KDN_OK;
    }
    switch (CI) {
        case 16: launch_one<DK, 16, BF16>(p, grid, st); break;
        case 32: launch_one<DK, 32, BF16>(p, grid, st); break;
        case 64: launch_one<DK, 64, BF16>(p, grid, st); break;
        default: return KDN_EUNSUPPORTED;
    }
    return KDN_OK;
}

template <bool BF16>
static int launch_main(const DiagParams& p, int64_t dk, int CI, int64_t grid, hipStream_t st) {
    switch (dk) {
        case 16: return launch_dk<16, BF16>(p, CI, grid, st);
        case 32: return launch_dk<32, BF16>(p, CI, grid, st);
        case 64: return launch_dk<64, BF16>(p, CI, grid, st);
        case 128: return launch_dk<128, BF16>(p, CI, grid, st);
        default: return KDN_EUNSUPPORTED;
    }
}

int diag_chunk() { return kDiagChunk; }

// Packed batches run the block kernel's 64-column tiles where the head is
// that wide, else 32- or d_v-column tiles.
int varlen_cols(int64_t dv) { return dv >= 64 ? 64 : (dv < 32 ? static_cast<int>(dv) : 32); }

// Main-pass grid of a packed batch: whole groups of 8 runs (item x head) x
// column tiles.
int64_t varlen_main_grid(int64_t items, int64_t H, int64_t dv) {
    return (items * H + 7) / 8 * 8 * (dv / varlen_cols(dv));
}

// The plan of a packed batch, one workgroup.  Sequences are ordered longest
// first (ties by index) by rank counting; a sequence longer than vl_seg
// tokens is cut into ceil(len / vl_seg) segments.  The main-pass items are
// every sequence's segments in that order, each sequence's in token order;
// the composite segments are every split sequence's segments but its last.
// A sequence's offsets into the item, composite and split-sequence tables
// are sums over the sequences ranked before it, taken in the same counting
// loop as its rank.  Past kMaxPlanSort sequences the order is the index
// order and the offsets are prefix sums.  Table writes stay within their
// capacities, and the counts in nwork are clamped to them, so a malformed
// offset table cannot send a later pass out of bounds.  `units` is the
// composite storage in (segment, head, sub-segment) units; each composite
// segment takes units / (segments x H) sub-segments (nwork[3]), at most one
// per 4 chunks, so fewer split sequences get finer sub-segments.
__global__ __launch_bounds__(kPlanThreads) void k_varlen_plan(DiagParams p, int64_t units) {
    __shared__ int64_t lens[kPlanLds];
    __shared__ int32_t nsg[kPlanLds];
    __shared__ int64_t part[3][kPlanThreads];
    const int32_t n = p.nseq;
    const int tid = threadIdx.x;
    const bool staged = n <= kPlanLds;
    if (staged) {
        for (int32_t s = tid; s < n; s += kPlanThreads) {
            const int64_t l = clamped_length(p.cu_seqlens, p.T, s);
            lens[s] = l;
            nsg[s] = static_cast<int32_t>(varlen_segments(p, l));
        }
        __syncthreads();
    }
    auto len = [&](int32_t s) { return staged ? lens[s] : clamped_length(p.cu_seqlens, p.T, s); };
    auto segs = [&](int32_t s) -> int64_t { return staged ? nsg[s] : varlen_segments(p, len(s)); };
    auto place = [&](int32_t s, int64_t nseg, int64_t rank, int64_t io, int64_t co, int64_t so) {
        p.seq_order[rank] = s;
        if (p.seq_item) p.seq_item[s] = io < p.vl_items ? static_cast<int32_t>(io) : -1;
        int64_t a, b;
        sequence_tokens(p, s, a, b);
        for (int64_t g = 0; g < nseg && io + g < p.vl_items; ++g) {
            p.item_seq[io + g] = s;
            p.item_seg[io + g] = static_cast<int32_t>(g);
            VarlenItemRec r;
            const int64_t t0 = nseg > 1 ? a + g * p.vl_seg : a;
            r.t_begin = t0 < b ? t0 : b;
            r.t_end = nseg > 1 && t0 + p.vl_seg < b ? t0 + p.vl_seg : b;
            r.sq = s;
            r.seg = static_cast<int32_t>(g);
            r.carry = g > 0 && co + g - 1 < p.vl_comps ? static_cast<int32_t>(co + g - 1) : -1;
            r.last = g + 1 == nseg ? 1 : 0;
            p.items[io + g] = r;
        }
        p.seq_comp[s] = nseg > 1 && co < p.vl_comps ? static_cast<int32_t>(co) : -1;
        for (int64_t g = 0; g + 1 < nseg && co + g < p.vl_comps; ++g) {
            p.comp_seq[co + g] = s;
            p.comp_seg[co + g] = static_cast<int32_t>(g);
        }
        if (nseg > 1 && so < p.vl_comps) p.split_seq[so] = s;
    };
    // this thread's sums of items, composite segments and split sequences
    int64_t ni = 0, nc = 0, ns = 0;
    const bool sorted = n <= kMaxPlanSort;
    const int32_t per = (n + kPlanThreads - 1) / kPlanThreads;
    const int32_t s0 = tid * per < n ? tid * per : n;
    const int32_t s1 = s0 + per < n ? s0 + per : n;
    if (sorted) {
        for (int32_t s = tid; s < n; s += kPlanThreads) {
            const int64_t ls = len(s);
            int64_t rank = 0, io = 0, co = 0, so = 0;
            for (int32_t u = 0; u < n; ++u) {
                const int64_t lu = len(u);
                if (lu > ls || (lu == ls && u < s)) {
                    const int64_t g = segs(u);
                    ++rank;
                    io += g;
                    co += g - 1;
                    so += g > 1 ? 1 : 0;
                }
            }
            const int64_t g = segs(s);
            place(s, g, rank, io, co, so);
            ni += g;
            nc += g - 1;
            ns += g > 1 ? 1 : 0;
        }
    } else {
        for (int32_t s = s0; s < s1; ++s) {
            const int64_t g = segs(s);
            ni += g;
            nc += g - 1;
            ns += g > 1 ? 1 : 0;
        }
    }
    part[0][tid] = ni;
    part[1][tid] = nc;
    part[2][tid] = ns;
    __syncthreads();
    if (!sorted) {
        // index order: inclusive prefix sums over the threads (Hillis-Steele
        // in LDS), then each thread places its run of sequences
        for (int o = 1; o < kPlanThreads; o <<= 1) {
            int64_t v[3];
#pragma unroll
            for (int x = 0; x < 3; ++x) v[x] = tid >= o ? part[x][tid - o] : 0;
            __syncthreads();
#pragma unroll
            for (int x = 0; x < 3; ++x) part[x][tid] += v[x];
            __syncthreads();
        }
        int64_t io = part[0][tid] - ni, co = part[1][tid] - nc, so = part[2][tid] - ns;
        for (int32_t s = s0; s < s1; ++s) {
            const int64_t g = segs(s);
            place(s, g, s, io, co, so);
            io += g;
            co += g - 1;
            so += g > 1 ? 1 : 0;
        }
    } else {
        // totals only: a tree sum in LDS
        for (int h = kPlanThreads / 2; h > 0; h >>= 1) {
            if (tid < h) {
#pragma unroll
                for (int x = 0; x < 3; ++x) part[x][tid] += part[x][tid + h];
            }
            __syncthreads();
        }
    }
    // the item slots past the plan's items: a sentinel record
    {
        const int64_t last = sorted ? 0 : kPlanThreads - 1;
        for (int64_t i = part[0][last] + tid; i < p.vl_items; i += kPlanThreads) {
            VarlenItemRec r{};
            r.sq = -1;
            p.items[i] = r;
        }
    }
    if (tid == 0) {
        const int64_t last = sorted ? 0 : kPlanThreads - 1;
        const int64_t ti = part[0][last], tc = part[1][last], ts = part[2][last];
        const int64_t c = tc < p.vl_comps ? tc : p.vl_comps;
        p.nwork[0] = static_cast<int32_t>(ti < p.vl_items ? ti : p.vl_items);
        p.nwork[1] = static_cast<int32_t>(c);
        p.nwork[2] = static_cast<int32_t>(ts < p.vl_comps ? ts : p.vl_comps);
        // sub-segments per composite segment: the unit budget spread over the
        // composite segments there are, at least 4 chunks each
        int64_t R = c > 0 ? units / (c * p.H) : 1;
        const int64_t rmax = p.vl_seg / (4 * kDiagChunkTokens);
        if (R > rmax) R = rmax;
        if (R < 1) R = 1;
        p.nwork[3] = static_cast<int32_t>(R);
    }
}

// Packed variable-length batch (p.cu_seqlens set, p.S == 1): the plan, frame
// scalars per sequence-aligned chunk, then one workgroup per (sequence, head,
// tile).
// Frame scalars of a packed batch (chunks aligned to sequence starts).
int diag_prep_varlen_launch(const DiagParams& p, bool bf16, bool true_i, hipStream_t st) {
    const int64_t n = p.H * p.T;
    if (n == 0) return KDN_OK;
    const dim3 grid(elem_groups(n));
    if (bf16 && true_i) hipLaunchKernelGGL((k_diag_prep_varlen<true, true>), grid, dim3(256), 0, st, p);
    else if (bf16) hipLaunchKernelGGL((k_diag_prep_varlen<true, false>), grid, dim3(256), 0, st, p);
    else if (true_i) hipLaunchKernelGGL((k_diag_prep_varlen<false, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_diag_prep_varlen<false, false>), grid, dim3(256), 0, st, p);
    return launch_status();
}

// Packed batch: the plan, the frame scalars, the composites and carries of
// split sequences, then the main pass over the plan's items (the grid covers
// the item capacity; workgroups past the plan's items return at once).
void varlen_plan_launch(const DiagParams& p, int32_t R, hipStream_t st) {
    hipLaunchKernelGGL(k_varlen_plan, dim3(1), dim3(kPlanThreads), 0, st, p, p.vl_comps * p.H * R);
}

int diag_varlen_launch(const DiagParams& p, int64_t dk, bool bf16, int32_t R, hipStream_t st) {
    varlen_plan_launch(p, R, st);
    // the block kernel keeps I in true units
    const int prc = diag_prep_varlen_launch(p, bf16, varlen_cols(p.dv) == 64, st);
    if (prc != KDN_OK) return prc;
    const int CI = varlen_cols(p.dv);
    const int64_t grid = varlen_main_grid(p.vl_items, p.H, p.dv);
    if (p.vl_comps > 0) {
        DiagParams pc = p;
        pc.echo_base = grid;   // composite records after the main pass's
        const int crc = diag_varlen_comp_launch(pc, dk, bf16, R, st);
        if (crc != KDN_OK) return crc;
    }
    if (grid == 0) return launch_status();
    int rc = record_event(p.main_begin, st);
    if (rc != KDN_OK) return rc;
    rc = bf16 ? launch_main<true>(p, dk, CI, grid, st) : launch_main<false>(p, dk, CI, grid, st);
    if (rc != KDN_OK) return rc;
    if ((rc = record_event(p.main_end, st)) != KDN_OK) return rc;
    return launch_status();
}

int diag_prep_launch(const DiagParams& p, int64_t B, bool bf16, bool true_i, hipStream_t st) {
    const int32_t nch = static_cast<int32_t>((p.T + kDiagChunk - 1) / kDiagChunk);
    const int64_t n = B * p.H * nch;
    if (n == 0) return KDN_OK;
    const dim3 grid(elem_groups(n));
    if (bf16 && true_i) hipLaunchKernelGGL((k_diag_prep<true, true>), grid, dim3(256), 0, st, p, n, nch);
    else if (bf16) hipLaunchKernelGGL((k_diag_prep<true, false>), grid, dim3(256), 0, st, p, n, nch);
    else if (true_i) hipLaunchKernelGGL((k_diag_prep<false, true>), grid, dim3(256), 0, st, p, n, nch);
    else hipLaunchKernelGGL((k_diag_prep<false, false>), grid, dim3(256), 0, st, p, n, nch);
    return launch_status();
}

// Ordered carry over segments: composites -> starting state of every segment.
int diag_carry_launch(const DiagParams& p, int64_t B, int64_t dk, bool iso, hipStream_t st) {
    const int64_t n = B * p.H * dk * p.dv;
    if (n == 0) return KDN_OK;
    hipLaunchKernelGGL(k_diag_carry, dim3(elem_groups(n)), dim3(256), 0, st,
                       p, dk, n, iso ? 1 : 0);
    return launch_status();
}

// T == 0: write the starting state as the final state (iso: mean only).
int copy_state_launch(const DiagParams& p, int64_t B, int64_t dk, bool iso, hipStream_t st) {
    const int64_t n = B * p.H * dk * p.dv;
    if (n == 0) return KDN_OK;
    hipLaunchKernelGGL(k_diag_copy_state, dim3(elem_groups(n)), dim3(256), 0, st,
                       p, n, iso ? 1 : 0);
    return launch_status();
}

// Enqueue the whole diagonal scan.  Arguments were validated by the caller;
// comp/gdec point into a workspace of the size the planner reported when S > 1.
int diag_scan_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st) {
    const int64_t BH = B * p.H;
    if (BH == 0) return KDN_OK;
    if (p.T == 0) return copy_state_launch(p, B, dk, false, st);
    const int CI = p.dv < 64 ? static_cast<int>(p.dv) : 64;
    const int64_t ntile = p.dv / CI;
    // the block kernel (64-column tiles) keeps the precision in true units
    int rc = diag_prep_launch(p, B, bf16, CI == 64, st);
    if (rc != KDN_OK) return rc;
    const int64_t g2 = BH * p.S * ntile;
    if (p.S > 1) {
        DiagParams pc = p;
        pc.echo_base = g2;   // composite records after the main pass's
        if ((rc = diag_comp_launch(pc, B, dk, bf16, R, st)) != KDN_OK) return rc;
    }
    if ((rc = record_event(p.main_begin, st)) != KDN_OK) return rc;
    rc = bf16 ? launch_main<true>(p, dk, CI, g2, st) : launch_main<false>(p, dk, CI, g2, st);
    if (rc != KDN_OK) return rc;
    if ((rc = record_event(p.main_end, st)) != KDN_OK) return rc;
    return launch_status();
}

}  // namespace kdn

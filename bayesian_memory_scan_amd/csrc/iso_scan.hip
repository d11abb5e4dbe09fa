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
// One wave per (head, segment, tile of NC <= 64 value columns), no barriers:
// every operand is loaded from global memory straight into the register
// layout its MFMA wants.  Lane (c, g) = lane c + 16 g.
//   * mu (d_k x NC) lives in MFMA accumulators as MT x NT tiles of 16 x 16.
//     Tiles interleave rows and columns: tile (m, n) element (i, j) is
//     mu[MT i + m][NT j + n], so lane (c, g), register r of tile (m, n) holds
//     mu[MT (4g + r) + m][NT c + n].  A lane's registers then cover contiguous
//     runs of columns (vector loads and stores) and of rows.
//   * A contraction may visit its summation index in any order, provided both
//     operands agree.  Q mu visits d_k row j = MT (4g + r) + m at k-step
//     (m, r), lane group g, so its B operand is the lane's own accumulator
//     register and its A operand is the run Q[t][4 MT g .. 4 MT g + 4 MT).
//     Q K^T visits the same order.
//   * The wave computes S^T = K Q^T rather than S: its accumulator layout,
//     S[t = c][s = 4g + r] in lane (c, g), register r, is the A-operand layout
//     of (S (.) D) V with token s = 4g + kk at k-step kk, so no transpose.
//   * (S (.) D) V and the state update visit token s = 4g + kk and share the
//     V operand V[s][NT c + n].  The update's A operand K[s][MT c + m] is
//     the chunk's k transposed; the main pass writes its q-side k to a
//     per-wave LDS tile and reads it back transposed (the only LDS use).
// The segment composite pass (COMPOSITE) runs only the state update from a
// zero state, adding the chunks last to first, each weighted by the decay
// after it; segments are then combined in order by the shared carry pass.
#include "kdn_lane.h"
#include "kdn_params.h"

namespace kdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kIsoChunk = 16;
// Value columns per wave: at d_k = d_v = 64 one wave holds the head's whole
// mu (64 registers) and two operand sets within the 256 registers of two
// waves per SIMD, and nothing (S = Q K^T, the q and k reads) is repeated
// across column tiles.
constexpr int kIsoCols = 64;

// One chunk's operands in lane (c, g); t0 is the chunk's first token.  The
// query-side set (q, k in the d_k visiting order, gates) and the update-side
// set (k transposed, v) are both loaded a whole chunk ahead.
template <int DK>
struct IsoQK {
    static constexpr int MT = DK / 16;
    float q[4 * MT];                   // Q[t0 + c][4 MT g + e]
    float k[4 * MT];                   // K[t0 + c][4 MT g + e]
    float F, G;                        // gates of token t0 + c
};

template <int DK, int NC, bool COMPOSITE>
struct IsoKV {
    static constexpr int MT = DK / 16;
    static constexpr int NT = NC / 16;
    float kt[COMPOSITE ? 4 : 1][MT];   // K[t0 + 4g + kk][MT c + m] (composite pass; the
                                       // main pass transposes its q-side k through LDS)
    float v[4][NT];                    // V[t0 + 4g + kk][tile columns NT c + n]
    float F, G;                        // gates of token t0 + c (composite pass)
};

template <int DK, int NC, bool COMPOSITE>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(DK <= 64 ? 2 : 1)))
void k_iso(DiagParams p) {
    constexpr int C = kIsoChunk;
    constexpr int MT = DK / 16;                // row tiles of mu
    constexpr int NT = NC / 16;                // column tiles of mu
    using QK = IsoQK<DK>;
    using KV = IsoKV<DK, NC, COMPOSITE>;
    constexpr int KR = DK + 4;                 // row stride of the LDS copy of k
    __shared__ float4 kbuf4[COMPOSITE ? 1 : C * KR / 4];
    float* const kbuf = reinterpret_cast<float*>(kbuf4);

    const int lane = threadIdx.x;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int ntile = static_cast<int>(p.dv / NC);
    const int64_t id = xcd_local_id();         // a head-segment's column tiles share an XCD
    const int tile = static_cast<int>(id % ntile);
    const int64_t rest = id / ntile;
    const int seg = static_cast<int>(rest % p.S);
    const int64_t bh = rest / p.S;
    const int nseg_run = COMPOSITE ? p.S - 1 : p.S;
    if (seg >= nseg_run) return;

    int64_t t_begin, t_end;
    segment_tokens(p, C, seg, t_begin, t_end);
    if (lane == 0) echo_bounds(p, blockIdx.x, COMPOSITE ? 4 : 3, bh, seg, tile, t_begin, t_end, -1);
    const int64_t DV = p.dv;
    const int64_t cb = static_cast<int64_t>(tile) * NC;   // first column of the tile

    const float* qh = static_cast<const float*>(p.q) + bh * p.T * DK;
    const float* kh = static_cast<const float*>(p.k) + bh * p.T * DK;
    const float* vh = static_cast<const float*>(p.v) + bh * p.T * DV;
    const float* Fh = p.F + bh * p.T;
    const float* Gh = p.G + bh * p.T;

    // macc[m][n][r] = mu[MT (4g + r) + m][cb + NT c + n]
    f32x4 macc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = 0.0f;
                if constexpr (!COMPOSITE) {
                    const int64_t off = static_cast<int64_t>(MT * (4 * g + r) + m) * DV + cb + NT * c + n;
                    if (p.S == 1) {
                        if (p.mu0) x = p.mu0[bh * DK * DV + off];
                    } else {
                        x = p.comp[((bh * p.S + seg) * 2 + 1) * DK * DV + off];
                    }
                }
                macc[m][n][r] = x;
            }

    // Operand loads of the chunk at token t0 through buffer resources that
    // end at the chunk's last token (rows past it read as 0; F as 1), and
    // hold no rows at all for a chunk outside the segment.
    auto chunk_rows = [&](int64_t t0) -> int64_t {
        if (t0 < t_begin) return 0;   // the composite pass's prefetch before the segment
        const int64_t L = t_end - t0;
        return L < 0 ? 0 : (L < C ? L : C);
    };
    auto load_qk = [&](int64_t t0, QK& x) __attribute__((always_inline)) {
        const int64_t L = chunk_rows(t0);
        const uint32_t off = static_cast<uint32_t>((c * DK + 4 * MT * g) * 4);
        buf_load<4 * MT>(buf_rsrc(qh + t0 * DK, L * DK * 4), off, x.q);
        buf_load<4 * MT>(buf_rsrc(kh + t0 * DK, L * DK * 4), off, x.k);
        float f[1], gg[1];
        buf_load<1>(buf_rsrc(Fh + t0, L * 4), static_cast<uint32_t>(c * 4), f);
        buf_load<1>(buf_rsrc(Gh + t0, L * 4), static_cast<uint32_t>(c * 4), gg);
        x.F = f[0];   // 0 past the chunk's end; compute() substitutes 1 there
        x.G = gg[0];
    };
    auto load_kv = [&](int64_t t0, KV& x) __attribute__((always_inline)) {
        const int64_t L = chunk_rows(t0);
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kh + t0 * DK, L * DK * 4);
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vh + t0 * DV, L * DV * 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int s_ = 4 * g + kk;
            if constexpr (COMPOSITE) buf_load<MT>(rk, static_cast<uint32_t>((s_ * DK + MT * c) * 4), x.kt[kk]);
            buf_load<NT>(rv, static_cast<uint32_t>((s_ * DV + cb + NT * c) * 4), x.v[kk]);
        }
        if constexpr (COMPOSITE) {
            float f[1], gg[1];
            buf_load<1>(buf_rsrc(Fh + t0, L * 4), static_cast<uint32_t>(c * 4), f);
            buf_load<1>(buf_rsrc(Gh + t0, L * 4), static_cast<uint32_t>(c * 4), gg);
            x.F = f[0];
            x.G = gg[0];
        }
    };

    float logsum = 0.0f;   // sum of log2 F over the segment
    // composite pass: the decay from the end of the chunk being added to the
    // end of the segment (chunks are added last to first)
    float dscale = 1.0f;
    // One chunk: qk is the query-side set (unused by the composite pass), kv
    // the update-side set; F and G come from kv in the composite pass.
    auto compute = [&](int64_t t0, QK& qk, const KV& kv) __attribute__((always_inline)) {
        // F past the chunk's end is 1 (no decay); the loads gave 0 there
        const float Fc = t0 + c < t_end ? (COMPOSITE ? kv.F : qk.F) : 1.0f;
        const float Gc = COMPOSITE ? kv.G : qk.G;
        const float b = row_prefix16(__log2f(Fc));         // b_t of token t0 + c (<= 0)
        const float blast = bcast<15>(b);
        const float wt = Gc * exp2f(blast - b);            // w of token t0 + c
        // b, G and w of token s = 4g + kk, from lane s of this row
        float bs[4], gs[4], ws[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int src = 16 * g + 4 * g + kk;
            bs[kk] = __shfl(b, src);
            gs[kk] = __shfl(Gc, src);
            ws[kk] = __shfl(wt, src);
        }
        if constexpr (!COMPOSITE) {
            // k of token t0 + c to LDS: the update reads it transposed.  One
            // wave owns kbuf and its LDS operations complete in order.
#pragma unroll
            for (int e = 0; e < 4 * MT; e += 4)
                *reinterpret_cast<float4*>(&kbuf[c * KR + 4 * MT * g + e]) =
                    make_float4(qk.k[e], qk.k[e + 1], qk.k[e + 2], qk.k[e + 3]);
            // S^T = K Q^T: register r = S[t = c][s = 4g + r]
            f32x4 sp[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) sp[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int e = 0; e < 4 * MT; ++e) sp[e & 1] = mfma4(qk.k[e], qk.q[e], sp[e & 1]);
            const f32x4 sacc = sp[0] + sp[1];
            // P[t = c][s = 4g + kk] = S e^{b_t - b_s} G_s [s <= t]
            float pa[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                pa[kk] = 4 * g + kk <= c ? sacc[kk] * exp2f(b - bs[kk]) * gs[kk] : 0.0f;
            // O = diag(e^b) Q mu_start + P V
            const float eb = exp2f(b);
#pragma unroll
            for (int e = 0; e < 4 * MT; ++e) qk.q[e] *= eb;
            f32x4 oacc[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) oacc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int n = 0; n < NT; ++n) oacc[n] = mfma4(qk.q[MT * r + m], macc[m][n][r], oacc[n]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int n = 0; n < NT; ++n) oacc[n] = mfma4(pa[kk], kv.v[kk][n], oacc[n]);
            const __amdgpu_buffer_rsrc_t ro = buf_rsrc(p.o + (bh * p.T + t0) * DV, chunk_rows(t0) * DV * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float row[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) row[n] = oacc[n][r];
                buf_store<NT>(ro, static_cast<uint32_t>(((4 * g + r) * DV + cb + NT * c) * 4), row);
            }
        }
        // main pass: mu = e^{b_last} mu + (w (.) K)^T V; composite pass, chunks
        // last to first: mu += dscale (w (.) K)^T V, then dscale *= e^{b_last}
        const float decay = exp2f(blast);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float aw[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float ktm;
                if constexpr (COMPOSITE) ktm = kv.kt[kk][m] * dscale;
                else ktm = kbuf[(4 * g + kk) * KR + MT * c + m];
                aw[kk] = ws[kk] * ktm;
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if constexpr (!COMPOSITE) macc[m][n] *= decay;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) macc[m][n] = mfma4(aw[kk], kv.v[kk][n], macc[m][n]);
            }
        }
        if constexpr (COMPOSITE) dscale *= decay;
        logsum += blast;
    };

    // The loads are unconditional (a chunk past the segment's end reads as
    // zeros without touching memory), so the compiler's wait counts stay
    // exact and never wait on the chunk being prefetched.
    const int64_t nch = (t_end - t_begin + C - 1) / C;
    if constexpr (COMPOSITE) {
        // Chunks last to first, so that the segment's first chunks are the
        // ones read most recently when the main pass starts on them.  Two
        // update-side sets: the previous chunk's loads are in flight while
        // one computes (a chunk before the segment reads nothing).
        QK none;
        KV xa, xb;
        const int64_t tl = t_begin + (nch - 1) * C;
        load_kv(tl, xa);
        for (int64_t ch = 0; ch < nch; ch += 2) {
            const int64_t t0 = tl - ch * C;
            load_kv(t0 - C, xb);
            compute(t0, none, xa);
            if (ch + 1 >= nch) break;
            load_kv(t0 - 2 * C, xa);
            compute(t0 - C, none, xb);
        }
    } else {
        // two sets of everything: each chunk's operands load a whole chunk ahead
        QK qa, qb;
        KV ka, kb;
        load_qk(t_begin, qa);
        load_kv(t_begin, ka);
        for (int64_t ch = 0; ch < nch; ch += 2) {
            const int64_t t0 = t_begin + ch * C;
            load_qk(t0 + C, qb);
            load_kv(t0 + C, kb);
            compute(t0, qa, ka);
            if (ch + 1 >= nch) break;
            load_qk(t0 + 2 * C, qa);
            load_kv(t0 + 2 * C, ka);
            compute(t0 + C, qb, kb);
        }
    }

    if constexpr (COMPOSITE) {
        float* slot = p.comp + ((bh * p.S + seg) * 2 + 1) * DK * DV;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float row[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) row[n] = macc[m][n][r];
                store_run<NT>(slot + static_cast<int64_t>(MT * (4 * g + r) + m) * DV + cb + NT * c, row);
            }
        if (lane == 0 && tile == 0) p.gdec[bh * p.S + seg] = exp2f(logsum);
    } else if (seg == p.S - 1 && p.mu_T) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float row[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) row[n] = macc[m][n][r];
                store_run<NT>(p.mu_T + (bh * DK + MT * (4 * g + r) + m) * DV + cb + NT * c, row);
            }
    }
}

int iso_chunk() { return kIsoChunk; }

// Column tiles of one head: min(d_v, kIsoCols) columns each.
int iso_tiles(int64_t dv) { return dv > kIsoCols ? static_cast<int>(dv / kIsoCols) : 1; }

template <int DK, bool COMPOSITE>
static int iso_launch_dv(const DiagParams& p, int64_t dv, int64_t grid, hipStream_t st) {
    switch (dv) {
        case 16: hipLaunchKernelGGL((k_iso<DK, 16, COMPOSITE>), dim3(grid), dim3(kWave), 0, st, p); break;
        case 32: hipLaunchKernelGGL((k_iso<DK, 32, COMPOSITE>), dim3(grid), dim3(kWave), 0, st, p); break;
        case 64:
        case 128: hipLaunchKernelGGL((k_iso<DK, kIsoCols, COMPOSITE>), dim3(grid), dim3(kWave), 0, st, p); break;
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
// One wave per (head, segment, column tile).
int iso_mean_launch(const DiagParams& p, int64_t B, int64_t dk, hipStream_t st) {
    const int64_t BH = B * p.H;
    if (BH == 0) return KDN_OK;
    if (p.T == 0) return copy_state_launch(p, B, dk, true, st);   // mu_T = mu0
    const int64_t grid = BH * p.S * iso_tiles(p.dv);
    int rc;
    if (p.S > 1) {
        DiagParams pc = p;
        pc.echo_base = grid;   // composite records after the main pass's
        if ((rc = iso_launch<true>(pc, dk, p.dv, grid, st)) != KDN_OK) return rc;
        if ((rc = diag_carry_launch(p, B, dk, true, st)) != KDN_OK) return rc;
    }
    if ((rc = record_event(p.main_begin, st)) != KDN_OK) return rc;
    if ((rc = iso_launch<false>(p, dk, p.dv, grid, st)) != KDN_OK) return rc;
    return record_event(p.main_end, st);
}

}  // namespace kdn

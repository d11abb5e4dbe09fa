// diag_comp.hip -- segment composites of the diagonal-precision scan on the
// fp32 matrix cores, and their ordered carry.
//
// With J = I - I_prior, the precision and information-mean updates of the
// diagonal scan (Palimpsa, "Learning to Remember, Learn, and Forget in
// Attention-Based Models", Metodologia 2, multiplied through by I_t) are the
// affine recurrences
//   J_t = alpha_t J_{t-1} + beta_t[i] k_t[j]^2,   eta_t = alpha_t eta_{t-1} + beta_t[i] v_t[i] k_t[j].
// Over a stretch of tokens starting from zero they give the composite
// (G, J, eta): G = prod alpha and, with w_s = prod_{u > s} alpha_u the decay of
// token s to the end of the stretch,
//   J = (w (.) K^2)^T B,      eta = (w (.) K)^T (B (.) V),
// two genuine contractions over the stretch's tokens, accumulated 16 tokens
// at a time on v_mfma_f32_16x16x4f32.
// Composites combine in order, (G2, X2) o (G1, X1) = (G2 G1, G2 X1 + X2), the
// associativity that makes these updates scannable (KLA summary,
// Metodologia 2).
//
// One wave per (head, sub-segment, tile of NC <= 32 value columns), with all
// d_k rows; no LDS and no barriers.  Every operand is loaded from global
// memory straight into its MFMA register layout (A[i][k] in lane i + 16k,
// B[k][j] in lane j + 16k, D[i][j] in lane j + 16(i/4), register i%4):
//   * J and eta live in accumulators as MT x NT tiles of 16 x 16 whose rows
//     and columns interleave: tile (m, n) element (i, j) is entry
//     [MT i + m][NT j + n], so lane (c, g), register r holds [MT (4g + r) + m][NT c + n];
//   * both contractions visit token s = 4g + kk at k-step kk, so lane (c, g)
//     reads the run k_s[MT c .. MT c + MT) for its A operands and the runs
//     beta_s, v_s [NT c .. NT c + NT) for its B operands: one vector load each;
//   * loads go through buffer resources that end at the sub-segment's last
//     token (rows past it read as 0), so the prefetched chunk stays in flight.
#include "kdn_lane.h"
#include "kdn_params.h"

#include <type_traits>

namespace kdn {

typedef float f32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4c mfma4c(float a, float b, f32x4c c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kCompCols = 32;   // value columns per wave: 2 x MT x 2 x 4 accumulator registers

// Column tiles of one head in the composite pass.
int comp_tiles(int64_t dv) { return dv > kCompCols ? static_cast<int>(dv / kCompCols) : 1; }

template <int DK, int NC, bool BF16>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(BF16 || DK < 128 ? 2 : 1)))
void k_diag_comp(DiagParams p, int32_t R) {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int C = 16;
    constexpr int MT = DK / 16;
    constexpr int NT = NC / 16;
    constexpr int ES = static_cast<int>(sizeof(E));

    const int lane = threadIdx.x;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int ntile = static_cast<int>(p.dv / NC);
    const int nsub = (p.S - 1) * R;
    const int64_t id = xcd_local_id();       // a sub-segment's column tiles share an XCD
    const int tile = static_cast<int>(id % ntile);
    const int64_t rest = id / ntile;
    const int sr = static_cast<int>(rest % nsub);
    const int64_t bh = rest / nsub;
    const int seg = sr / R;
    const int sub = sr % R;
    int64_t t_begin, t_end;
    sub_tokens(p, C, R, seg, sub, t_begin, t_end);
    if (lane == 0) echo_bounds(p, blockIdx.x, 2, bh, seg, sub, t_begin, t_end, tile);
    const int64_t DV = p.dv;
    const int64_t cb = static_cast<int64_t>(tile) * NC;

    const E* kh = static_cast<const E*>(p.k) + bh * p.T * DK;
    const E* vh = static_cast<const E*>(p.v) + bh * p.T * DV;
    // beta == NULL: Palimpsa-M gating, beta_t[i] = d_t
    const E* bth = p.beta ? static_cast<const E*>(p.beta) + bh * p.T * DV : nullptr;
    const E* dh = static_cast<const E*>(p.d) + bh * p.T;
    const float4* sch = p.scal + bh * p.T;

    f32x4c J[MT][NT], X[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            J[m][n] = f32x4c{0.0f, 0.0f, 0.0f, 0.0f};
            X[m][n] = J[m][n];
        }

    // one chunk's operands in lane (c, g): token s = 4g + kk for the
    // contractions, token c for the decay scalars
    struct Ops {
        float k[4][MT];     // k_s[MT c + m]
        float b[4][NT];     // beta_s[cb + NT c + n]
        float v[4][NT];     // v_s[cb + NT c + n]
        float d[4];         // d_s (the input gate under Palimpsa-M gating)
        float ad;           // A d of token t0 + c (0 past the end)
    };
    auto load = [&](int64_t t0, Ops& x) __attribute__((always_inline)) {
        const int64_t L0 = t_end - t0;
        const int64_t L = (t0 < t_begin || L0 < 0) ? 0 : (L0 < C ? L0 : C);   // 0: nothing is read
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kh + t0 * DK, L * DK * ES);
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vh + t0 * DV, L * DV * ES);
        // beta and d are both loaded, with no branch (compute() picks d under
        // Palimpsa-M gating): a load behind a branch makes the compiler wait
        // for every load in flight, the prefetched chunk's included.  Without
        // beta its resource is empty, so those loads return 0 and read nothing.
        const __amdgpu_buffer_rsrc_t rb = bth ? buf_rsrc(bth + t0 * DV, L * DV * ES) : buf_rsrc(dh, 0);
        const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dh + t0, L * ES);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int s_ = 4 * g + kk;
            buf_load_widen<E, MT>(rk, static_cast<uint32_t>((s_ * DK + MT * c) * ES), x.k[kk]);
            buf_load_widen<E, NT>(rv, static_cast<uint32_t>((s_ * DV + cb + NT * c) * ES), x.v[kk]);
            buf_load_widen<E, NT>(rb, static_cast<uint32_t>((s_ * DV + cb + NT * c) * ES), x.b[kk]);
            float d1[1];
            buf_load_widen<E, 1>(rd, static_cast<uint32_t>(s_ * ES), d1);
            x.d[kk] = d1[0];
        }
        float ad[1];
        buf_load<1>(buf_rsrc(sch + t0, L * 16), static_cast<uint32_t>(c * 16 + 12), ad);
        x.ad = ad[0];
    };

    // Chunks are visited last to first.  Every token's weight is its decay to
    // the sub-segment's end, w_s = exp(-sum_{u > s} A d_u): no accumulator is
    // rescaled per chunk, and the exponent is built by additions only (Rsum,
    // the log-decay of the chunks already visited, plus the in-chunk suffix),
    // so its rounding error stays relative to its own size.
    float Rsum = 0.0f;
    auto compute = [&](const Ops& x) __attribute__((always_inline)) {
        const float P = row_prefix16(x.ad);          // in-chunk inclusive sum of A d
        const float Tc = bcast<15>(P);                // the chunk's total
        const float wt = fast_exp(-(Rsum + (Tc - P)));   // weight of token t0 + c
        float ws[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ws[kk] = __shfl(wt, 16 * g + 4 * g + kk);
        // beta == NULL: Palimpsa-M gating, beta_t[i] = d_t
        float bs[4][NT], bv[4][NT];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                bs[kk][n] = bth ? x.b[kk][n] : x.d[kk];
                bv[kk][n] = bs[kk][n] * x.v[kk][n];
            }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float wk[4], wk2[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                wk[kk] = ws[kk] * x.k[kk][m];
                wk2[kk] = wk[kk] * x.k[kk][m];
            }
            // k-step outermost: 2 NT independent accumulators between two
            // MFMAs on the same one
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    J[m][n] = mfma4c(wk2[kk], bs[kk][n], J[m][n]);
                    X[m][n] = mfma4c(wk[kk], bv[kk][n], X[m][n]);
                }
        }
        Rsum += Tc;
    };

    // two operand sets: the previous chunk loads while this one computes
    // (a chunk before the sub-segment reads nothing)
    const int64_t nch = (t_end - t_begin + C - 1) / C;
    Ops xa, xb;
    load(t_begin + (nch - 1) * C, xa);
    for (int64_t i = 0; i < nch; i += 2) {
        const int64_t t0 = t_begin + (nch - 1 - i) * C;
        load(t0 - C, xb);
        compute(xa);
        if (i + 1 >= nch) break;
        load(t0 - 2 * C, xa);
        compute(xb);
    }

    const int64_t slot = (bh * (p.S - 1) + seg) * R + sub;
    float* out = p.sub + slot * 2 * DK * DV;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float rowJ[NT], rowX[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                rowJ[n] = J[m][n][r];
                rowX[n] = X[m][n][r];
            }
            const int64_t off = static_cast<int64_t>(MT * (4 * g + r) + m) * DV + cb + NT * c;
            store_run<NT>(out + off, rowJ);
            store_run<NT>(out + static_cast<int64_t>(DK) * DV + off, rowX);
        }
    if (lane == 0 && tile == 0) p.gsub[slot] = fast_exp(-Rsum);
}

// Ordered carry: sub-segment composites -> the starting (J, eta) of every
// main segment.  One thread per memory entry of every head.
__device__ __forceinline__ void carry_sub_entry(const DiagParams& p, int64_t dk, int64_t e, int32_t R) {
    const int64_t n_per_head = dk * p.dv;
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

__global__ __launch_bounds__(256) void k_diag_carry_sub(DiagParams p, int64_t dk, int64_t n_total, int32_t R) {
    for (int64_t e = elem_first(); e < n_total; e += elem_stride()) carry_sub_entry(p, dk, e, R);
}

template <int DK, bool BF16>
static int comp_launch_dv(const DiagParams& p, int64_t dv, int64_t grid, int32_t R, hipStream_t st) {
    switch (dv) {
        case 16: hipLaunchKernelGGL((k_diag_comp<DK, 16, BF16>), dim3(grid), dim3(kWave), 0, st, p, R); break;
        case 32:
        case 64:
        case 128: hipLaunchKernelGGL((k_diag_comp<DK, kCompCols, BF16>), dim3(grid), dim3(kWave), 0, st, p, R); break;
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

// Composites of segments 0..S-2 in R sub-segments each (one wave per
// sub-segment and column tile), then the carry into every segment's starting
// state (p.comp).  Needs the per-token scalars.
int diag_comp_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st) {
    const int64_t BH = B * p.H;
    const int64_t grid = BH * (p.S - 1) * R * comp_tiles(p.dv);
    int rc = bf16 ? comp_launch<true>(p, dk, grid, R, st) : comp_launch<false>(p, dk, grid, R, st);
    if (rc != KDN_OK) return rc;
    const int64_t n = BH * dk * p.dv;
    hipLaunchKernelGGL(k_diag_carry_sub, dim3(elem_groups(n)), dim3(256), 0, st,
                       p, dk, n, R);
    return launch_status();
}

}  // namespace kdn

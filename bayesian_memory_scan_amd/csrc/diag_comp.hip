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

// Wave tiles of one head in the composite pass.  fp32 inputs: 32-column
// tiles with every key row.  bf16 inputs: waves summing J take at most 2 x 8
// MFMA tiles of 16 x 16 (32 key rows x 128 value columns), waves summing X
// at most 8 x 2 (128 x 32).  Each wave cuts only its own fp32 factor into
// limbs, w k^2 over its key rows or w beta v over its value columns, so the
// narrow side of its tile is the one it splits.
constexpr int comp_bf_mt(int dk, int part) { return part == 0 ? (dk / 16 < 2 ? dk / 16 : 2) : (dk / 16 < 8 ? dk / 16 : 8); }
constexpr int comp_bf_nt(int dv, int part) { return part == 0 ? (dv / 16 < 8 ? dv / 16 : 8) : (dv / 16 < 2 ? dv / 16 : 2); }
constexpr int comp_bf_tiles(int dk, int dv, int part) {
    return (dk / (16 * comp_bf_mt(dk, part))) * (dv / (16 * comp_bf_nt(dv, part)));
}
int comp_tiles(int64_t dk, int64_t dv, bool bf16) {
    if (!bf16) return dv > kCompCols ? static_cast<int>(dv / kCompCols) : 1;
    const int k = static_cast<int>(dk), v = static_cast<int>(dv);
    return comp_bf_tiles(k, v, 0) + comp_bf_tiles(k, v, 1);   // J waves, then X waves
}

// Composite unit `rest` (the column tile taken out): its token row bh,
// output slot and token bounds.  A fixed-length batch: sub-segment `sub` of
// segment `seg` of row bh (sub_tokens).  A packed batch: varlen_comp_unit,
// run = sequence * H + head.  False when a packed batch's plan has no such
// unit.
struct CompUnit {
    int64_t bh, slot, run, t_begin, t_end;
    int32_t seg, sub, sq;
};

__device__ __forceinline__ bool comp_unit(const DiagParams& p, int64_t rest, int32_t R, CompUnit& u) {
    if (p.cu_seqlens) {
        int64_t h;
        if (!varlen_comp_unit(p, rest, h, u.sq, u.seg, u.sub, u.t_begin, u.t_end)) return false;
        u.bh = h;
        u.slot = rest;
        u.run = static_cast<int64_t>(u.sq) * p.H + h;
        return true;
    }
    const int64_t nsub = static_cast<int64_t>(p.S - 1) * R;
    const int32_t sr = static_cast<int32_t>(rest % nsub);
    u.bh = rest / nsub;
    u.seg = sr / R;
    u.sub = sr % R;
    u.sq = 0;
    sub_tokens(p, kDiagChunkTokens, R, u.seg, u.sub, u.t_begin, u.t_end);
    u.slot = (u.bh * (p.S - 1) + u.seg) * R + u.sub;
    u.run = u.bh;
    return true;
}

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
    const int64_t id = xcd_local_id();       // a sub-segment's column tiles share an XCD
    const int tile = static_cast<int>(id % ntile);
    CompUnit u;
    if (!comp_unit(p, id / ntile, R, u)) return;
    const int64_t bh = u.bh;
    const int64_t t_begin = u.t_begin, t_end = u.t_end;
    if (lane == 0) echo_bounds(p, blockIdx.x, 2, u.run, u.seg, u.sub, t_begin, t_end, tile, u.sq);
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

    const int64_t slot = u.slot;
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

// ---------------------------------------------------------------------------
// bf16 inputs: the same two contractions on v_mfma_f32_16x16x32_bf16, with
// every product exact.
//
// bf16 keys are exact in one bf16 limb, so X takes A = k (one limb) against
// B = w beta v.  J takes A = w k^2 against B = beta (exact in one limb).  The
// fp32 factors w beta v and w k^2 are cut into three bf16 limbs by truncation:
// hi = x with the low 16 bits of its pattern cleared, then the same on
// x - hi, and the rest, which has at most 8 significant bits, is exact in
// bf16.  So hi + mid + lo == x exactly, every limb product is exact in the
// MFMA's fp32 accumulation, and
//   J = sum_limbs (w k^2)_limb^T beta,   X = k^T sum_limbs (w beta v)_limb
// accumulate the same products as fp32 arithmetic on the rounded fp32
// factors: six MFMAs of 16x16x32 (bf16 rate, about 14x that of
// 16x16x4 fp32 measured on gfx950) per 16 x 16 tile and 32 tokens.
//
// One wave per (head, sub-segment, part, tile of MT x NT 16 x 16 tiles):
// J waves at most 2 x 8 such tiles, X waves at most 8 x 2, so each splits
// the factor on its tile's narrow side (comp_bf_mt, comp_bf_nt) and no
// wave cuts more than 16 elements per lane and block into limbs.
// Operand layout of 16x16x32: lane (c, g) holds
// A[row c][k = 8g .. 8g+7] and B[k = 8g .. 8g+7][column c], D[rows 4g .. 4g+3]
// [column c].  Rows and columns interleave as in the fp32 kernel: tile (m, n)
// row c is key row rb + MT c + m and column c is value column cb + NT c + n,
// so one lane's keys of a token are one contiguous run (MT elements), and
// likewise its beta and v.  Token k of a 32-token block is 8g + e; pairs of
// consecutive tokens share one 32-bit operand word (low half the earlier).
// Blocks are visited last to first, with the decay weights built by additions
// as in the fp32 kernel.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4c mfma_bf(u32x4c a, u32x4c b, f32x4c c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8c, a), __builtin_bit_cast(bf16x8c, b),
                                                   c, 0, 0, 0);
}

// The top halves of two fp32 patterns as one bf16 pair: a in the low half.
// One v_perm_b32 (bytes 2, 3 of a, then bytes 2, 3 of b).
__device__ __forceinline__ uint32_t pack_top(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Three-limb split of the pair (xa, xb): limb words l[0..2], with
// l[0] + l[1] + l[2] == x exactly in each half.
// (No contraction here: fusing x - hi with the product that made x would
// split the unrounded product instead of x.)
__device__ __forceinline__ void split3(float xa, float xb, uint32_t& l0, uint32_t& l1, uint32_t& l2) {
#pragma clang fp contract(off)
    const uint32_t ua = __float_as_uint(xa), ub = __float_as_uint(xb);
    l0 = pack_top(ua, ub);
    const float ra = xa - __uint_as_float(ua & 0xffff0000u);
    const float rb = xb - __uint_as_float(ub & 0xffff0000u);
    const uint32_t va = __float_as_uint(ra), vb = __float_as_uint(rb);
    l1 = pack_top(va, vb);
    const float sa = ra - __uint_as_float(va & 0xffff0000u);
    const float sb = rb - __uint_as_float(vb & 0xffff0000u);
    l2 = pack_top(__float_as_uint(sa), __float_as_uint(sb));
}

// bf16 element e (0-based) of a run held as 32-bit words, widened to fp32.
template <int N>
__device__ __forceinline__ float bf_elem(const uint32_t (&w)[N], int e) {
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
}
// bf16 element e of run a (low half) and of run b (high half) as one word.
template <int N>
__device__ __forceinline__ uint32_t bf_pair(const uint32_t (&a)[N], const uint32_t (&b)[N], int e) {
    return __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
}

// n 16-bit elements (n = 1, 2, 4, 8) at byte offset off, as 32-bit words.
template <int NW>
__device__ __forceinline__ void buf_words(__amdgpu_buffer_rsrc_t r, uint32_t off, int n, uint32_t (&w)[NW]) {
    if (n == 8) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 4 && i < NW; ++i) w[i] = u[i];
    } else if (n == 4) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = u[0];
        if constexpr (NW > 1) w[1] = u[1];
    } else if (n == 2) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else {
        w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
}

template <int DK, int DV, int PART, bool MG>
__device__ __forceinline__ void comp_bf_part(const DiagParams& p, int32_t R, int64_t unit, int tile) {
    constexpr int KB = 32;                                     // tokens per k-step
    constexpr int MT = comp_bf_mt(DK, PART);
    constexpr int NT = comp_bf_nt(DV, PART);
    constexpr int TC = DV / (16 * NT);                         // wave tiles across the columns
    constexpr int KW = (MT + 1) / 2;                           // 32-bit words of a lane's key run
    constexpr int BW = (NT + 1) / 2;                           // ... of its beta / v run
    static_assert(MT == 1 || MT == 2 || MT == 4 || MT == 8, "key rows per lane run");
    static_assert(NT == 1 || NT == 2 || NT == 4 || NT == 8, "value columns per lane run");

    const int lane = threadIdx.x;
    const int g = lane >> 4;
    const int c = lane & 15;
    CompUnit u;
    if (!comp_unit(p, unit, R, u)) return;
    const int64_t bh = u.bh;
    const int64_t t_begin = u.t_begin, t_end = u.t_end;
    if (lane == 0)
        echo_bounds(p, blockIdx.x, 2, u.run, u.seg, u.sub, t_begin, t_end,
                    PART ? comp_bf_tiles(DK, DV, 0) + tile : tile, u.sq);
    const int rb = (tile / TC) * 16 * MT;    // first key row of the wave tile
    const int cb = (tile % TC) * 16 * NT;    // first value column
    const int64_t DV_ = p.dv;

    const uint16_t* kh = static_cast<const uint16_t*>(p.k) + bh * p.T * DK;
    const uint16_t* vh = static_cast<const uint16_t*>(p.v) + bh * p.T * DV_;
    // MG (beta == NULL): Palimpsa-M gating, beta_t[i] = d_t
    const uint16_t* bth = MG ? nullptr : static_cast<const uint16_t*>(p.beta) + bh * p.T * DV_;
    const uint16_t* dh = static_cast<const uint16_t*>(p.d) + bh * p.T;
    const float4* sch = p.scal + bh * p.T;

    f32x4c J[MT][NT], X[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            J[m][n] = f32x4c{0.0f, 0.0f, 0.0f, 0.0f};
            X[m][n] = J[m][n];
        }

    // one block's raw operands in lane (c, g): tokens 8g + e
    struct Raw {
        uint32_t k[8][KW];   // k_t[rb + MT c .. + MT)
        uint32_t b[8][BW];   // beta_t[cb + NT c .. + NT)  (or d_t under Palimpsa-M gating)
        uint32_t v[8][BW];   // v_t[cb + NT c .. + NT)
        float ad;            // A d of token tb + (lane % 32) (0 past the end)
    };
    // tokens of the block at tb that exist (0 for a block before the sub-segment)
    auto block_len = [&](int64_t tb) -> int64_t {
        const int64_t L0 = t_end - tb;
        return (tb < t_begin || L0 < 0) ? 0 : (L0 < KB ? L0 : KB);
    };
    // A block's loads in the order of their first use: A d, beta, v, then k.
    auto load = [&](int64_t tb, Raw& x) __attribute__((always_inline)) {
        const int64_t L = block_len(tb);
        float ad[1];
        buf_load<1>(buf_rsrc(sch + tb, L * 16), static_cast<uint32_t>((lane & 31) * 16 + 12), ad);
        x.ad = ad[0];
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vh + tb * DV_, L * DV_ * 2);
        const __amdgpu_buffer_rsrc_t rb_ = MG ? buf_rsrc(dh + tb, L * 2) : buf_rsrc(bth + tb * DV_, L * DV_ * 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s_ = 8 * g + e;
            if constexpr (MG) {
                const uint32_t d1 = __builtin_amdgcn_raw_buffer_load_b16(rb_, static_cast<uint32_t>(s_ * 2), 0, 0);
#pragma unroll
                for (int h = 0; h < BW; ++h) x.b[e][h] = d1 | (d1 << 16);
            } else {
                buf_words<BW>(rb_, static_cast<uint32_t>((s_ * DV_ + cb + NT * c) * 2), NT, x.b[e]);
            }
            if constexpr (PART == 1) buf_words<BW>(rv, static_cast<uint32_t>((s_ * DV_ + cb + NT * c) * 2), NT, x.v[e]);
        }
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kh + tb * DK, L * DK * 2);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            buf_words<KW>(rk, static_cast<uint32_t>(((8 * g + e) * DK + rb + MT * c) * 2), MT, x.k[e]);
    };

    float Rsum = 0.0f;
    // One block: weights, B operands, then the A operands and MFMAs row tile
    // by row tile.
    auto compute = [&](const Raw& x) __attribute__((always_inline)) {
        // decay of token tb + t to the sub-segment's end: exp(-(Rsum + sum of
        // A d over the block's tokens after t)), by additions only
        float P = row_prefix16(x.ad);                        // inclusive, within each 16
        const int lo_bits = __builtin_amdgcn_readlane(__float_as_int(P), 15);
        P += (lane & 16) ? __int_as_float(lo_bits) : 0.0f;   // inclusive over lanes 0..31
        const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(P), 31));
        const float wt = fast_exp(-(Rsum + (total - P)));    // weight of token tb + lane % 32
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = __shfl(wt, 8 * g + e);

        // B operands: beta (exact) and the limbs of w beta v, per column tile
        u32x4c Bb[NT], B0[NT], B1[NT], B2[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e0 = 2 * q, e1 = 2 * q + 1;
                if constexpr (PART == 0) {
                    Bb[n][q] = bf_pair(x.b[e0], x.b[e1], n);
                } else {
                    const float ya = w[e0] * (bf_elem(x.b[e0], n) * bf_elem(x.v[e0], n));
                    const float yb = w[e1] * (bf_elem(x.b[e1], n) * bf_elem(x.v[e1], n));
                    uint32_t l0, l1, l2;
                    split3(ya, yb, l0, l1, l2);
                    B0[n][q] = l0;
                    B1[n][q] = l1;
                    B2[n][q] = l2;
                }
            }
        // A operands row tile by row tile: k (exact) and the limbs of w k^2
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            u32x4c Ak, A0, A1, A2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e0 = 2 * q, e1 = 2 * q + 1;
                if constexpr (PART == 1) {
                    Ak[q] = bf_pair(x.k[e0], x.k[e1], m);
                } else {
                    const float ka = bf_elem(x.k[e0], m), kb = bf_elem(x.k[e1], m);
                    uint32_t l0, l1, l2;
                    split3(w[e0] * (ka * ka), w[e1] * (kb * kb), l0, l1, l2);
                    A0[q] = l0;
                    A1[q] = l1;
                    A2[q] = l2;
                }
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if constexpr (PART == 0) J[m][n] = mfma_bf(A0, Bb[n], J[m][n]);
                else X[m][n] = mfma_bf(Ak, B0[n], X[m][n]);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if constexpr (PART == 0) J[m][n] = mfma_bf(A1, Bb[n], J[m][n]);
                else X[m][n] = mfma_bf(Ak, B1[n], X[m][n]);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if constexpr (PART == 0) J[m][n] = mfma_bf(A2, Bb[n], J[m][n]);
                else X[m][n] = mfma_bf(Ak, B2[n], X[m][n]);
            }
        }
        Rsum += total;
    };

    // Two operand sets, two blocks per trip: a block's loads are issued
    // before the other set's block is computed, so each has a whole block's
    // work to land in (a block before the sub-segment reads nothing).
    const int64_t nblk = (t_end - t_begin + KB - 1) / KB;
    Raw xa, xb;
    int64_t tb = t_begin + (nblk - 1) * KB;
    load(tb, xa);
    int64_t i = 0;
    for (; i + 2 <= nblk; i += 2, tb -= 2 * KB) {
        load(tb - KB, xb);
        compute(xa);
        load(tb - 2 * KB, xa);
        compute(xb);
    }
    if (i < nblk) compute(xa);

    const int64_t slot = u.slot;
    float* out = p.sub + slot * 2 * DK * DV_;
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
            const int64_t off = static_cast<int64_t>(rb + MT * (4 * g + r) + m) * DV_ + cb + NT * c;
            if constexpr (PART == 0) store_run<NT>(out + off, rowJ);
            else store_run<NT>(out + static_cast<int64_t>(DK) * DV_ + off, rowX);
        }
    if (PART == 0 && lane == 0 && tile == 0) p.gsub[slot] = fast_exp(-Rsum);
}

// One wave per (sub-segment, part, tile): the unit's J waves first, then its
// X waves, so that each wave holds one accumulator set (two waves per SIMD).
template <int DK, int DV>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2))) void k_diag_comp_bf(DiagParams p, int32_t R) {
    constexpr int TJ = comp_bf_tiles(DK, DV, 0);
    constexpr int TX = comp_bf_tiles(DK, DV, 1);
    const int64_t id = xcd_local_id();       // a sub-segment's tiles share an XCD
    const int tp = static_cast<int>(id % (TJ + TX));
    const int64_t unit = id / (TJ + TX);
    if (p.beta) {
        if (tp >= TJ) comp_bf_part<DK, DV, 1, false>(p, R, unit, tp - TJ);
        else comp_bf_part<DK, DV, 0, false>(p, R, unit, tp);
    } else {
        if (tp >= TJ) comp_bf_part<DK, DV, 1, true>(p, R, unit, tp - TJ);
        else comp_bf_part<DK, DV, 0, true>(p, R, unit, tp);
    }
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

// Packed batch: the ordered carry of every split sequence.  One thread per
// (split sequence, head, memory entry) runs from the sequence's own starting
// state through its segments' sub-segment composites; composite slot c of
// head h then holds the state that segment c - c0 + 1 starts from, c0 the
// sequence's first composite segment.  A grid of at most kCarryGroups
// workgroups walks the entries of the split sequences there are.
constexpr int64_t kCarryGroups = 1024;
__global__ __launch_bounds__(256) void k_varlen_carry(DiagParams p, int64_t dk, int64_t n_total) {
    const int64_t n_per_head = dk * p.dv;
    const int64_t n_seq = p.H * n_per_head;
    const int64_t nsplit = p.nwork[2];
    const int32_t R = p.nwork[3];
    for (int64_t e = elem_first(); e < n_total; e += elem_stride()) {
        const int64_t k = e / n_seq;
        if (k >= nsplit) break;   // e only grows
        const int64_t h = e % n_seq / n_per_head;
        const int64_t r = e % n_per_head;
        const int32_t sq = p.split_seq[k];
        const int32_t c0 = p.seq_comp[sq];
        if (c0 < 0) continue;
        int64_t a, b;
        sequence_tokens(p, sq, a, b);
        const int64_t nseg = varlen_segments(p, b - a);
        const int64_t off = (static_cast<int64_t>(sq) * p.H + h) * n_per_head + r;
        const float m0 = p.mu0 ? p.mu0[off] : 0.0f;
        float J = 0.0f, eta;
        if (p.I0) {
            const float I0 = p.I0[off];
            J = I0 - p.I_prior;
            eta = I0 * m0;
        } else {
            eta = p.I_prior * m0;
        }
        for (int64_t g = 0; g + 1 < nseg; ++g) {
            const int64_t c = c0 + g;
            if (c >= p.vl_comps) break;
            for (int u = 0; u < R; ++u) {
                const int64_t slot = (c * p.H + h) * R + u;
                const float* sub = p.sub + slot * 2 * n_per_head;
                const float G = p.gsub[slot];
                J = __builtin_fmaf(G, J, sub[r]);
                eta = __builtin_fmaf(G, eta, sub[n_per_head + r]);
            }
            float* cin = p.comp + (c * p.H + h) * 2 * n_per_head;
            cin[r] = J;
            cin[n_per_head + r] = eta;
        }
    }
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

template <int DK>
static int comp_bf_launch_dv(const DiagParams& p, int64_t grid, int32_t R, hipStream_t st) {
    switch (p.dv) {
        case 16: hipLaunchKernelGGL((k_diag_comp_bf<DK, 16>), dim3(grid), dim3(kWave), 0, st, p, R); break;
        case 32: hipLaunchKernelGGL((k_diag_comp_bf<DK, 32>), dim3(grid), dim3(kWave), 0, st, p, R); break;
        case 64: hipLaunchKernelGGL((k_diag_comp_bf<DK, 64>), dim3(grid), dim3(kWave), 0, st, p, R); break;
        case 128: hipLaunchKernelGGL((k_diag_comp_bf<DK, 128>), dim3(grid), dim3(kWave), 0, st, p, R); break;
        default: return KDN_EUNSUPPORTED;
    }
    return launch_status();
}

static int comp_bf_launch(const DiagParams& p, int64_t dk, int64_t grid, int32_t R, hipStream_t st) {
    switch (dk) {
        case 16: return comp_bf_launch_dv<16>(p, grid, R, st);
        case 32: return comp_bf_launch_dv<32>(p, grid, R, st);
        case 64: return comp_bf_launch_dv<64>(p, grid, R, st);
        case 128: return comp_bf_launch_dv<128>(p, grid, R, st);
        default: return KDN_EUNSUPPORTED;
    }
}

// Packed batch: composites of every split sequence's segments but its last,
// in the plan's sub-segments (the grid covers the composite storage of
// vl_comps x H x R units; waves past the plan's composites return at once),
// then the carries.
int diag_varlen_comp_launch(const DiagParams& p, int64_t dk, bool bf16, int32_t R, hipStream_t st) {
    const int64_t grid = p.vl_comps * p.H * R * comp_tiles(dk, p.dv, bf16);
    if (grid == 0) return KDN_OK;
    int rc = bf16 ? comp_bf_launch(p, dk, grid, R, st) : comp_launch<false>(p, dk, grid, R, st);
    if (rc != KDN_OK) return rc;
    const int64_t n = p.vl_comps * p.H * dk * p.dv;
    const int64_t groups = elem_groups(n) < kCarryGroups ? elem_groups(n) : kCarryGroups;
    hipLaunchKernelGGL(k_varlen_carry, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, st, p, dk, n);
    return launch_status();
}

// Composites of segments 0..S-2 in R sub-segments each (one wave per
// sub-segment and column tile), then the carry into every segment's starting
// state (p.comp).  Needs the per-token scalars.
int diag_comp_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st) {
    const int64_t BH = B * p.H;
    const int64_t grid = BH * (p.S - 1) * R * comp_tiles(dk, p.dv, bf16);
    int rc = bf16 ? comp_bf_launch(p, dk, grid, R, st) : comp_launch<false>(p, dk, grid, R, st);
    if (rc != KDN_OK) return rc;
    const int64_t n = BH * dk * p.dv;
    hipLaunchKernelGGL(k_diag_carry_sub, dim3(elem_groups(n)), dim3(256), 0, st,
                       p, dk, n, R);
    return launch_status();
}

}  // namespace kdn

// diag_bwd_kernels.h -- gradient of the diagonal-precision memory scan: the
// checkpoint and reverse-pass kernels (instantiated by diag_bwd.hip for whole
// rows and packed batches, by diag_bwd_seg.hip for rows cut into segments).
//
// Forward (Palimpsa, "Learning to Remember, Learn, and Forget in
// Attention-Based Models", Metodologia 1-2; read-out as in the KLA summary,
// Metodologia 1), per head and memory entry [j][i]:
//   I_t = alpha_t I_{t-1} + (1 - alpha_t) I_prior + beta_t[i] k_t[j]^2
//   eta_t = alpha_t eta_{t-1} + beta_t[i] v_t[i] k_t[j]     (eta = I mu)
//   mu_t = eta_t / I_t,   o_t[i] = sum_j q_t[j] mu_t[j][i],   alpha_t = exp(-A d_t)
// The pages train with these layers but print no gradient; this file runs the
// adjoint of the information form.  With g_t = q_t[j] dout_t[i] the adjoints
// of the state after token t obey, backwards in time,
//   lam_eta_t = alpha_{t+1} lam_eta_{t+1} + g_t / I_t
//   lam_I_t   = alpha_{t+1} lam_I_{t+1}  - g_t mu_t / I_t
// and the input gradients are contractions of them:
//   dbeta_t[i] = sum_j lam_I k_j^2 + lam_eta v_i k_j     dv_t[i] = beta_i sum_j lam_eta k_j
//   dk_t[j]    = sum_i 2 lam_I beta_i k_j + lam_eta beta_i v_i
//   dq_t[j]    = sum_i mu_t dout_t[i]
//   dalpha_t   = sum_ji lam_I_t (I_{t-1} - I_prior) + lam_eta_t eta_{t-1}
// The state is rebuilt as J = I - I_prior (J_t = alpha_t J_{t-1} + beta k^2)
// and eta, in the scaled frame of the forward pass (J~ = s J, eta~ = s eta
// with s = prod 1/alpha since the frame start), where both are plain
// accumulations.  The scaled adjoints L = lam_eta / s and M = lam_I / s
// accumulate the same way,
//   L += g / I~,   M -= g mu / I~     (I~ = J~ + s I_prior),
// a frame change multiplies (J~, eta~) and (L, M) by the same rho, and
//   dalpha_t = (rho_t / alpha_t) sum_ji M_t J~_{t-1} + L_t eta~_{t-1}
// involves no cancellation (J >= 0).
//
// Work decomposition (one GPU):
//   * a checkpoint pass runs the state recurrence forward and stores the state
//     before every 16-token chunk (unscaled);
//   * the reverse pass walks chunks last to first.  Inside a chunk it rebuilds
//     the states of 3 or 4 tokens at a time from the chunk's checkpoint, keeps them
//     in registers and walks those tokens backwards;
//   * lane <-> key row j, 16 value columns per lane (one DPP row of 16 lanes
//     holds the 16 columns' value-side operands, which reach the fmacs as
//     row broadcasts); a wave covers 64 rows x 16 columns and a workgroup
//     d_k rows x min(d_v, 64) columns;
//   * sums over i (dq, dk) are in-lane, then over the column waves through
//     LDS once per chunk, then over column tiles in a finishing pass; sums
//     over j (dbeta, dv) go through a 64-lane butterfly per token, then LDS.
#pragma once

#include "kdn_lane.h"
#include "kdn_params.h"

namespace kdn {

constexpr int kBwdChunk = 16;   // tokens per chunk: the checkpoint interval

// Recompute schedule of a whole chunk.  The reverse pass needs the state after
// each token, last token first; only the state before the chunk is stored.
// With `slots` register-held states, the cheapest order of checkpoint loads,
// forward steps (in place, or copied into a free slot) and reverse steps was
// found by a shortest-path search over (tokens left, states held), counting a
// copy step 1.6 in-place steps (its register moves); recompute_schedule.py in
// this directory prints these tables.  Against holding `slots` consecutive
// states rebuilt from the checkpoint each time, 3 slots need 36 steps per 16
// tokens instead of 61, and 4 slots 30 instead of 40.
enum : int8_t { kRecLoad = 0, kRecStep = 1, kRecRev = 2 };
struct RecOp {
    int8_t kind;   // kRecLoad: checkpoint -> slot dst; kRecStep: token tok from slot src into slot dst
    int8_t src;    // (src == dst: in place); kRecRev: reverse step of token tok, its state in slot src
    int8_t dst;
    int8_t tok;
};
template <int SLOTS>
struct RecSchedule;

// 16 tokens, 3 slots: 36 steps, 13 of them copies, 3 loads (cost 43.95)
template <>
struct RecSchedule<3> {
    static constexpr int N = 55;
    static constexpr RecOp ops[N] = {
        {0, 0, 0, -1},
        {1, 0, 0, 0},
        {1, 0, 0, 1},
        {1, 0, 0, 2},
        {1, 0, 0, 3},
        {1, 0, 0, 4},
        {1, 0, 0, 5},
        {1, 0, 0, 6},
        {1, 0, 1, 7},
        {1, 1, 1, 8},
        {1, 1, 1, 9},
        {1, 1, 1, 10},
        {1, 1, 1, 11},
        {1, 1, 1, 12},
        {1, 1, 2, 13},
        {1, 2, 2, 14},
        {1, 2, 2, 15},
        {2, 2, 2, 15},
        {1, 1, 2, 13},
        {1, 2, 2, 14},
        {2, 2, 2, 14},
        {1, 1, 2, 13},
        {2, 2, 2, 13},
        {2, 1, 1, 12},
        {1, 0, 1, 7},
        {1, 1, 1, 8},
        {1, 1, 1, 9},
        {1, 1, 2, 10},
        {1, 2, 2, 11},
        {2, 2, 2, 11},
        {1, 1, 2, 10},
        {2, 2, 2, 10},
        {2, 1, 1, 9},
        {1, 0, 1, 7},
        {1, 1, 2, 8},
        {2, 2, 2, 8},
        {2, 1, 1, 7},
        {2, 0, 0, 6},
        {0, 0, 0, -1},
        {1, 0, 0, 0},
        {1, 0, 0, 1},
        {1, 0, 1, 2},
        {1, 1, 1, 3},
        {1, 1, 2, 4},
        {1, 2, 2, 5},
        {2, 2, 2, 5},
        {1, 1, 2, 4},
        {2, 2, 2, 4},
        {2, 1, 1, 3},
        {1, 0, 1, 2},
        {2, 1, 1, 2},
        {2, 0, 0, 1},
        {0, 0, 0, -1},
        {1, 0, 0, 0},
        {2, 0, 0, 0}};
};

// 16 tokens, 4 slots: 30 steps, 13 of them copies, 3 loads (cost 37.95)
template <>
struct RecSchedule<4> {
    static constexpr int N = 49;
    static constexpr RecOp ops[N] = {
        {0, 0, 0, -1},
        {1, 0, 0, 0},
        {1, 0, 0, 1},
        {1, 0, 0, 2},
        {1, 0, 0, 3},
        {1, 0, 0, 4},
        {1, 0, 0, 5},
        {1, 0, 0, 6},
        {1, 0, 1, 7},
        {1, 1, 1, 8},
        {1, 1, 1, 9},
        {1, 1, 1, 10},
        {1, 1, 2, 11},
        {1, 2, 2, 12},
        {1, 2, 2, 13},
        {1, 2, 3, 14},
        {1, 3, 3, 15},
        {2, 3, 3, 15},
        {1, 2, 3, 14},
        {2, 3, 3, 14},
        {2, 2, 2, 13},
        {1, 1, 2, 11},
        {1, 2, 3, 12},
        {2, 3, 3, 12},
        {2, 2, 2, 11},
        {2, 1, 1, 10},
        {1, 0, 1, 7},
        {1, 1, 2, 8},
        {1, 2, 3, 9},
        {2, 3, 3, 9},
        {2, 2, 2, 8},
        {2, 1, 1, 7},
        {2, 0, 0, 6},
        {0, 0, 0, -1},
        {1, 0, 0, 0},
        {1, 0, 0, 1},
        {1, 0, 1, 2},
        {1, 1, 1, 3},
        {1, 1, 2, 4},
        {1, 2, 3, 5},
        {2, 3, 3, 5},
        {2, 2, 2, 4},
        {2, 1, 1, 3},
        {1, 0, 1, 2},
        {2, 1, 1, 2},
        {2, 0, 0, 1},
        {0, 0, 0, -1},
        {1, 0, 0, 0},
        {2, 0, 0, 0}};
};

template <int DK, int DV>
struct BwdShape {
    static constexpr int RH = DK / 64;                 // waves along the key rows
    static constexpr int CI = DV < 64 ? DV : 64;       // value columns per workgroup
    static constexpr int CG = CI / 16;                 // waves along the value columns
    static constexpr int W = RH * CG;
    static constexpr int NTH = W * kWave;
    static constexpr int NTILE = DV / CI;
    static constexpr int BLK = DK * CI;                // floats of one checkpoint half
    // token states held in registers at once: 3, so that two waves share a
    // SIMD (256 registers per lane) at every tile shape
    static constexpr int HELD = 3;
    static_assert(DK == 64 || DK == 128, "key rows: one or two waves of 64");
};

template <int DK, int CI, bool REV>
struct BwdStage {
    float k[kBwdChunk][DK];
    float q[REV ? kBwdChunk : 1][DK];
    float b[kBwdChunk][CI];
    float v[kBwdChunk][CI];
    float g[REV ? kBwdChunk : 1][CI];      // dout
    float4 sc[kBwdChunk + 1];              // frame scalars; [L] = next chunk's first token
};

// The reverse pass's q and dout of a chunk, single-buffered where the space
// counts: the output sums between the chunk's two barriers do not read them,
// so the next chunk's can be written there (8 KB less at d_k = 64, enough
// for two workgroups per CU).
template <int DK, int CI>
struct BwdQG {
    float q[kBwdChunk][DK];
    float g[kBwdChunk][CI];                // dout
};

// One 16-byte vector of a column tile's own operands (beta, v, dout), read
// exactly once: non-temporal, so that they do not push the chunk checkpoints
// (read up to three times) out of L2.  k and q are shared by a head's column
// tiles and stay cached.
__device__ __forceinline__ uint4 ld16_once(const void* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(u[0], u[1], u[2], u[3]);
}

// Global -> registers (in flight while the previous chunk computes) -> LDS.
template <int DK, int CI, int NTH, bool BF16, bool REV>
struct BwdLoader {
    using E = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int VW = BF16 ? 8 : 4;
    static constexpr int VK = kBwdChunk * DK / VW;
    static constexpr int VB = kBwdChunk * CI / VW;
    static constexpr int VG = kBwdChunk * CI / 4;
    static constexpr int NVK = (VK + NTH - 1) / NTH;
    static constexpr int NVB = (VB + NTH - 1) / NTH;
    static constexpr int NVG = (VG + NTH - 1) / NTH;

    uint4 rk[NVK], rq[REV ? NVK : 1], rb[NVB], rv[NVB];
    float4 rg[REV ? NVG : 1];
    float4 rsc;

    // tokens tbase + t of the token axis; t_end: the run's end (scalars past it are the identity)
    __device__ __forceinline__ void fetch(const BwdParams& p, int64_t tbase, int tile, int64_t t0,
                                          int L, int64_t t_end, int tid) {
        const E* kh = static_cast<const E*>(p.k) + tbase * DK;
        const E* qh = static_cast<const E*>(p.q) + tbase * DK;
        // beta == NULL: Palimpsa-M gating, beta_t[i] = d_t
        const E* bth = p.beta ? static_cast<const E*>(p.beta) + tbase * p.dv + tile * CI : nullptr;
        const E* dh = static_cast<const E*>(p.d) + tbase;
        const E* vh = static_cast<const E*>(p.v) + tbase * p.dv + tile * CI;
#pragma unroll
        for (int n = 0; n < NVK; ++n) {
            const int vi = tid + n * NTH;
            if (vi < VK && vi * VW < L * DK) {
                rk[n] = ld16(kh + t0 * DK + static_cast<int64_t>(vi) * VW);
                if constexpr (REV) rq[n] = ld16(qh + t0 * DK + static_cast<int64_t>(vi) * VW);
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int cv = vi % (CI / VW);
            if (vi < VB && row < L) {
                const int64_t off = (t0 + row) * p.dv + cv * VW;
                rb[n] = bth ? ld16_once(bth + off) : splat16<BF16>(dh, t0 + row);
                rv[n] = ld16_once(vh + off);
            }
        }
        if constexpr (REV) {
            const float* gh = p.dout + tbase * p.dv + tile * CI;
#pragma unroll
            for (int n = 0; n < NVG; ++n) {
                const int vi = tid + n * NTH;
                const int row = vi / (CI / 4);
                const int cv = vi % (CI / 4);
                if (vi < VG && row < L) {
                    const uint4 u = ld16_once(gh + (t0 + row) * p.dv + cv * 4);
                    rg[n] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                        __uint_as_float(u.w));
                }
            }
        }
        if (tid <= L) {
            const int64_t t = t0 + tid;
            rsc = t < t_end ? p.scal[tbase + t] : make_float4(1.0f, 0.0f, 1.0f, 0.0f);
        }
    }

    template <class St>
    __device__ __forceinline__ void commit_parts(St& S, float (*qd)[DK], float (*gd)[CI], int L, int tid) {
#pragma unroll
        for (int n = 0; n < NVK; ++n) {
            const int vi = tid + n * NTH;
            if (vi < VK && vi * VW < L * DK) {
                const int row = vi * VW / DK;
                const int c0 = vi * VW % DK;
                float f[VW];
                widen<BF16>(rk[n], f);
#pragma unroll
                for (int e = 0; e < VW; ++e) S.k[row][c0 + e] = f[e];
                if constexpr (REV) {
                    widen<BF16>(rq[n], f);
#pragma unroll
                    for (int e = 0; e < VW; ++e) qd[row][c0 + e] = f[e];
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int vi = tid + n * NTH;
            const int row = vi / (CI / VW);
            const int c0 = (vi % (CI / VW)) * VW;
            if (vi < VB && row < L) {
                float fb[VW], fv[VW];
                widen<BF16>(rb[n], fb);
                widen<BF16>(rv[n], fv);
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    S.b[row][c0 + e] = fb[e];
                    S.v[row][c0 + e] = fv[e];
                }
            }
        }
        if constexpr (REV) {
#pragma unroll
            for (int n = 0; n < NVG; ++n) {
                const int vi = tid + n * NTH;
                const int row = vi / (CI / 4);
                const int c0 = (vi % (CI / 4)) * 4;
                if (vi < VG && row < L) *reinterpret_cast<float4*>(&gd[row][c0]) = rg[n];
            }
        }
        if (tid <= L) S.sc[tid] = rsc;
    }
    __device__ __forceinline__ void commit(BwdStage<DK, CI, REV>& S, int L, int tid) {
        commit_parts(S, S.q, S.g, L, tid);
    }
    // the reverse pass: q and dout into their own single buffer
    __device__ __forceinline__ void commit(BwdStage<DK, CI, false>& S, BwdQG<DK, CI>& X, int L, int tid) {
        commit_parts(S, X.q, X.g, L, tid);
    }
};

// One forward token on a lane's 16 entries, in place:
//   state *= rho (frame change), J~ += beta_c s k_j^2, eta~ += beta_c v_c s k_j.
// bs = beta_c s and bvs = beta_c v_c s are held by lane c of each DPP row.
__device__ __forceinline__ void bwd_step_inplace(float (&I)[16], float (&E)[16], float rho,
                                                 float bs, float bvs, float kj, float k2j) {
    const uint32_t rb = __builtin_amdgcn_readfirstlane(__float_as_uint(rho));
    if (rb != 0x3f800000u) {
        const float r = __uint_as_float(rb);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            scale_inplace(I[c], r);
            scale_inplace(E[c], r);
        }
    }
    Unroll<0, 16>::run([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        fmac_bcast<c>(I[c], bs, k2j);
    });
    Unroll<0, 16>::run([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        fmac_bcast<c>(E[c], bvs, kj);
    });
}

// The same token, reading the state before it from (Ii, Ei) and writing the
// state after it to (Io, Eo).
__device__ __forceinline__ void bwd_step_copy(const float (&Ii)[16], const float (&Ei)[16],
                                              float (&Io)[16], float (&Eo)[16], float rho,
                                              float bs, float bvs, float kj, float k2j) {
    const uint32_t rb = __builtin_amdgcn_readfirstlane(__float_as_uint(rho));
    if (rb != 0x3f800000u) {
        const float r = __uint_as_float(rb);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            Io[c] = Ii[c] * r;
            Eo[c] = Ei[c] * r;
        }
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            Io[c] = Ii[c];
            Eo[c] = Ei[c];
        }
    }
    Unroll<0, 16>::run([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        fmac_bcast<c>(Io[c], bs, k2j);
    });
    Unroll<0, 16>::run([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        fmac_bcast<c>(Eo[c], bvs, kj);
    });
}

__device__ __forceinline__ void load16(const float* src, float (&x)[16]) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const float4 f = reinterpret_cast<const float4*>(src)[n];
        x[4 * n] = f.x; x[4 * n + 1] = f.y; x[4 * n + 2] = f.z; x[4 * n + 3] = f.w;
    }
}

// Checkpoint slot c (0 <= c <= nch) of run r (= bh * NTILE + tile), each slot
// 2 * BLK floats (J then eta).  Slots 0 .. nch-1 of a run are contiguous; the
// final states (slot nch) of all runs follow after every run's slots, so the
// per-run stride stays nch slots (a power of two for power-of-two T).
template <int BLK>
__device__ __forceinline__ float* ckpt_slot(float* base, int64_t r, int64_t c, int64_t nch, int64_t nruns) {
    return c < nch ? base + (r * nch + c) * 2 * BLK : base + (nruns * nch + r) * 2 * BLK;
}

// One run of the gradient: a (batch, head) row of a fixed-length batch, or a
// (sequence, head) of a packed variable-length batch, and one column tile.
struct BwdRun {
    int64_t state;      // slot of the run's starting and final states ([nruns][dk][dv])
    int64_t tbase;      // token-axis index of its row's token 0 (a token t is tbase + t)
    int64_t t_begin;    // the run's tokens on its row: [t_begin, t_end)
    int64_t t_end;
    int64_t nch;        // 16-token chunks from t_begin (the last one ragged)
    float* ck0;         // checkpoint before chunk 0; chunk c < nch at ck0 + c * 2 BLK
    float* ckfin;       // the final state
    int64_t rt;         // (row, column tile) index: row * NTILE + tile
    int seg;            // the run's segment of its row or sequence (0 when not cut)
    bool last;          // the run ends its row or sequence
    // runs in segments: its adjoint slots (adj, lam), its decay (adjg) and
    // the forward carry it starts from (comp, for seg > 0)
    int64_t slot, gidx, cslot;
    int tile;
    bool valid;         // false: a padding workgroup of a packed batch
};

// Fixed-length rows: XCD-local ids (a segment's column tiles share an XCD);
// segment `seg` of S owns the row's chunks [seg n / S, (seg + 1) n / S) of n,
// as in the forward pass's plan, and its checkpoints are that range of the
// row's (ckpt_slot).  A packed batch: runs follow the plan's longest-first
// order in groups of 8 runs x NTILE tiles (a run's tiles 8 blocks apart, so
// on one XCD), as in the forward pass; each sequence's chunks and final
// state sit at its plan offset inside its (head, tile) block of ck_stride
// slots.
template <int BLK, int NTILE, bool SEG>
__device__ __forceinline__ BwdRun bwd_run(const BwdParams& p) {
    BwdRun r;
    if (!SEG && p.cu_seqlens == nullptr) {
        // whole rows
        const int64_t wg = xcd_local_id();
        r.tile = static_cast<int>(wg % NTILE);
        const int64_t bh = wg / NTILE;
        r.seg = 0;
        r.state = bh;
        r.tbase = bh * p.T;
        r.t_begin = 0;
        r.t_end = p.T;
        r.nch = p.nchunks;
        r.last = true;
        r.rt = bh * NTILE + r.tile;
        r.ck0 = ckpt_slot<BLK>(p.ckpt, r.rt, 0, r.nch, p.nruns * NTILE);
        r.ckfin = ckpt_slot<BLK>(p.ckpt, r.rt, r.nch, r.nch, p.nruns * NTILE);
        r.valid = true;
        return r;
    }
    if (SEG && p.cu_seqlens == nullptr) {
        // the divisions leave their results in VGPRs; the run's fields are
        // wave-uniform and go back to SGPRs for the kernel's lifetime
        const int64_t wg = xcd_local_id();
        r.tile = static_cast<int>(wg % NTILE);
        const int64_t rs = wg / NTILE;
        r.seg = static_cast<int>(uniform64(rs % p.S));
        const int64_t bh = uniform64(rs / p.S);
        r.state = bh;
        r.tbase = bh * p.T;
        const int64_t n = p.nchunks;
        const int64_t c0 = uniform64(r.seg * n / p.S), c1 = uniform64((r.seg + 1) * n / p.S);
        r.t_begin = c0 * kBwdChunk;
        r.t_end = c1 * kBwdChunk < p.T ? c1 * kBwdChunk : p.T;
        r.nch = c1 - c0;
        r.last = r.seg == p.S - 1;
        r.rt = bh * NTILE + r.tile;
        r.ck0 = ckpt_slot<BLK>(p.ckpt, r.rt, c0, n, p.nruns * NTILE);
        r.ckfin = ckpt_slot<BLK>(p.ckpt, r.rt, n, n, p.nruns * NTILE);
        r.slot = r.rt * p.S + r.seg;
        r.gidx = bh * p.S + r.seg;
        r.cslot = bh * p.S + r.seg;
        r.valid = true;
        return r;
    }
    if (SEG) {
        // a packed batch whose long sequences run in segments: item `item` of
        // the forward plan (sequence sq, segment g) on head h, in groups of 8
        // runs x NTILE tiles as below
        const int64_t blk = blockIdx.x;
        const int64_t within = blk % (8 * NTILE);
        r.tile = static_cast<int>(within / 8);
        const int64_t wg = blk / (8 * NTILE) * 8 + within % 8;
        const int64_t item = uniform64(wg / p.H);
        const int64_t h = uniform64(wg % p.H);
        r.valid = item < p.nwork[0];
        if (!r.valid) return r;
        const int32_t sq = p.item_seq[item];
        r.seg = p.item_seg[item];
        int64_t a = p.cu_seqlens[sq], b = p.cu_seqlens[sq + 1];
        a = a < 0 ? 0 : (a > p.T ? p.T : a);
        b = b < a ? a : (b > p.T ? p.T : b);
        const int64_t t0 = a + static_cast<int64_t>(r.seg) * p.vl_seg;
        r.t_begin = t0 < b ? t0 : b;
        // a sequence up to vl_thr tokens long is one whole item
        const bool whole = b - a <= p.vl_thr;
        r.t_end = !whole && r.t_begin + p.vl_seg < b ? r.t_begin + p.vl_seg : b;
        r.nch = uniform64((r.t_end - r.t_begin + kBwdChunk - 1) / kBwdChunk);
        r.last = r.t_end == b;
        r.state = static_cast<int64_t>(sq) * p.H + h;
        r.rt = r.state * NTILE + r.tile;
        r.tbase = h * p.T;
        float* const base = p.ckpt + ((h * NTILE + r.tile) * p.ck_stride + p.seq_ckoff[sq]) * 2 * BLK;
        r.ck0 = base + (r.t_begin - a) / kBwdChunk * 2 * BLK;
        r.ckfin = base + (b - a + kBwdChunk - 1) / kBwdChunk * 2 * BLK;
        r.slot = (item * p.H + h) * NTILE + r.tile;
        r.gidx = item * p.H + h;
        const int32_t c0 = p.seq_comp[sq];
        r.cslot = r.seg > 0 && c0 >= 0 && c0 + r.seg - 1 < p.vl_comps ? (c0 + r.seg - 1) * p.H + h : -1;
        return r;
    }
    r.seg = 0;
    r.last = true;
    const int64_t blk = blockIdx.x;
    const int64_t within = blk % (8 * NTILE);
    r.tile = static_cast<int>(within / 8);
    const int64_t wg = blk / (8 * NTILE) * 8 + within % 8;
    r.valid = wg < static_cast<int64_t>(p.nseq) * p.H;
    if (!r.valid) return r;
    const int64_t h = uniform64(wg % p.H);
    const int32_t sq = p.seq_order[uniform64(wg / p.H)];
    r.state = static_cast<int64_t>(sq) * p.H + h;
    r.rt = r.state * NTILE + r.tile;
    r.tbase = h * p.T;
    int64_t a = p.cu_seqlens[sq], b = p.cu_seqlens[sq + 1];
    a = a < 0 ? 0 : (a > p.T ? p.T : a);
    b = b < a ? a : (b > p.T ? p.T : b);
    r.t_begin = a;
    r.t_end = b;
    r.nch = uniform64((b - a + kBwdChunk - 1) / kBwdChunk);
    r.ck0 = p.ckpt + ((h * NTILE + r.tile) * p.ck_stride + p.seq_ckoff[sq]) * 2 * BLK;
    r.ckfin = r.ck0 + r.nch * 2 * BLK;
    return r;
}

// The state before chunk c of a run (c == nch: its final state).
template <int BLK>
__device__ __forceinline__ float* ck_at(const BwdRun& r, int64_t c) {
    return c < r.nch ? r.ck0 + c * 2 * BLK : r.ckfin;
}

__device__ __forceinline__ void store16(float* dst, const float (&x)[16]) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
        reinterpret_cast<float4*>(dst)[n] = make_float4(x[4 * n], x[4 * n + 1], x[4 * n + 2], x[4 * n + 3]);
}

// A lane's 16 entries inside one checkpoint half of BLK floats are
// interleaved by float4: float4 n of lane l sits at (n * BLK/16 + l) * 4, so
// each of the four vector accesses of a wave covers 1 KB of contiguous memory.
//
// Both halves (J, then eta) of a lane's 16 entries in checkpoint slot `slot`,
// through one buffer resource: the lane's offset is one VGPR and the float4
// offsets are scalar, so no 64-bit addresses stay live between the loads.
template <int BLK>
__device__ __forceinline__ void load_ckpt(const float* slot, int64_t l, float (&J)[16], float (&E)[16]) {
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(slot, 2 * BLK * 4);
    const uint32_t vo = static_cast<uint32_t>(l) * 16;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, vo, n * BLK, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, vo, 4 * BLK + n * BLK, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            J[4 * n + i] = __uint_as_float(a[i]);
            E[4 * n + i] = __uint_as_float(b[i]);
        }
    }
}

template <int BLK>
__device__ __forceinline__ void store16_ckpt(float* half, int64_t l, const float (&x)[16]) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
        reinterpret_cast<float4*>(half)[n * (BLK / 16) + l] =
            make_float4(x[4 * n], x[4 * n + 1], x[4 * n + 2], x[4 * n + 3]);
}

// Starting state of a lane's 16 entries, unscaled: I0 (or I_prior), its
// excess J0 = I0 - I_prior, mu0 (absent: 0) and eta0 = I0 mu0.
__device__ __forceinline__ void start_state(const BwdParams& p, int64_t off, float (&I)[16],
                                            float (&J)[16], float (&E)[16], float (&m0)[16]) {
    if (p.I0) load16(p.I0 + off, I);
    else {
#pragma unroll
        for (int c = 0; c < 16; ++c) I[c] = p.I_prior;
    }
    if (p.mu0) load16(p.mu0 + off, m0);
    else {
#pragma unroll
        for (int c = 0; c < 16; ++c) m0[c] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        J[c] = I[c] - p.I_prior;
        E[c] = I[c] * m0[c];
    }
}

// ---------------------------------------------------------------------------
// Checkpoint pass: the state before every chunk, unscaled, in the slab layout
// [bh][tile][chunk][I | eta][column wave][row][16] the reverse pass reads.
// ---------------------------------------------------------------------------
// The run's adjoint slot (2 BLK floats in the checkpoint layout).
template <int BLK>
__device__ __forceinline__ float* adj_slot(float* base, const BwdRun& r) {
    return base + r.slot * 2 * BLK;
}

// With ADJ (rows cut into S > 1 segments) every segment starts from its own
// starting state (segment 0: the row's; later ones: the forward composites'
// carry), and segments 1.. also build their adjoint composite.  The adjoint
// of the state after token t obeys lam_t = alpha_{t+1} lam_{t+1} + b_t with
// b_t = (g_t / I_t, -g_t mu_t / I_t), g_t = q_t[j] dout_t[i], so for a
// segment of tokens [a, e)
//   alpha_a lam_a = sum_{t in [a, e)} P_t b_t + P_{e-1} (alpha_e lam_e),
//   P_t = prod_{u = a..t} alpha_u,
// where the sum is known from the forward states alone: it is accumulated
// here (the run's adj slot) with P_{e-1} (adjg), and a carry pass chains the
// segments from the row's or sequence's end.  The last segment stores the
// adjoint that the final state's gradients start (its lam slot).  Runs are
// a fixed-length row's segments or a packed batch's items (bwd_run).
template <int DK, int DV, bool BF16, bool ADJ>
__global__ __launch_bounds__((BwdShape<DK, DV>::NTH)) void k_diag_bwd_ckpt(BwdParams p) {
    using Sh = BwdShape<DK, DV>;
    constexpr int C = kBwdChunk;
    constexpr int CI = Sh::CI;
    __shared__ BwdStage<DK, CI, ADJ> stg[2];
    BwdLoader<DK, CI, Sh::NTH, BF16, ADJ> ld;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = tid / kWave;
    const int rh = w / Sh::CG;
    const int cg = w % Sh::CG;
    const int j = rh * 64 + lane;
    const int lc = cg * 16 + (lane & 15);      // this lane's value column in the tile (for operands)
    const BwdRun run = bwd_run<Sh::BLK, Sh::NTILE, ADJ>(p);
    if (!run.valid) return;
    if (p.cu_seqlens && p.vl_seg > 0) {
        // a packed batch that can hold split sequences: their runs take the
        // ADJ instantiation, the whole sequences' the plain one
        const bool split = p.seq_comp[uniform64(run.state / p.H)] >= 0;
        if (split != ADJ) return;
    }
    const int tile = run.tile;
    const int64_t nch = run.nch;
    const float I_prior = p.I_prior;
    const int64_t ent = (run.state * DK + j) * p.dv + tile * CI + cg * 16;   // this lane's 16 entries

    float I[16], m0[16], J[16], E[16];
    if (ADJ && run.seg > 0 && run.cslot >= 0) {
        const float* cin = p.comp + run.cslot * 2 * DK * p.dv + (ent - run.state * DK * p.dv);
        load16(cin, J);
        load16(cin + DK * p.dv, E);
    } else {
        start_state(p, ent, I, J, E, m0);
    }
    const int64_t lid = cg * DK + j;            // this lane's index in a checkpoint half
    float* ck = ck_at<Sh::BLK>(run, 0);
    store16_ckpt<Sh::BLK>(ck, lid, J);
    store16_ckpt<Sh::BLK>(ck + Sh::BLK, lid, E);

    // adjoint composite of segments 1..: sums of P_t b_t (eta and I parts)
    const bool acc = ADJ && run.seg > 0;
    float Ba[ADJ ? 16 : 1], Bb[ADJ ? 16 : 1];
    float P = 1.0f;
    if constexpr (ADJ) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            Ba[c] = 0.0f;
            Bb[c] = 0.0f;
        }
    }

    auto chunk_len = [&](int64_t c) -> int {
        const int64_t rem = run.t_end - (run.t_begin + c * C);
        return static_cast<int>(rem < C ? rem : C);
    };
    auto fetch = [&](int64_t c) { ld.fetch(p, run.tbase, tile, run.t_begin + c * C, chunk_len(c), run.t_end, tid); };
    const int64_t nrun = nch;
    if (nrun > 0) {
        fetch(0);
        ld.commit(stg[0], chunk_len(0), tid);
    }
    __syncthreads();
    if (nrun > 1) fetch(1);

    for (int64_t c = 0; c < nrun; ++c) {
        const int b = static_cast<int>(c & 1);
        const BwdStage<DK, CI, ADJ>& S = stg[b];
        const int L = chunk_len(c);
        auto token = [&](int tt) __attribute__((always_inline)) {
            const float4 sc = S.sc[tt];
            const float kj = S.k[tt][j];
            const float b = S.b[tt][lc] * sc.z;
            const float bvs = dpp_src(b * S.v[tt][lc]);
            bwd_step_inplace(J, E, sc.x, dpp_src(b), bvs, kj, kj * kj);
            if constexpr (ADJ) {
                if (acc) {
                    // (J, E): the state after token t in its frame (scale s_t):
                    // 1 / I_t = s_t / I~, mu = E / I~
                    P *= fast_exp(-uniform(sc.w));
                    const float st = uniform(sc.z);
                    const float sIp = st * I_prior;
                    const float xq = (P * st) * S.q[tt][j];
                    const float gc = dpp_src(S.g[tt][lc]);
                    const float ngc = dpp_src(-S.g[tt][lc]);
                    Unroll<0, 16>::run([&](auto cc) {
                        constexpr int e = decltype(cc)::value;
                        const float r = fast_rcp(J[e] + sIp);
                        const float xr = xq * r;
                        fmac_bcast<e>(Ba[e], gc, xr);
                        fmac_bcast<e>(Bb[e], ngc, xr * (E[e] * r));
                    });
                }
            }
        };
        if (L == C) {
            // a whole chunk, unrolled: constant stage offsets, operand reads
            // scheduled ahead by the compiler
            Unroll<0, C>::run([&](auto u) { token(decltype(u)::value); });
        } else {
            for (int tt = 0; tt < L; ++tt) token(tt);
        }
        // unscale and store the state before chunk c + 1 (the next segment
        // stores its own first one)
        const float inv_s = 1.0f / uniform(S.sc[L - 1].z);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            J[e] *= inv_s;
            E[e] *= inv_s;
        }
        if (c + 1 < nrun || run.last) {
            float* dst = ck_at<Sh::BLK>(run, c + 1);
            store16_ckpt<Sh::BLK>(dst, lid, J);
            store16_ckpt<Sh::BLK>(dst + Sh::BLK, lid, E);
        }
        if (c + 1 < nrun) ld.commit(stg[b ^ 1], chunk_len(c + 1), tid);
        __syncthreads();
        if (c + 2 < nrun) fetch(c + 2);
    }

    if constexpr (ADJ) {
        if (acc) {
            float* dst = adj_slot<Sh::BLK>(p.adj, run);
            store16_ckpt<Sh::BLK>(dst, lid, Ba);
            store16_ckpt<Sh::BLK>(dst + Sh::BLK, lid, Bb);
            if (tid == 0 && tile == 0) p.adjg[run.gidx] = P;
        }
        if (run.last) {
            // the gradients of the final state (J, E now unscaled):
            // lam_eta = dmu_T / I_T, lam_I = dI_T - dmu_T mu_T / I_T
            float La[16], Lb[16];
            Unroll<0, 16>::run([&](auto cc) {
                constexpr int e = decltype(cc)::value;
                const float gm = p.dmu_T ? p.dmu_T[ent + e] : 0.0f;
                const float gi = p.dI_T ? p.dI_T[ent + e] : 0.0f;
                const float rI = 1.0f / (J[e] + I_prior);
                La[e] = gm * rI;
                Lb[e] = gi - gm * E[e] * rI * rI;
            });
            float* dst = adj_slot<Sh::BLK>(p.lam, run);
            store16_ckpt<Sh::BLK>(dst, lid, La);
            store16_ckpt<Sh::BLK>(dst + Sh::BLK, lid, Lb);
        }
    }
}

// SEG: rows cut into segments (p.S > 1), a separate instantiation so that
// the unsegmented kernel carries none of its prologue and epilogue code.
template <int DK, int DV, bool BF16, bool SEG>
__global__ __launch_bounds__((BwdShape<DK, DV>::NTH)) __attribute__((amdgpu_waves_per_eu(2)))
void k_diag_bwd(BwdParams p) {
    using Sh = BwdShape<DK, DV>;
    constexpr int C = kBwdChunk;
    constexpr int CI = Sh::CI;
    constexpr int CG = Sh::CG;
    constexpr int RH = Sh::RH;
    constexpr int W = Sh::W;
    constexpr int NTH = Sh::NTH;
    constexpr int HELD = Sh::HELD;
    // q and dout single-buffered where that makes room for a second
    // workgroup per CU (4 or fewer waves); with 8 waves, one workgroup fills
    // the CU anyway and they stay in the double-buffered stage
    constexpr bool QG1 = W <= 4;
    using Stage = BwdStage<DK, CI, !QG1>;
    __shared__ Stage stg[2];
    __shared__ BwdQG<QG1 ? DK : 1, QG1 ? CI : 1> qg;
    __shared__ float2 dqk[C][CG][DK];          // per-wave dq and (dk / s) partial sums
    __shared__ float pq[C][RH][CG][32];        // per-wave sums over rows: P (0..15), Q (16..31)
    __shared__ float2 xs[C][W];                // per-wave dalpha sums (X1, X2) of token t + 1
    __shared__ float4 xsc[C];                  // their per-token factors
    BwdLoader<DK, CI, NTH, BF16, true> ld;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = tid / kWave;
    const int rh = w / CG;
    const int cg = w % CG;
    const int j = rh * 64 + lane;
    const int lc = cg * 16 + (lane & 15);
    auto commit_stage = [&](int bb, int L) __attribute__((always_inline)) {
        if constexpr (QG1) ld.commit(stg[bb], qg, L, tid);
        else ld.commit(stg[bb], L, tid);
    };
    const BwdRun run = bwd_run<Sh::BLK, Sh::NTILE, SEG>(p);
    if (!run.valid) return;
    const int tile = run.tile;
    const int64_t T = p.T;
    const int64_t nch = run.nch;
    const float I_prior = p.I_prior;
    const int64_t ent = (run.state * DK + j) * p.dv + tile * CI + cg * 16;   // this lane's 16 entries
    // this column tile's slices of the partial-sum buffers
    float* const part_dq = p.part_dq + tile * p.BH * T * DK;
    float* const part_dk = p.part_dk + tile * p.BH * T * DK;
    float* const part_da = p.part_da + tile * p.BH * T;
    float* const part_dip = p.part_dip + tile * p.BH * T;

    float L[16], M[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        L[c] = 0.0f;
        M[c] = 0.0f;
    }

    const int64_t lid = cg * DK + j;            // this lane's index in a checkpoint half

    auto chunk_len = [&](int64_t c) -> int {
        const int64_t rem = run.t_end - (run.t_begin + c * C);
        return static_cast<int>(rem < C ? rem : C);
    };
    auto fetch = [&](int64_t c) { ld.fetch(p, run.tbase, tile, run.t_begin + c * C, chunk_len(c), run.t_end, tid); };

    if (nch > 0) {
        fetch(nch - 1);
        commit_stage(0, chunk_len(nch - 1));
        const float inv_s = 1.0f / uniform(p.scal[run.tbase + run.t_end - 1].z);
        if (SEG && !run.last) {
            // a segment before the last: the adjoint flowing into its end,
            // unscaled, from the carry pass; to the last token's frame
            // (s = s_{e-1})
            float La[16], Lb[16];
            load_ckpt<Sh::BLK>(adj_slot<Sh::BLK>(p.lam, run), lid, La, Lb);
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                L[c] = La[c] * inv_s;
                M[c] = Lb[c] * inv_s;
            }
        } else {
            // Gradients arriving through the final state, in the last token's
            // frame (s = s_{T-1}): lam_eta = dmu_T / I_T and lam_I = dI_T -
            // dmu_T mu_T / I_T, scaled by 1 / s.  The checkpoint pass stored
            // the final state (J_T, eta_T) unscaled after the last chunk.
            float JT[16], ET[16];
            load_ckpt<Sh::BLK>(run.ckfin, lid, JT, ET);
            Unroll<0, 16>::run([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                const float gm = p.dmu_T ? p.dmu_T[ent + c] : 0.0f;
                const float gi = p.dI_T ? p.dI_T[ent + c] : 0.0f;
                const float rI = 1.0f / (JT[c] + I_prior);          // 1 / I_T
                L[c] = gm * rI * inv_s;
                M[c] = (gi - gm * ET[c] * rI * rI) * inv_s;
            });
        }
    }
    __syncthreads();

    // A reverse step's LDS operands (token tt of the staged chunk: its frame
    // scalars and the next token's, k_j, q_j, beta_c, v_c, dout_c), loaded
    // apart from the step so that a recompute step can load them ahead.
    struct RevRaw { float4 sct, scn; float k, q, b, v, g; };
    auto rev_raw = [&](const Stage& S, int tt) __attribute__((always_inline)) {
        RevRaw r;
        r.sct = S.sc[tt];
        r.scn = S.sc[tt + 1];
        r.k = S.k[tt][j];
        if constexpr (QG1) r.q = qg.q[tt][j];
        else r.q = S.q[tt][j];
        r.b = S.b[tt][lc];
        r.v = S.v[tt][lc];
        if constexpr (QG1) r.g = qg.g[tt][lc];
        else r.g = S.g[tt][lc];
        return r;
    };
    // one reverse step: token tt, (J, E) its state after the token
    auto reverse_step = [&](const RevRaw& rr, int tt, int64_t t0, int Lc,
                            const float (&J)[16], const float (&E)[16]) __attribute__((always_inline)) {
        const int64_t t = t0 + tt;
        const float4 sct = rr.sct;
        const float sIp = uniform(sct.z) * I_prior;     // s_t I_prior: I~ = J~ + s I_prior
        const bool has_next = t + 1 < run.t_end;
        {
            // dalpha of token t+1: (L, M) still belong to it (its frame), (J, E)
            // is the state before it (computed for every token, written when
            // token t+1 exists)
            float x1a = 0.0f, x1b = 0.0f, x2 = 0.0f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                x1a = fmaf(M[c], J[c], x1a);
                x1b = fmaf(L[c], E[c], x1b);
                x2 += M[c];
            }
            const float tot = wave_sum2(x1a + x1b, x2);
            if (lane == 0) xs[tt][w].x = tot;
            if (lane == 32) xs[tt][w].y = tot;
            const float4 scn = rr.scn;
            const float rho_n = has_next ? uniform(tt + 1 < Lc ? scn.x : scn.x / sct.z) : 1.0f;
            if (tid == 0 && has_next) {
                // rho_{t+1} / alpha_{t+1}: 1 / s_t where token t+1 starts a frame
                // (rho = alpha / s_t there), else 1 / alpha_{t+1}
                const bool start = __float_as_uint(rho_n) != 0x3f800000u;
                const float fac = start ? 1.0f / sct.z : fast_exp(scn.w);
                xsc[tt] = make_float4(fac, (1.0f - fast_exp(-scn.w)) * scn.z, 0.0f, 0.0f);
            }
            if (__float_as_uint(rho_n) != 0x3f800000u) {
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    scale_inplace(L[c], rho_n);
                    scale_inplace(M[c], rho_n);
                }
            }
        }

        const float kj = rr.k;
        const float qj = rr.q;
        const float k2j = kj * kj;
        const float bc = dpp_src(rr.b);
        const float bvc = dpp_src(rr.b * rr.v);
        const float gc = dpp_src(rr.g);
        const float ngc = dpp_src(-rr.g);
        float dq4[4], dka[2], dkb[2];
        // The row sums P_c = sum_j M k_j^2 and Q_c = sum_j L k_j are folded into
        // the 64-lane butterfly as soon as column c is done (the first two
        // levels pair P_c with Q_c, then column c with c + 8).
        float wlo[8], x8[8];
        Unroll<0, 16>::run([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            const float r = fast_rcp(J[c] + sIp);
            const float mu = E[c] * r;
            const float qr = qj * r;
            fmac_bcast<c>(L[c], gc, qr);                    // L += q_j dout_c / I~
            fmac_bcast<c>(M[c], ngc, qr * mu);              // M -= q_j dout_c mu / I~
            // dq_j += dout_c mu; sum_c beta_c M; sum_c beta_c v_c L (first
            // products start the accumulators)
            if constexpr (c < 4) dq4[c] = bcast<c>(gc) * mu;
            else fmac_bcast<c>(dq4[c & 3], gc, mu);
            if constexpr (c < 2) {
                dka[c] = bcast<c>(bc) * M[c];
                dkb[c] = bcast<c>(bvc) * L[c];
            } else {
                fmac_bcast<c>(dka[c & 1], bc, M[c]);
                fmac_bcast<c>(dkb[c & 1], bvc, L[c]);
            }
            const float wc = swap32_add(M[c] * k2j, L[c] * kj);
            if constexpr (c < 8) wlo[c] = wc;
            else x8[c - 8] = swap16_add(wlo[c - 8], wc);
        });
        const float red = wave_sum32_tail(x8, lane);
        if (!(lane & 1)) pq[tt][rh][cg][(lane >> 5) * 16 + ((lane >> 1) & 15)] = red;
        dqk[tt][cg][j] = make_float2((dq4[0] + dq4[1]) + (dq4[2] + dq4[3]),
                                     2.0f * kj * (dka[0] + dka[1]) + (dkb[0] + dkb[1]));
    };

    for (int64_t c = nch - 1; c >= 0; --c) {
        const int b = static_cast<int>((nch - 1 - c) & 1);
        const Stage& S = stg[b];
        const int Lc = chunk_len(c);
        const int64_t t0 = run.t_begin + c * C;
        const float* ck = ck_at<Sh::BLK>(run, c);
        const int nheld = (Lc + HELD - 1) / HELD;
        auto operands = [&](int tt, float& rho, float& bs, float& bvs,
                            float& kj) __attribute__((always_inline)) {
            const float4 sc = S.sc[tt];
            rho = sc.x;
            kj = S.k[tt][j];
            const float b = S.b[tt][lc] * sc.z;
            bvs = dpp_src(b * S.v[tt][lc]);
            bs = dpp_src(b);
        };

        if (Lc == C) {
            // a whole chunk: the fixed recompute schedule, unrolled (slot
            // indices and stage offsets are constants)
            using RS = RecSchedule<HELD>;
            float sJ[HELD][16], sE[HELD][16];
            // a step's LDS operands: frame scalars (rho, s), k_j, beta_c, v_c
            struct Raw { float scx, scz, k, b, v; };
            auto raw = [&](int tt) __attribute__((always_inline)) {
                Raw r;
                const float4 sc = S.sc[tt];
                r.scx = sc.x;
                r.scz = sc.z;
                r.k = S.k[tt][j];
                r.b = S.b[tt][lc];
                r.v = S.v[tt][lc];
                return r;
            };
            Raw pre{};
            RevRaw rpre{};
            Unroll<0, RS::N>::run([&](auto ii) {
                constexpr int i = decltype(ii)::value;
                constexpr RecOp op = RS::ops[i];
                if constexpr (op.kind == kRecLoad) {
                    load_ckpt<Sh::BLK>(ck, lid, sJ[op.dst], sE[op.dst]);
                } else if constexpr (op.kind == kRecStep) {
                    // A step right after a step finds its operands loaded; a
                    // step right before a step or a reverse step loads that
                    // one's before its own arithmetic, so their LDS latency
                    // overlaps it.
                    constexpr int ip = i > 0 ? i - 1 : 0;
                    constexpr int in = i + 1 < RS::N ? i + 1 : i;
                    constexpr bool pre_in = i > 0 && RS::ops[ip].kind == kRecStep;
                    constexpr bool pre_out = i + 1 < RS::N && RS::ops[in].kind == kRecStep;
                    constexpr bool pre_rev = i + 1 < RS::N && RS::ops[in].kind == kRecRev;
                    Raw o;
                    if constexpr (pre_in) o = pre;
                    else o = raw(op.tok);
                    if constexpr (pre_out) pre = raw(RS::ops[in].tok);
                    if constexpr (pre_rev) rpre = rev_raw(S, RS::ops[in].tok);
                    const float rho = o.scx;
                    const float kj = o.k;
                    const float bb = o.b * o.scz;
                    const float bvs = dpp_src(bb * o.v);
                    const float bs = dpp_src(bb);
                    if constexpr (op.src == op.dst)
                        bwd_step_inplace(sJ[op.dst], sE[op.dst], rho, bs, bvs, kj, kj * kj);
                    else
                        bwd_step_copy(sJ[op.src], sE[op.src], sJ[op.dst], sE[op.dst], rho, bs, bvs, kj,
                                      kj * kj);
                } else {
                    constexpr int ip = i > 0 ? i - 1 : 0;
                    if constexpr (i > 0 && RS::ops[ip].kind == kRecStep)
                        reverse_step(rpre, op.tok, t0, Lc, sJ[op.src], sE[op.src]);
                    else
                        reverse_step(rev_raw(S, op.tok), op.tok, t0, Lc, sJ[op.src], sE[op.src]);
                }
                // keep each op's loads and temporaries within the op (beyond
                // the prefetch above): hoisting across ops raises register
                // pressure past the budget
                __builtin_amdgcn_sched_barrier(0);
            });
        }

        // the ragged last chunk: groups of HELD consecutive states, each
        // rebuilt from the checkpoint
        for (int m = Lc == C ? -1 : nheld - 1; m >= 0; --m) {
            float gJ[HELD][16], gE[HELD][16];
            load_ckpt<Sh::BLK>(ck, lid, gJ[0], gE[0]);
            {
                // software-pipelined like the checkpoint pass
                const int n = HELD * m;
                float2 scx = make_float2(S.sc[0].x, S.sc[0].z);
                float kj = S.k[0][j], bj = S.b[0][lc], vj = S.v[0][lc];
                for (int tt = 0; tt < n; ++tt) {
                    const int tn = tt + 1 < n ? tt + 1 : tt;
                    const float2 scx_n = make_float2(S.sc[tn].x, S.sc[tn].z);
                    const float kj_n = S.k[tn][j], bj_n = S.b[tn][lc], vj_n = S.v[tn][lc];
                    const float b = bj * scx.y;
                    const float bvs = dpp_src(b * vj);
                    bwd_step_inplace(gJ[0], gE[0], scx.x, dpp_src(b), bvs, kj, kj * kj);
                    scx = scx_n;
                    kj = kj_n;
                    bj = bj_n;
                    vj = vj_n;
                }
            }
            Unroll<0, HELD>::run([&](auto uu) {
                constexpr int u = decltype(uu)::value;
                const int tt = HELD * m + u;
                if (tt < Lc) {
                    float rho, bs, bvs, kj;
                    operands(tt, rho, bs, bvs, kj);
                    if constexpr (u == 0)
                        bwd_step_inplace(gJ[0], gE[0], rho, bs, bvs, kj, kj * kj);
                    else
                        bwd_step_copy(gJ[u - 1], gE[u - 1], gJ[u], gE[u], rho, bs, bvs, kj, kj * kj);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            Unroll<0, HELD>::run([&](auto uu) {
                constexpr int u = HELD - 1 - decltype(uu)::value;
                const int tt = HELD * m + u;
                if (tt < Lc) reverse_step(rev_raw(S, tt), tt, t0, Lc, gJ[u], gE[u]);
            });
        }

        __syncthreads();
        // the previous chunk's loads fly while this chunk's outputs are written
        if (c > 0) fetch(c - 1);

        // ---- chunk outputs ---- (written once and read only by later
        // passes: non-temporal, so that they do not push this pass's chunk
        // checkpoints, read up to three times, out of L2)
        const int64_t tokbase = run.tbase + t0;                   // token index into the token axis
        for (int e = tid; e < Lc * CI; e += NTH) {
            const int tt = e / CI;
            const int ci = e % CI;
            const int g = ci / 16;
            const int cc = ci % 16;
            float P = 0.0f, Q = 0.0f;
#pragma unroll
            for (int r = 0; r < RH; ++r) {
                P += pq[tt][r][g][cc];
                Q += pq[tt][r][g][16 + cc];
            }
            const float s = S.sc[tt].z;
            const float bi = S.b[tt][ci];
            const float vi = S.v[tt][ci];
            const int64_t o = (tokbase + tt) * p.dv + tile * CI + ci;
            if (p.dbeta) __builtin_nontemporal_store(s * fmaf(vi, Q, P), &p.dbeta[o]);
            __builtin_nontemporal_store(s * bi * Q, &p.dv_out[o]);
        }
        if (!p.beta) {
            // Palimpsa-M gating: beta_t[i] = d_t, so d_t collects sum_i dbeta_t[i]
            float* const part_db = p.part_db + tile * p.BH * T;
            for (int tt = tid; tt < Lc; tt += NTH) {
                float sum = 0.0f;
                for (int ci = 0; ci < CI; ++ci) {
                    float P = 0.0f, Q = 0.0f;
#pragma unroll
                    for (int r = 0; r < RH; ++r) {
                        P += pq[tt][r][ci / 16][ci % 16];
                        Q += pq[tt][r][ci / 16][16 + ci % 16];
                    }
                    sum += fmaf(S.v[tt][ci], Q, P);
                }
                part_db[tokbase + tt] = S.sc[tt].z * sum;
            }
        }
        for (int e = tid; e < Lc * DK; e += NTH) {
            const int tt = e / DK;
            const int jj = e % DK;
            float sq = 0.0f, sk = 0.0f;
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                const float2 x = dqk[tt][g][jj];
                sq += x.x;
                sk += x.y;
            }
            const int64_t o = (tokbase + tt) * DK + jj;
            __builtin_nontemporal_store(sq, &part_dq[o]);
            __builtin_nontemporal_store(sk * S.sc[tt].z, &part_dk[o]);
        }
        for (int tt = tid; tt < Lc; tt += NTH) {
            if (t0 + tt + 1 < run.t_end) {
                float X1 = 0.0f, X2 = 0.0f;
#pragma unroll
                for (int ww = 0; ww < W; ++ww) {
                    X1 += xs[tt][ww].x;
                    X2 += xs[tt][ww].y;
                }
                const float4 f = xsc[tt];
                part_da[tokbase + tt + 1] = f.x * X1;
                part_dip[tokbase + tt + 1] = f.y * X2;
            }
        }
        if (c > 0) commit_stage(b ^ 1, chunk_len(c - 1));
        __syncthreads();
    }

    // ---- the starting state (before token 0; for a later segment of a
    //      row, the state before its first token, its first checkpoint) ----
    float I0[16], J0[16], E0[16], m0[16];
    if (SEG && run.seg > 0) load_ckpt<Sh::BLK>(ck_at<Sh::BLK>(run, 0), lid, J0, E0);
    else start_state(p, ent, I0, J0, E0, m0);
    __shared__ float2 xfin[W];
    float di[16], dm[16];   // gradients of the starting state's I0 and mu0
    if (run.t_end > run.t_begin) {
        float x1a = 0.0f, x1b = 0.0f, x2 = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            x1a = fmaf(M[c], J0[c], x1a);
            x1b = fmaf(L[c], E0[c], x1b);
            x2 += M[c];
        }
        const float tot = wave_sum2(x1a + x1b, x2);
        if (lane == 0) xfin[w].x = tot;
        if (lane == 32) xfin[w].y = tot;
        // token 0 starts a frame with s = 1 and rho = alpha_0
        const float alpha0 = fast_exp(-uniform(p.scal[run.tbase + run.t_begin].w));
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            L[c] *= alpha0;
            M[c] *= alpha0;
        }
        __syncthreads();
        if (tid == 0) {
            float X1 = 0.0f, X2 = 0.0f;
            for (int ww = 0; ww < W; ++ww) {
                X1 += xfin[ww].x;
                X2 += xfin[ww].y;
            }
            part_da[run.tbase + run.t_begin] = X1;
            part_dip[run.tbase + run.t_begin] = (1.0f - alpha0) * X2;
        }
        // a later segment's first token is not the row's: the starting
        // state's gradients belong to segment 0
        if (SEG && run.seg > 0) return;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            di[c] = fmaf(L[c], m0[c], M[c]);   // through I0 directly and through eta0 = I0 mu0
            dm[c] = L[c] * I0[c];
        }
    } else {
        // no token: the final state is the starting state
        if (p.dmu_T) load16(p.dmu_T + ent, dm);
        else {
#pragma unroll
            for (int c = 0; c < 16; ++c) dm[c] = 0.0f;
        }
        if (p.dI_T) load16(p.dI_T + ent, di);
        else {
#pragma unroll
            for (int c = 0; c < 16; ++c) di[c] = 0.0f;
        }
    }
    if (p.dI0 && p.I0) store16(p.dI0 + ent, di);
    if (p.dmu0 && p.mu0) store16(p.dmu0 + ent, dm);
    __syncthreads();
    {
        float x = 0.0f;
        if (!p.I0) {
#pragma unroll
            for (int c = 0; c < 16; ++c) x += di[c];
        }
        const float tot = wave_sum2(x, 0.0f);
        if (lane == 0) xfin[w].x = tot;
        __syncthreads();
        if (tid == 0) {
            float X = 0.0f;
            for (int ww = 0; ww < W; ++ww) X += xfin[ww].x;
            p.part_dip0[tile * p.nruns + run.state] = X;
        }
    }
}

}  // namespace kdn

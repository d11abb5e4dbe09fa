// kdn_params.h -- kernel parameter blocks and launcher entry points shared
// between the C-ABI layer and the kernel translation units.
#pragma once

#include "kdn_internal.h"

namespace kdn {

// Segmented scan over a d_k x d_v state per head: the diagonal-precision scan,
// or the gated mean of the isotropic filter (F, G set, beta/d unused).
struct DiagParams {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;   // diagonal: beta [BH,T,dv]
    const void* d;      // diagonal: d [BH,T]
    const float* F;     // isotropic: forget gate F_t [BH,T]
    const float* G;     // isotropic: write gate G_t [BH,T]
    const float* A;
    const float* I0;
    const float* mu0;
    float* o;
    float* I_T;
    float* mu_T;
    float4* scal;  // [BH][T] per-token scalars of the diagonal scan (rho, dP, s, -log alpha)
    float* comp;   // [BH][S][2][dk][dv]: segment composites, then carry-in states
    float* gdec;   // [BH][S]: decay product of each segment (isotropic scan)
    float* sub;    // [BH][S-1][R][2][dk][dv]: sub-segment composites (diagonal scan)
    float* gsub;   // [BH][S-1][R]: decay product of each sub-segment
    int64_t H;
    int64_t T;
    int64_t dv;
    float I_prior;
    int32_t S;
    int32_t nchunks;
    const int64_t* cu_seqlens;   // packed variable-length batch: [nseq + 1] offsets, or NULL
    int32_t* seq_order;          // its sequences, longest first (written by the plan pass)
    int32_t nseq;
    int64_t* echo;               // bounds echo (kdn_scan_opts), or NULL
    int64_t echo_cap;            // its capacity in int64 words
    int64_t echo_base;           // first record slot of the launch being made
    void* main_begin;            // caller's events around the main pass (kdn_scan_opts), or NULL
    void* main_end;
};

// ---------------------------------------------------------------------------
// Token bounds of the work units: every kernel takes them from these, and the
// bounds echo reports what they returned.
// ---------------------------------------------------------------------------

// Packed variable-length batch: tokens of sequence s, [cu[s], cu[s+1]),
// clamped into [0, T] so that a malformed offset table cannot send a
// workgroup out of bounds.
__device__ __forceinline__ void sequence_tokens(const DiagParams& p, int32_t s, int64_t& t0,
                                                int64_t& t1) {
    int64_t a = p.cu_seqlens[s], b = p.cu_seqlens[s + 1];
    a = a < 0 ? 0 : (a > p.T ? p.T : a);
    b = b < a ? a : (b > p.T ? p.T : b);
    t0 = a;
    t1 = b;
}

// The sequence holding packed token t: the last s with cu[s] <= t.
__device__ __forceinline__ int32_t find_sequence(const DiagParams& p, int64_t t) {
    int32_t lo = 0, hi = p.nseq;
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) / 2;
        if (p.cu_seqlens[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Plan of a packed batch, run by one workgroup of kPlanThreads: order[rank] =
// s with the sequences ranked longest first (ties by index), by counting.
// Lengths are staged in LDS (lens, kPlanLds entries) when they fit; past
// kMaxPlanSort sequences the quadratic count is skipped and the order is the
// identity.  Every thread of the workgroup must call it.
constexpr int32_t kPlanThreads = 1024;
constexpr int32_t kPlanLds = 4096;
constexpr int32_t kMaxPlanSort = 16384;

__device__ __forceinline__ int64_t clamped_length(const int64_t* cu, int64_t T, int32_t s) {
    int64_t a = cu[s], b = cu[s + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    b = b < a ? a : (b > T ? T : b);
    return b - a;
}

__device__ inline void plan_longest_first(const int64_t* cu, int32_t n, int64_t T, int32_t* order,
                                          int64_t* lens) {
    const bool staged = n <= kPlanLds;
    if (staged) {
        for (int32_t s = threadIdx.x; s < n; s += kPlanThreads) lens[s] = clamped_length(cu, T, s);
        __syncthreads();
    }
    for (int32_t s = threadIdx.x; s < n; s += kPlanThreads) {
        int32_t rank = s;
        if (n <= kMaxPlanSort) {
            const int64_t ls = staged ? lens[s] : clamped_length(cu, T, s);
            rank = 0;
            for (int32_t u = 0; u < n; ++u) {
                const int64_t lu = staged ? lens[u] : clamped_length(cu, T, u);
                rank += (lu > ls || (lu == ls && u < s)) ? 1 : 0;
            }
        }
        order[rank] = s;
    }
}

// Token bounds of segment `seg`: whole chunks [seg*n/S, (seg+1)*n/S) of the
// n = p.nchunks chunks of C tokens.
__device__ __forceinline__ void segment_tokens(const DiagParams& p, int C, int seg,
                                               int64_t& t0, int64_t& t1) {
    const int64_t c0 = static_cast<int64_t>(seg) * p.nchunks / p.S;
    const int64_t c1 = static_cast<int64_t>(seg + 1) * p.nchunks / p.S;
    t0 = c0 * C;
    t1 = c1 * C < p.T ? c1 * C : p.T;
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

// One bounds-echo record {kind, run, segment, part, t_begin, t_end,
// sequence, 0} at slot p.echo_base + unit, if an echo buffer was given and
// the record fits.  Called by one lane per work unit.
constexpr int kEchoWords = KDN_ECHO_WORDS;
__device__ __forceinline__ void echo_bounds(const DiagParams& p, int64_t unit, int64_t kind, int64_t run,
                                            int64_t seg, int64_t part, int64_t t0, int64_t t1,
                                            int64_t sequence) {
    if (p.echo == nullptr) return;
    const int64_t slot = p.echo_base + unit;
    if ((slot + 1) * kEchoWords > p.echo_cap) return;
    int64_t* r = p.echo + slot * kEchoWords;
    r[0] = kind;
    r[1] = run;
    r[2] = seg;
    r[3] = part;
    r[4] = t0;
    r[5] = t1;
    r[6] = sequence;
    r[7] = 0;
}

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const void* d;
    const float* A;
    float* I;
    float* mu;
    float* o;
    int64_t H;
    float I_prior;
};

struct MobParams {
    const float* a;
    const float* p;
    const float* Lam;
    const float* lambda0;
    float* lambda_out;
    float* F;        // [BH,T] forget gates (NULL: precision path only)
    float* G;        // [BH,T] write gates
    float* blk;      // [BH][nblk][4] block composites
    int64_t T;
    int32_t nblk;
};

// Diagonal KDN with process noise: per-entry scalar Kalman filter.
struct NoiseParams {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const float* a;       // [BH,T] decay
    const float* p;       // [BH,T] process-noise variance
    const float* lam0;    // [BH,dk,dv] or NULL (-> 1)
    const float* mu0;     // [BH,dk,dv] or NULL (-> 0)
    float* o;             // [BH,T,dv]
    float* lam_T;         // [BH,dk,dv] or NULL
    float* mu_T;          // [BH,dk,dv] or NULL
    int64_t H;
    int64_t T;
    int64_t dv;
};

int noise_launch(const NoiseParams& p, int64_t B, int64_t dk, bool bf16, hipStream_t st);

// Gradient of the diagonal-precision scan.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* beta;
    const void* d;
    const float* A;
    const float* I0;
    const float* mu0;
    const float* dout;    // [BH,T,dv]
    const float* dI_T;    // [BH,dk,dv] or NULL
    const float* dmu_T;   // [BH,dk,dv] or NULL
    float* dv_out;        // [BH,T,dv]
    float* dbeta;         // [BH,T,dv]
    float* dd;            // [BH,T]
    float* dA;            // [H]
    float* dI_prior;      // [1] or NULL
    float* dI0;           // [BH,dk,dv] or NULL
    float* dmu0;          // [BH,dk,dv] or NULL
    float* dq;            // [BH,T,dk]
    float* dk;            // [BH,T,dk]
    const float4* scal;   // [BH][T] frame scalars (rho, dP, s, A d) from the prep pass
    float* ckpt;          // [BH][ntile][nch+1][2][dk*CI]: state before each chunk and the final state, unscaled
    float* part_dq;       // [ntile][BH,T,dk] column-tile partial sums (== dq when ntile == 1)
    float* part_dk;       // [ntile][BH,T,dk] (== dk when ntile == 1)
    float* part_da;       // [ntile][BH,T]: d loss / d alpha_t per column tile
    float* part_dip;      // [ntile][BH,T]: d loss / d I_prior through token t, per tile
    float* part_dip0;     // [ntile][BH]: through the starting state (I0 == NULL)
    float* part_db;       // [ntile][BH,T]: sum_i dbeta_t[i] per tile (Palimpsa-M gating only)
    float* part_head;     // [BH][tok_split][2]: sums of the dA and dI_prior terms per token range
    int64_t BH;           // token rows: B*H, or H for a packed batch (its token axis is [H, total_T])
    int64_t H;
    int64_t T;            // tokens per row (total_T for a packed batch)
    int64_t dv;
    float I_prior;
    int32_t nchunks;      // chunks per row (fixed-length rows only)
    int32_t ntile;
    int32_t tok_split;    // token ranges per row in the finishing sums (bwd_token_split)
    // packed variable-length batch (cu_seqlens != NULL): runs are (sequence, head)
    const int64_t* cu_seqlens;   // [nseq + 1] token offsets into total_T
    int32_t* seq_order;          // sequences, longest first (written by the plan pass)
    int64_t* seq_ckoff;          // [nseq] first checkpoint slot of each sequence (plan pass)
    int32_t nseq;
    int64_t nruns;               // state slots: B*H, or nseq*H
    int64_t ck_stride;           // checkpoint slots per (head, column tile) of a packed batch
};

int diag_chunk();
int varlen_cols(int64_t dv);
int32_t bwd_token_split(int64_t rows, int64_t T);
int diag_bwd_launch(const BwdParams& p, const DiagParams& prep, int64_t B, int64_t dk,
                    bool bf16, hipStream_t st);
int diag_varlen_bwd_launch(const BwdParams& p, const DiagParams& prep, int64_t dk, bool bf16,
                           hipStream_t st);
int diag_prep_launch(const DiagParams& p, int64_t B, bool bf16, bool true_i, hipStream_t st);
int diag_prep_varlen_launch(const DiagParams& p, bool bf16, bool true_i, hipStream_t st);
int diag_scan_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st);
int diag_varlen_launch(const DiagParams& p, int64_t dk, bool bf16, hipStream_t st);
int copy_state_launch(const DiagParams& p, int64_t B, int64_t dk, bool iso, hipStream_t st);
int decode_launch(const DecodeParams& p, int64_t B, int64_t dk, int64_t dv, bool bf16, hipStream_t st);
int comp_tiles(int64_t dk, int64_t dv, bool bf16);
int diag_comp_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st);
int diag_carry_launch(const DiagParams& p, int64_t B, int64_t dk, bool iso, hipStream_t st);
int mob_block();
int mobius_launch(const MobParams& p, int64_t BH, hipStream_t st);
int iso_chunk();
int iso_tiles(int64_t dv);
int iso_mean_launch(const DiagParams& p, int64_t B, int64_t dk, hipStream_t st);

}  // namespace kdn

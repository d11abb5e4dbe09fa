// kdn_params.h -- kernel parameter blocks and launcher entry points shared
// between the C-ABI layer and the kernel translation units.
#pragma once

#include "kdn_internal.h"

namespace kdn {

// Segmented scan over a d_k x d_v state per head: the diagonal-precision scan,
// or the gated mean of the isotropic filter (F, G set, beta/d unused).
// One main-pass item of a packed batch as the plan writes it: everything a
// workgroup needs in one 32-byte record.
struct VarlenItemRec {
    int64_t t_begin, t_end;     // packed tokens of the segment
    int32_t sq;                 // its sequence, or -1 past the plan's items
    int32_t seg;                // its segment within the sequence
    int32_t carry;              // composite slot of its starting state, or -1 (the sequence's own)
    int32_t last;               // 1: the sequence's last segment (writes the final state)
};

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
    // Packed batch: sequences longer than vl_thr tokens are cut into segments
    // of vl_seg tokens (the last one shorter); the plan pass writes the tables.
    // A packed batch's comp / sub / gsub are indexed by composite segment c
    // (a segment that is not its sequence's last): comp [vl_comps][H][2][dk][dv]
    // holds the carry into segment c + 1 of its sequence, sub
    // [vl_comps][H][R][2][dk][dv] and gsub [vl_comps][H][R] its sub-segments.
    int32_t* item_seq;           // [vl_items] sequence of each main-pass item, dispatch order
    int32_t* item_seg;           // [vl_items] the item's segment within its sequence
    struct VarlenItemRec* items; // [vl_items] each item's bounds and carry (sq < 0: past the plan's items)
    int32_t* seq_comp;           // [nseq] first composite segment of a split sequence, else -1
    int32_t* comp_seq;           // [vl_comps] sequence of each composite segment
    int32_t* comp_seg;           // [vl_comps] its segment within the sequence
    int32_t* split_seq;          // [vl_comps] the split sequences, in plan order
    int32_t* seq_item;           // [nseq] first item of each sequence, or NULL (not written)
    int32_t* nwork;              // [4]: items, composite segments, split sequences (each <= capacity),
                                 // sub-segments per composite segment
    int64_t vl_seg;              // segment length of a split sequence (multiple of 256), 0 = no split
    int64_t vl_thr;              // a sequence is split when longer than this (>= vl_seg)
    int64_t vl_items;            // capacity of the item tables
    int64_t vl_comps;            // capacity of the composite tables
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

constexpr int kDiagChunkTokens = 16;   // tokens per chunk of the diagonal scan

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

// Packed batch: segments of a sequence of len tokens (1 when it is not split).
__device__ __forceinline__ int64_t varlen_segments(const DiagParams& p, int64_t len) {
    return p.vl_seg > 0 && len > p.vl_thr ? (len + p.vl_seg - 1) / p.vl_seg : 1;
}

// One main-pass work item of a packed batch, run wg = item * H + head: the
// item's sequence and segment from the plan's tables, its tokens (segment g
// of sequence s holds [cu[s] + g vl_seg, min(cu[s] + (g + 1) vl_seg,
// cu[s+1]))), whether it is the sequence's last segment (it then writes the
// final state), and the composite slot holding its starting state (-1: the
// sequence's own starting state).  False past the plan's items.
struct VarlenItem {
    int64_t bh, sb, t_begin, t_end, carry;
    int32_t sq, seg;
    bool last;
};

__device__ __forceinline__ bool varlen_item(const DiagParams& p, int64_t wg, VarlenItem& it) {
    const int64_t item = wg / p.H;
    if (item >= p.vl_items) return false;
    // one record, written by the plan for every slot up to the capacity
    const int4* rec = reinterpret_cast<const int4*>(p.items + item);
    const int4 lo = rec[0], hi = rec[1];
    it.sq = hi.x;
    if (it.sq < 0) return false;
    it.bh = wg % p.H;
    it.t_begin = (static_cast<int64_t>(static_cast<uint32_t>(lo.y)) << 32) | static_cast<uint32_t>(lo.x);
    it.t_end = (static_cast<int64_t>(static_cast<uint32_t>(lo.w)) << 32) | static_cast<uint32_t>(lo.z);
    it.seg = hi.y;
    it.carry = hi.z;
    it.last = hi.w != 0;
    it.sb = static_cast<int64_t>(it.sq) * p.H + it.bh;
    return true;
}

// One composite unit of a packed batch, rest = (c * H + h) * R + u with R
// the plan's sub-segments per composite segment (nwork[3]): sub-segment u of
// composite segment c (segment `seg` of sequence `sq`) on head h, the
// segment's vl_seg / 16 chunks split evenly over R.  Its output slot is
// rest.  False past the plan's composite segments.
__device__ __forceinline__ bool varlen_comp_unit(const DiagParams& p, int64_t rest,
                                                 int64_t& h, int32_t& sq, int32_t& seg, int32_t& sub,
                                                 int64_t& t0, int64_t& t1) {
    const int32_t R = p.nwork[3];
    sub = static_cast<int32_t>(rest % R);
    const int64_t ch = rest / R;
    h = ch % p.H;
    const int64_t c = ch / p.H;
    if (c >= p.nwork[1]) return false;
    sq = p.comp_seq[c];
    seg = p.comp_seg[c];
    int64_t a, b;
    sequence_tokens(p, sq, a, b);
    const int64_t m = p.vl_seg / kDiagChunkTokens;
    const int64_t s0 = a + static_cast<int64_t>(seg) * p.vl_seg;
    const int64_t x0 = s0 + (sub * m / R) * kDiagChunkTokens;
    const int64_t x1 = s0 + ((sub + 1) * m / R) * kDiagChunkTokens;
    t0 = x0 < b ? x0 : b;
    t1 = x1 < b ? x1 : b;
    return true;
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
                                            int64_t sequence, int64_t extra = 0) {
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
    r[7] = extra;
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
    // Fixed-length rows cut into S segments of whole chunks (S == 1: none;
    // always 1 for a packed batch).  Slots of 2 dk*CI floats in the
    // checkpoint layout, per (row, column tile, segment):
    int32_t S;
    const float* comp;           // [BH][S][2][dk][dv]: each segment's starting (I - I_prior, eta)
    float* adj;                  // [BH*ntile][S][slot]: segment s's adjoint composite (s >= 1)
    float* lam;                  // [BH*ntile][S][slot]: the adjoint flowing into segment s's end
    float* adjg;                 // [BH][S]: product of alpha over segment s
    // A packed batch whose long sequences run in segments (vl_seg > 0): the
    // forward plan's tables; runs are (item, head, tile); comp holds the
    // forward composites' carries [vl_comps][H][2][dk][dv]; adj and lam are
    // [vl_items][H][ntile][slot], adjg [vl_items][H].
    const int32_t* item_seq;
    const int32_t* item_seg;
    const int32_t* seq_item;
    const int32_t* seq_comp;
    const int32_t* split_seq;
    const int32_t* nwork;
    int64_t vl_seg;
    int64_t vl_thr;
    int64_t vl_items;
    int64_t vl_comps;
};

int diag_chunk();
int varlen_cols(int64_t dv);
int diag_varlen_comp_launch(const DiagParams& p, int64_t dk, bool bf16, int32_t R, hipStream_t st);
int32_t bwd_token_split(int64_t rows, int64_t T);
int diag_bwd_launch(const BwdParams& p, const DiagParams& prep, int64_t B, int64_t dk,
                    bool bf16, int32_t R, hipStream_t st);
// join: where non-null, an event the reverse pass waits for on st (the
// whole sequences' checkpoint pass of a packed batch, run on another stream)
int diag_bwd_seg_launch(const BwdParams& p, int64_t dk, bool bf16, hipStream_t st, hipEvent_t join = nullptr);
void varlen_plan_launch(const DiagParams& p, int32_t R, hipStream_t st);
int diag_varlen_bwd_launch(const BwdParams& p, const DiagParams& prep, int64_t dk, bool bf16,
                           int32_t R, hipStream_t st);
int diag_prep_launch(const DiagParams& p, int64_t B, bool bf16, bool true_i, hipStream_t st);
int diag_prep_varlen_launch(const DiagParams& p, bool bf16, bool true_i, hipStream_t st);
int diag_scan_launch(const DiagParams& p, int64_t B, int64_t dk, bool bf16, int32_t R, hipStream_t st);
int diag_varlen_launch(const DiagParams& p, int64_t dk, bool bf16, int32_t R, hipStream_t st);
int64_t varlen_main_grid(int64_t items, int64_t H, int64_t dv);
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

/*
 * kdnscan.h -- C ABI of libkdnscan: precision-tracking associative-memory
 * scans on AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (page title, section):
 *   [Palimpsa] "Learning to Remember, Learn, and Forget in Attention-Based
 *              Models" (technical summary), Metodologia 1: forget gate
 *              alpha_t = exp(-A d_t); Metodologia 2: the diagonal precision
 *              ("importance") update of I_t and the precision-weighted mean
 *              update of mu_t.
 *   [KLA]      "Riassunto Tecnico: Kalman Linear Attention (KLA)",
 *              Metodologia 1: OU decay and process noise, observation
 *              precision, read-out of the posterior mean by the query;
 *              Metodologia 2: the precision update is a Mobius
 *              (fractional-linear) map, composed by an associative prefix
 *              scan, and the mean update is affine once precisions are known;
 *              Metodologia 3: forget and write gates from precision ratios.
 *   [KDN]      "Kalman Delta Networks" abstract: Diagonal and Isotropic KDN,
 *              Mobius uncertainty recurrences, constant-memory decoding.
 *
 * Conventions shared by every entry point
 *   - All tensors are contiguous, row-major, and live in device memory
 *     (hipMalloc'd or torch CUDA tensors); the caller owns every buffer.
 *     Scalars and workspace_bytes are host values.
 *   - The memory state of one head is a d_k x d_v matrix: entry [j][i]
 *     couples key channel j with value channel i.  Read-out:
 *     o_t[i] = sum_j q_t[j] mu_t[j][i], taken after token t's update.
 *   - Calls enqueue kernels on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and return without synchronising.  The
 *     library never allocates device memory (the packed-batch gradient keeps
 *     one extra stream and two events per device, see there).
 *   - Arguments are validated before any HIP call; a rejected call touches
 *     no memory.  Return values: KDN_OK or a negative KDN_E* code (see
 *     kdn_status_string).  Values inside tensors are not checked: they are
 *     preconditions (A > 0, d >= 0, beta >= 0, I0 > 0, a > 0, p >= 0,
 *     Lambda >= 0, lambda0 > 0).  Under them every precision stays > 0.
 *   - Supported head sizes: d_k, d_v in {16, 32, 64, 128}; other values
 *     return KDN_EUNSUPPORTED.  Every pointer must be 16-byte aligned.
 *   - Size limits (KDN_EINVAL beyond them): T (or total_T) < 2^31; every
 *     element count B*H*T*d < 2^62; and one workgroup per head (or per head
 *     and column tile, segment or 4096-token block, whichever the call
 *     launches) must leave the grid within 2^32 - 1 work-items at 512
 *     threads per workgroup, about 8.4 million such units.
 *
 * Workspace protocol (entry points that take one)
 *   - workspace == NULL and workspace_bytes != NULL: write the number of
 *     bytes needed to *workspace_bytes and return KDN_OK without launching.
 *   - otherwise the call runs; if it needs workspace and workspace is NULL
 *     or *workspace_bytes is smaller than needed, it returns KDN_EWORKSPACE
 *     (writing the needed size when workspace_bytes != NULL).
 */
#ifndef KDNSCAN_H
#define KDNSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDN_F32 = 0, KDN_BF16 = 1 } kdn_dtype;

enum {
    KDN_OK = 0,
    KDN_EINVAL = -1,        /* bad size, NULL required pointer, misalignment, I_prior <= 0 */
    KDN_EUNSUPPORTED = -2,  /* valid but not implemented (head size outside the list) */
    KDN_EWORKSPACE = -3,    /* workspace missing or too small */
    KDN_EHIP = -4,          /* a HIP launch failed */
    KDN_ESCRATCH = -5       /* the call needs more than the fixed scratch of the no-allocation entry holds */
};

/*
 * Diagonal-precision scan, forward [Palimpsa Metodologia 1-2; KLA Metodologia 1].
 * For every head (b, h) and token t = 0..T-1, with every entry [j][i]:
 *   alpha_t = exp(-A[h] d_t)
 *   I_t  = alpha_t I_{t-1} + (1 - alpha_t) I_prior + beta_t[i] k_t[j]^2
 *   mu_t = alpha_t (I_{t-1} / I_t) mu_{t-1} + beta_t[i] v_t[i] k_t[j] / I_t
 *   o_t[i] = sum_j q_t[j] mu_t[j][i]
 * Inputs (in_dtype: KDN_F32 = float, KDN_BF16 = bfloat16):
 *   q, k [B,H,T,d_k];  v, beta [B,H,T,d_v];  d [B,H,T].
 *   beta == NULL selects Palimpsa-M gating [Palimpsa Metodologia 3]: the
 *   step gate d_t is also the input gate, beta_t[i] = d_t for every i.
 *   A [H] float (forget rate per head);  I_prior > 0 (scalar prior precision).
 *   I0, mu0 [B,H,d_k,d_v] float: starting state; NULL -> I_prior and 0.
 * Outputs (float): o [B,H,T,d_v]; I_T, mu_T [B,H,d_k,d_v] final state, or
 *   NULL to skip.  I_T may alias I0 and mu_T may alias mu0 (continuation);
 *   no other aliasing between inputs and outputs is allowed.
 * Workspace: always needed when B*H*T > 0: 16 bytes of per-token frame
 * scalars per (head, token), plus, when the plan splits long sequences into
 * segments (whose composites are carried in order), the segment composites
 * and carry-in states.  Query its size first.
 */
int kdn_diag_scan_fwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                      kdn_dtype in_dtype,
                      const void* q, const void* k, const void* v,
                      const void* beta, const void* d,
                      const float* A, float I_prior,
                      const float* I0, const float* mu0,
                      float* o, float* I_T, float* mu_T,
                      void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Diagonal-precision scan over a packed variable-length batch: the same
 * recurrence as kdn_diag_scan_fwd, restarted at every sequence start
 * [Palimpsa Metodologia 1-3; Palimpsa-M gating with beta == NULL].
 *   cu_seqlens: DEVICE int64 [N+1], cu[0] = 0 <= cu[1] <= ... <= cu[N] =
 *     total_T; sequence s owns packed tokens [cu[s], cu[s+1]) (empty
 *     sequences allowed).  Offsets outside [0, total_T] are clamped (the
 *     kernels never leave the buffers), but then the results are undefined.
 *   q, k [H,total_T,d_k]; v, beta [H,total_T,d_v]; d [H,total_T] (in_dtype;
 *     beta may be NULL); A [H] float; I_prior > 0.
 *   I0, mu0 [N,H,d_k,d_v] float or NULL: each sequence's starting state.
 *   Outputs: o [H,total_T,d_v]; I_T, mu_T [N,H,d_k,d_v] or NULL.
 *   Workspace: 16 bytes per (head, packed token) of frame scalars, the plan
 *   (a few int32 per sequence and per segment), and for split sequences the
 *   carried states and sub-segment composites (kdn_diag_varlen_plan).
 * Work plan: chunks of 16 tokens aligned to each sequence start.  A
 * sequence longer than its fair share of the chip (kdn_diag_varlen_plan) is
 * cut into segments of seg_tokens tokens [KLA Metodologia 2: associative
 * composition]: the segments' composites are built on the matrix cores and
 * carried in order, so every segment runs from its true starting state.
 * The main pass runs one workgroup per (segment, head, column tile: 64
 * columns, or 32 / d_v columns when d_v < 64), sequences longest first (the
 * order and the tables are computed on the device from cu_seqlens; up to
 * 16384 sequences, beyond that in index order), a sequence's segments in
 * token order.  Results agree with the unsplit scan up to rounding.
 */
int kdn_diag_scan_varlen_fwd(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                             kdn_dtype in_dtype, const int64_t* cu_seqlens,
                             const void* q, const void* k, const void* v,
                             const void* beta, const void* d,
                             const float* A, float I_prior,
                             const float* I0, const float* mu0,
                             float* o, float* I_T, float* mu_T,
                             void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Diagonal KDN with process noise, forward [KDN abstract, Diagonal KDN:
 * one-step posteriors projected onto diagonal Gaussians by mean-field VI,
 * residual writes weighted by the Kalman gain; predict step KLA
 * Metodologia 1].  Memory column i of head (b, h) is a latent vector
 * observed through v_t[i] = k_t^T s_i + noise of precision beta_t[i]; each
 * entry [j][i] keeps a mean and a precision lambda.  Per token:
 *   predict  variance 1/lambda -> a_t^2/lambda + p_t (= sp),  mean -> a_t mu
 *   update   mu[j][i] += sp k_j (v_i - sum_l k_l mu[l][i]) / (sum_l k_l^2 sp_l + 1/beta_i)
 *            lambda[j][i] = 1/sp + beta_i k_j^2
 *   read     o_t[i] = sum_j q_t[j] mu_t[j][i]
 * so lambda follows the Mobius map l -> ((1 + w p) l + w a^2) / (p l + a^2),
 * w = beta k^2.
 * Inputs: q, k [B,H,T,d_k]; v, beta [B,H,T,d_v] (in_dtype); a, p [B,H,T]
 *   float (decay, process-noise variance); lambda0, mu0 [B,H,d_k,d_v] float
 *   or NULL (-> 1 and 0).
 * Outputs (float): o [B,H,T,d_v]; lambda_T, mu_T [B,H,d_k,d_v] or NULL.
 *   No workspace: each head's sequence runs in one workgroup pass.
 */
int kdn_diag_noise_scan_fwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                            kdn_dtype in_dtype,
                            const void* q, const void* k, const void* v, const void* beta,
                            const float* a, const float* p,
                            const float* lambda0, const float* mu0,
                            float* o, float* lambda_T, float* mu_T, void* stream);

/*
 * Gradient of kdn_diag_scan_fwd (reverse mode).  The pages train with these
 * layers [Palimpsa summary, Metodologia 3; KDN abstract, pretraining] but
 * print no gradient: this is the exact adjoint of the recurrence above, in
 * fp32.  For the scalar loss
 *   L = sum d_o * o + sum d_I_T * I_T + sum d_mu_T * mu_T
 * it writes (float, all outputs overwritten, none accumulated into):
 *   dq, dk [B,H,T,d_k];  dv, dbeta [B,H,T,d_v];  dd [B,H,T];
 *   dA [H] (summed over the batch);  dI_prior [1] or NULL;
 *   dI0, dmu0 [B,H,d_k,d_v] or NULL (allowed only when I0 / mu0 are given;
 *   with I0 == NULL the start I_prior's share goes to dI_prior).
 *   With beta == NULL (Palimpsa-M gating, beta_t[i] = d_t) dbeta must be
 *   NULL and dd includes the input-gate share sum_i dL/dbeta_t[i].
 * Inputs: those of the forward call (same dtype rules), plus d_o [B,H,T,d_v]
 *   float (required), d_I_T, d_mu_T [B,H,d_k,d_v] float or NULL (= 0).
 * Supported: d_k in {64, 128}, d_v in {16, 32, 64, 128} (else
 *   KDN_EUNSUPPORTED).  The forward pass is recomputed from checkpoints the
 *   call writes into its workspace (8 bytes per state entry per 16 tokens,
 *   plus per-token partial sums); query its size as for the forward call.
 *   Outputs must not alias inputs.  Deterministic: no atomics.
 * Rows too few to fill the chip are cut into the forward plan's segments
 * (kdn_diag_plan) [KLA Metodologia 2]: the forward composites give every
 * segment its starting state; the adjoint recurrence, linear as well, is
 * composed per segment while the checkpoints are written and carried from
 * the row's end, so every segment's reverse pass runs at once.
 */
int kdn_diag_scan_bwd(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                      kdn_dtype in_dtype,
                      const void* q, const void* k, const void* v,
                      const void* beta, const void* d,
                      const float* A, float I_prior,
                      const float* I0, const float* mu0,
                      const float* d_o, const float* d_I_T, const float* d_mu_T,
                      float* dq, float* dk, float* dv, float* dbeta, float* dd,
                      float* dA, float* dI_prior, float* dI0, float* dmu0,
                      void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Gradient of kdn_diag_scan_varlen_fwd (reverse mode) over a packed batch of
 * N variable-length sequences [Palimpsa Metodologia 3, Palimpsa-M training
 * on packed sequences], the exact adjoint of the same recurrence per
 * (sequence, head), in fp32.  For the scalar loss
 *   L = sum d_o * o + sum d_I_T * I_T + sum d_mu_T * mu_T
 * it writes (float, overwritten):
 *   dq, dk [H,total_T,d_k];  dv, dbeta [H,total_T,d_v];  dd [H,total_T];
 *   dA [H] (summed over every sequence);  dI_prior [1] or NULL;
 *   dI0, dmu0 [N,H,d_k,d_v] or NULL (allowed only when I0 / mu0 are given).
 * Inputs: those of kdn_diag_scan_varlen_fwd (cu_seqlens int64 [N+1] on the
 *   device, q, k [H,total_T,d_k], v, beta [H,total_T,d_v], d [H,total_T],
 *   I0, mu0 [N,H,d_k,d_v] or NULL), plus d_o [H,total_T,d_v] float
 *   (required when N*H*total_T > 0), d_I_T, d_mu_T [N,H,d_k,d_v] float or NULL.
 *   beta == NULL is Palimpsa-M gating (dbeta must then be NULL).
 * Supported: d_k in {64, 128}, d_v in {16, 32, 64, 128}.  Each sequence runs
 *   from its own starting state, its chunks aligned to its first token; runs
 *   are dispatched longest sequence first.  Workspace as for the other calls
 *   (query with workspace == NULL): frame scalars, the plan, checkpoints
 *   (8 bytes per state entry per 16 tokens of each sequence, plus one final
 *   state per sequence) and per-token partial sums.  Deterministic.
 * Streams: where the batch can hold sequences longer than a fair share of
 *   the chip, the whole sequences' checkpoint pass runs on a second stream
 *   of the current device, forked from `stream` and joined back before the
 *   reverse pass; all later work is ordered on `stream` as usual.  That
 *   stream and its two events are created on the first such call on a device
 *   (default priority) and kept until the process ends.  A `stream` under
 *   graph capture does not fork.  The current device must be the device of
 *   `stream`.
 */
int kdn_diag_scan_varlen_bwd(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                             kdn_dtype in_dtype, const int64_t* cu_seqlens,
                             const void* q, const void* k, const void* v,
                             const void* beta, const void* d,
                             const float* A, float I_prior,
                             const float* I0, const float* mu0,
                             const float* d_o, const float* d_I_T, const float* d_mu_T,
                             float* dq, float* dk, float* dv, float* dbeta, float* dd,
                             float* dA, float* dI_prior, float* dI0, float* dmu0,
                             void* workspace, size_t* workspace_bytes, void* stream);

/*
 * Isotropic scalar-precision filter [KDN abstract, Isotropic KDN;
 * KLA Metodologia 1-3].  Per head, per token:
 *   lambda_t = M_t(lambda_{t-1}),  M_t = [[1 + Lambda_t p_t, Lambda_t a_t^2],
 *                                         [p_t,              a_t^2          ]]
 *   acting as l -> (m11 l + m12) / (m21 l + m22): predict (the mean decays
 *   by a_t, process noise p_t) then add observation precision Lambda_t.
 *   The maps are composed by an associative prefix scan.  Then the gates
 *   lambda^-_t = lambda_{t-1} / (a_t^2 + p_t lambda_{t-1}),
 *   F_t = a_t lambda^-_t / lambda_t,  G_t = Lambda_t / lambda_t
 *   drive the affine mean scan mu_t = F_t mu_{t-1} + G_t k_t v_t^T with
 *   read-out o_t[i] = sum_j q_t[j] mu_t[j][i].
 * Inputs (float): a, p, Lambda [B,H,T]; lambda0 [B,H] or NULL (-> 1).
 *   d_k == 0 && d_v == 0 runs the precision path only (q, k, v, mu0, o,
 *   mu_T ignored).  Otherwise q, k [B,H,T,d_k], v [B,H,T,d_v]; mu0
 *   [B,H,d_k,d_v] or NULL (-> 0).
 * Outputs (float): lambda_out [B,H,T] or NULL; o [B,H,T,d_v] (required for
 *   the mean path); mu_T [B,H,d_k,d_v] or NULL.
 * Workspace: per-block Mobius composites, the gates and per-chunk mean
 *   composites.
 */
int kdn_mobius_precision_scan(int64_t B, int64_t H, int64_t T,
                              const float* a, const float* p, const float* Lambda,
                              const float* lambda0, float* lambda_out,
                              int64_t d_k, int64_t d_v,
                              const float* q, const float* k, const float* v,
                              const float* mu0, float* o, float* mu_T,
                              void* workspace, size_t* workspace_bytes, void* stream);

/*
 * One-token decode of the diagonal recurrence [Palimpsa Metodologia 1-2;
 * constant-memory decoding, KDN abstract].  The same update as
 * kdn_diag_scan_fwd for a single token, applied in place:
 *   q, k [B,H,d_k]; v, beta [B,H,d_v]; d [B,H] (in_dtype);  A [H] float;
 *   beta == NULL: Palimpsa-M gating (beta[i] = d), as for the scan;
 *   I, mu [B,H,d_k,d_v] float, read and overwritten with the new state;
 *   o [B,H,d_v] float.
 */
int kdn_decode_step(int64_t B, int64_t H, int64_t d_k, int64_t d_v, kdn_dtype in_dtype,
                    const void* q, const void* k, const void* v,
                    const void* beta, const void* d,
                    const float* A, float I_prior,
                    float* I, float* mu, float* o, void* stream);

/*
 * Plan of a diagonal scan (host only, no HIP call): the token chunk length
 * staged per step, the number of sequence segments S, the number of
 * sub-segments R each composite segment is cut into, and the segment token
 * bounds seg_bounds[0..S] (seg_bounds may be NULL; it must hold S+1 entries
 * when given, S <= max_segments).  `segments` is the request of the call
 * being planned: 0 for the automatic choice, n >= 1 for n segments (clamped
 * to [1, min(64, number of chunks)]), as in kdn_scan_opts.  Segment s owns
 * whole chunks [floor(s n / S), floor((s+1) n / S)) of the n = ceil(T / chunk)
 * chunks; sub-segment r of segment s owns the segment's chunks
 * [c0 + floor(r m / R), c0 + floor((r+1) m / R)), m the segment's chunk count.
 */
int kdn_diag_plan(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v, int32_t segments,
                  int32_t* chunk, int32_t* segments_out, int32_t* subsegments,
                  int64_t* seg_bounds, int32_t max_segments);

/*
 * Options of the extended entry points below.  A zero-initialised struct (or
 * a NULL pointer) gives exactly the behaviour of the plain entry point.
 *   segments: 0 = automatic plan; n >= 1 = cut each sequence into n segments
 *     (clamped as in kdn_diag_plan; the isotropic mean scan clamps to its own
 *     chunk count).  Results agree with any segmenting up to rounding.
 *   bounds_echo / echo_capacity: a device buffer of echo_capacity int64
 *     words, or NULL.  When given, every workgroup (or one-wave work unit)
 *     of the scan writes one record of KDN_ECHO_WORDS words holding the token
 *     bounds it actually used: {kind, run, segment, part, t_begin, t_end,
 *     sequence, 0}, kind 1 = main pass (run = b*H + h, part = column tile),
 *     2 = diagonal segment composite (part = sub-segment), 3 = isotropic mean
 *     scan (part = column tile), 4 = isotropic segment composite; for a
 *     packed batch run = s*H + h of sequence s = `sequence`.  Kind 2 records
 *     hold the wave's tile in the `sequence` word (bf16 inputs: its index
 *     among the unit's waves, those summing J first, then those summing
 *     eta) and, for a packed batch,
 *     the sequence in the last word (0 otherwise).  Record r of
 *     kind k sits at a fixed slot; records that would pass echo_capacity are
 *     dropped; slots of work units with nothing to do stay untouched (clear
 *     the buffer first).  For testing the integer bookkeeping.
 *   main_begin / main_end: hipEvent_t handles, or NULL.  Each given event is
 *     recorded on the call's stream right before (main_begin) and right after
 *     (main_end) the call's main pass, the kernel that reads every token and
 *     writes o, so a caller can time that kernel apart from the frame-scalar
 *     and segment-composite passes around it.  Not recorded when the call has
 *     no main pass (B*H == 0 or T == 0); a failed record returns KDN_EHIP.
 *   echo_words (out): the words the call's records span (written on every
 *     call, queries included).
 */
#define KDN_ECHO_WORDS 8
typedef struct kdn_scan_opts {
    int32_t segments;
    int32_t reserved;
    int64_t* bounds_echo;
    int64_t echo_capacity;
    int64_t echo_words;
    void* main_begin;
    void* main_end;
} kdn_scan_opts;

/*
 * Plan of a packed batch's forward scan (kdn_diag_scan_varlen_fwd[_ex]),
 * computed on the host from the sizes alone.  segments: 0 (automatic) or 1
 * (no split).  seg_tokens: the segment length (a multiple of 256) of a
 * split sequence, or 0 when no sequence can be split; a sequence of len >
 * seg_tokens tokens runs as ceil(len / seg_tokens) segments, segment g
 * holding its tokens [g seg_tokens, min((g + 1) seg_tokens, len)).  It is
 * the fair share ceil(H total_T tiles / 256) tokens (tiles = d_v / 64, or 1
 * when d_v < 64) rounded up to a multiple of 256, at least 512.
 * max_items, max_composites: capacities of the plan's tables (N plus
 * total_T / seg_tokens, and total_T / seg_tokens).  subsegments: R, the
 * composite storage holds max_composites x H x R sub-segment composites.
 * The composite of each segment but a sequence's last is built in
 * R' = min(seg_tokens / 64, floor(max_composites R / C)) sub-segments, C the
 * number of such segments in the batch (known on the device only),
 * sub-segment r holding the segment's 16-token chunks
 * [floor(r m / R'), floor((r + 1) m / R')), m = seg_tokens / 16.  Any output
 * may be NULL.
 */
int kdn_diag_varlen_plan(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                         int32_t segments, int64_t* seg_tokens, int32_t* subsegments,
                         int64_t* max_items, int64_t* max_composites);

/* kdn_diag_scan_bwd with options (opts may be NULL): only `segments` applies
 * (0: the automatic plan, n >= 1: n segments per row, clamped as in
 * kdn_diag_plan); bounds_echo, main_begin and main_end must be NULL. */
int kdn_diag_scan_bwd_ex(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                         kdn_dtype in_dtype,
                         const void* q, const void* k, const void* v,
                         const void* beta, const void* d,
                         const float* A, float I_prior,
                         const float* I0, const float* mu0,
                         const float* d_o, const float* d_I_T, const float* d_mu_T,
                         float* dq, float* dk, float* dv, float* dbeta, float* dd,
                         float* dA, float* dI_prior, float* dI0, float* dmu0, kdn_scan_opts* opts,
                         void* workspace, size_t* workspace_bytes, void* stream);

/* kdn_diag_scan_fwd with options (opts may be NULL). */
int kdn_diag_scan_fwd_ex(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                         kdn_dtype in_dtype,
                         const void* q, const void* k, const void* v,
                         const void* beta, const void* d,
                         const float* A, float I_prior,
                         const float* I0, const float* mu0,
                         float* o, float* I_T, float* mu_T, kdn_scan_opts* opts,
                         void* workspace, size_t* workspace_bytes, void* stream);

/* kdn_diag_scan_varlen_fwd with options (opts may be NULL; segments must be
 * 0, the automatic plan of kdn_diag_varlen_plan, or 1: every sequence in one
 * segment, however long). */
int kdn_diag_scan_varlen_fwd_ex(int64_t N, int64_t H, int64_t total_T, int64_t d_k, int64_t d_v,
                                kdn_dtype in_dtype, const int64_t* cu_seqlens,
                                const void* q, const void* k, const void* v,
                                const void* beta, const void* d,
                                const float* A, float I_prior,
                                const float* I0, const float* mu0,
                                float* o, float* I_T, float* mu_T, kdn_scan_opts* opts,
                                void* workspace, size_t* workspace_bytes, void* stream);

/* kdn_mobius_precision_scan with options (opts may be NULL; segments applies
 * to the gated mean scan). */
int kdn_mobius_precision_scan_ex(int64_t B, int64_t H, int64_t T,
                                 const float* a, const float* p, const float* Lambda,
                                 const float* lambda0, float* lambda_out,
                                 int64_t d_k, int64_t d_v,
                                 const float* q, const float* k, const float* v,
                                 const float* mu0, float* o, float* mu_T, kdn_scan_opts* opts,
                                 void* workspace, size_t* workspace_bytes, void* stream);

/*
 * kdn_diag_scan_fwd for callers that cannot allocate device memory: code
 * under stream capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and rules as kdn_diag_scan_fwd minus the
 * workspace: the call uses a fixed scratch array of
 * KDN_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, reserved when the
 * library is loaded and held until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree) and its result is the same as the plain
 * call's; where the plain call's plan would need more scratch than the array
 * holds, the composite segments are cut into fewer sub-segments (same
 * results up to rounding), and if even that does not fit it returns
 * KDN_ESCRATCH.  (Roughly: 16 bytes per head-token of frame scalars, plus,
 * for segmented long sequences, 8 d_k d_v bytes per head and segment.)
 * The current device must be the device of `stream`.  Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents: calls that
 * overlap on one GPU (other streams, other threads) race and must be ordered
 * by the caller.
 */
#define KDN_NOALLOC_SCRATCH_BYTES (64u << 20)
int kdn_diag_scan_fwd_noalloc(int64_t B, int64_t H, int64_t T, int64_t d_k, int64_t d_v,
                              kdn_dtype in_dtype,
                              const void* q, const void* k, const void* v,
                              const void* beta, const void* d,
                              const float* A, float I_prior,
                              const float* I0, const float* mu0,
                              float* o, float* I_T, float* mu_T, void* stream);

/* Human-readable text of a status code; never NULL. */
const char* kdn_status_string(int status);

/* Text of the HIP error behind the calling thread's last KDN_EHIP (or "no
 * error"); never NULL.  Diagnostic only. */
const char* kdn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KDNSCAN_H */

// diag_bwd_seg.hip -- gradient of rows cut into segments: the kernels of
// diag_bwd_kernels.h with segment starting states and adjoint composites,
// and the carry of the adjoint between segments.
#include "diag_bwd_kernels.h"

namespace kdn {

// Rows cut into segments: the adjoint flowing into each segment's end,
// from the row's end backwards, lam(s - 1) = B_s + G_s lam(s) (one thread
// per element of a (row, tile) slot).
__global__ __launch_bounds__(256) void k_bwd_adj_carry(BwdParams p, int64_t slot, int64_t n_total,
                                                       int32_t ntile) {
    const int S = p.S;
    for (int64_t e = elem_first(); e < n_total; e += elem_stride()) {
        const int64_t rt = e / slot;
        const int64_t x = e % slot;
        const int64_t bh = rt / ntile;
        float lam = p.lam[(rt * S + S - 1) * slot + x];
        for (int s = S - 1; s >= 1; --s) {
            lam = fmaf(p.adjg[bh * S + s], lam, p.adj[(rt * S + s) * slot + x]);
            p.lam[(rt * S + s - 1) * slot + x] = lam;
        }
    }
}

// ---------------------------------------------------------------------------
// Reverse pass.
// ---------------------------------------------------------------------------
// A packed batch whose long sequences run in segments: the same chain per
// split sequence, over its consecutive items (seq_item), from its last
// segment back (one thread per element of a (sequence, head, tile) slot).
__global__ __launch_bounds__(256) void k_bwd_adj_carry_varlen(BwdParams p, int64_t slot, int64_t n_total,
                                                              int32_t ntile) {
    const int64_t per_seq = p.H * ntile * slot;
    const int64_t nsplit = p.nwork[2];
    for (int64_t e = elem_first(); e < n_total; e += elem_stride()) {
        const int64_t k = e / per_seq;
        if (k >= nsplit) break;   // e only grows
        const int64_t ht = e % per_seq / slot;   // head * ntile + tile
        const int64_t x = e % slot;
        const int32_t sq = p.split_seq[k];
        const int32_t fi = p.seq_item[sq];
        if (fi < 0) continue;
        int64_t a = p.cu_seqlens[sq], b = p.cu_seqlens[sq + 1];
        a = a < 0 ? 0 : (a > p.T ? p.T : a);
        b = b < a ? a : (b > p.T ? p.T : b);
        int64_t nseg = b - a > p.vl_thr ? (b - a + p.vl_seg - 1) / p.vl_seg : 1;
        if (fi + nseg > p.vl_items) nseg = p.vl_items - fi;
        const int64_t h = ht / ntile;
        auto at = [&](int64_t item) { return (item * p.H) * ntile + ht; };
        float lam = p.lam[at(fi + nseg - 1) * slot + x];
        for (int64_t g = nseg - 1; g >= 1; --g) {
            const int64_t item = fi + g;
            lam = fmaf(p.adjg[item * p.H + h], lam, p.adj[at(item) * slot + x]);
            p.lam[at(item - 1) * slot + x] = lam;
        }
    }
}

// One workgroup per (row, segment, column tile) or (item, head, tile):
// checkpoints and adjoint composites, the adjoint carry, then the reverse
// pass.
template <int DK, int DV, bool BF16>
static int launch_seg_shape(const BwdParams& p, hipStream_t st, hipEvent_t join) {
    using Sh = BwdShape<DK, DV>;
    const int64_t g = p.cu_seqlens ? (p.vl_items * p.H + 7) / 8 * 8 * Sh::NTILE
                                   : p.BH * p.S * Sh::NTILE;
    if (g == 0) return KDN_OK;
    const dim3 grid(static_cast<uint32_t>(g));
    // A packed batch: the split sequences rank before every whole one (they
    // are the longer ones), so their items are the plan's first, at most two
    // per composite segment; the checkpoint pass with adjoint composites
    // needs no more (past kMaxPlanSort sequences the order is the index
    // order and the grid covers every item).
    int64_t gc = g;
    if (p.cu_seqlens && p.nseq <= kMaxPlanSort) {
        const int64_t split_items = 2 * p.vl_comps < p.vl_items ? 2 * p.vl_comps : p.vl_items;
        gc = (split_items * p.H + 7) / 8 * 8 * Sh::NTILE;
    }
    if (gc > 0) hipLaunchKernelGGL((k_diag_bwd_ckpt<DK, DV, BF16, true>), dim3(static_cast<uint32_t>(gc)),
                                   dim3(Sh::NTH), 0, st, p);
    const int64_t slot = 2 * Sh::BLK;
    if (p.cu_seqlens) {
        if (p.vl_comps > 0) {
            const int64_t n = p.vl_comps * p.H * Sh::NTILE * slot;
            const int64_t groups = elem_groups(n) < 1024 ? elem_groups(n) : 1024;
            hipLaunchKernelGGL(k_bwd_adj_carry_varlen, dim3(static_cast<uint32_t>(groups)), dim3(256), 0, st, p,
                               slot, n, static_cast<int32_t>(Sh::NTILE));
        }
    } else {
        const int64_t n = p.BH * Sh::NTILE * slot;
        hipLaunchKernelGGL(k_bwd_adj_carry, dim3(elem_groups(n)), dim3(256), 0, st, p, slot, n,
                           static_cast<int32_t>(Sh::NTILE));
    }
    if (join != nullptr) {
        const hipError_t e = hipStreamWaitEvent(st, join, 0);
        if (e != hipSuccess) {
            note_hip_error(e);
            return KDN_EHIP;
        }
    }
    hipLaunchKernelGGL((k_diag_bwd<DK, DV, BF16, true>), grid, dim3(Sh::NTH), 0, st, p);
    return launch_status();
}

template <int DK, bool BF16>
static int launch_seg_dv(const BwdParams& p, hipStream_t st, hipEvent_t join) {
    switch (p.dv) {
        case 16: return launch_seg_shape<DK, 16, BF16>(p, st, join);
        case 32: return launch_seg_shape<DK, 32, BF16>(p, st, join);
        case 64: return launch_seg_shape<DK, 64, BF16>(p, st, join);
        case 128: return launch_seg_shape<DK, 128, BF16>(p, st, join);
        default: return KDN_EUNSUPPORTED;
    }
}

int diag_bwd_seg_launch(const BwdParams& p, int64_t dk, bool bf16, hipStream_t st, hipEvent_t join) {
    if (dk == 64) return bf16 ? launch_seg_dv<64, true>(p, st, join) : launch_seg_dv<64, false>(p, st, join);
    return bf16 ? launch_seg_dv<128, true>(p, st, join) : launch_seg_dv<128, false>(p, st, join);
}

}  // namespace kdn

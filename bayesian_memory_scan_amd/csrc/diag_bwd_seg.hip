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
// One workgroup per (row, segment, column tile): checkpoints and adjoint
// composites, the adjoint carry, then the reverse pass.
template <int DK, int DV, bool BF16>
static int launch_seg_shape(const BwdParams& p, hipStream_t st) {
    using Sh = BwdShape<DK, DV>;
    const int64_t g = p.BH * p.S * Sh::NTILE;
    if (g == 0) return KDN_OK;
    const dim3 grid(static_cast<uint32_t>(g));
    hipLaunchKernelGGL((k_diag_bwd_ckpt<DK, DV, BF16, true>), grid, dim3(Sh::NTH), 0, st, p);
    const int64_t slot = 2 * Sh::BLK;
    const int64_t n = p.BH * Sh::NTILE * slot;
    hipLaunchKernelGGL(k_bwd_adj_carry, dim3(elem_groups(n)), dim3(256), 0, st, p, slot, n,
                       static_cast<int32_t>(Sh::NTILE));
    hipLaunchKernelGGL((k_diag_bwd<DK, DV, BF16, true>), grid, dim3(Sh::NTH), 0, st, p);
    return launch_status();
}

template <int DK, bool BF16>
static int launch_seg_dv(const BwdParams& p, hipStream_t st) {
    switch (p.dv) {
        case 16: return launch_seg_shape<DK, 16, BF16>(p, st);
        case 32: return launch_seg_shape<DK, 32, BF16>(p, st);
        case 64: return launch_seg_shape<DK, 64, BF16>(p, st);
        case 128: return launch_seg_shape<DK, 128, BF16>(p, st);
        default: return KDN_EUNSUPPORTED;
    }
}

int diag_bwd_seg_launch(const BwdParams& p, int64_t dk, bool bf16, hipStream_t st) {
    if (dk == 64) return bf16 ? launch_seg_dv<64, true>(p, st) : launch_seg_dv<64, false>(p, st);
    return bf16 ? launch_seg_dv<128, true>(p, st) : launch_seg_dv<128, false>(p, st);
}

}  // namespace kdn

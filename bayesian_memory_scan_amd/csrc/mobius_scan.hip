// mobius_scan.hip -- scalar-precision (isotropic) filter as a Mobius scan.
//
// Per head the posterior precision follows lambda_t = M_t(lambda_{t-1}) with
// the fractional-linear map (KLA, "Riassunto Tecnico: Kalman Linear
// Attention", Metodologia 2; Isotropic KDN, "Kalman Delta Networks" abstract)
//   M_t = [[1 + Lambda_t p_t, Lambda_t a_t^2], [p_t, a_t^2]],
//   l -> (m11 l + m12) / (m21 l + m22),
// i.e. predict (mean decays by a_t, process noise p_t: variance a_t^2/l + p_t)
// then add the observation precision Lambda_t.  Maps compose by 2x2 matrix
// products with the later map on the left; the product is associative, which
// is what makes an O(log T)-depth prefix scan possible.  All entries are
// positive for a > 0, p >= 0, Lambda >= 0, so applying a composite to
// lambda_0 > 0 involves no cancellation; composites are kept in range by
// exact power-of-two rescaling (a fractional-linear map is unchanged by a
// common factor).
//
// Two launches:
//   k_mob_reduce: per (head, block of 4096 tokens) the block's composite;
//   k_mob_apply:  per (head, block) the carry-in (ordered product of earlier
//                 block composites), the in-block exclusive scan of
//                 per-thread composites (DPP-free: __shfl_up within the wave,
//                 LDS across the 4 waves), then each thread walks its 16
//                 tokens sequentially from its starting precision and writes
//                 lambda_t and the gates of KLA Metodologia 3:
//                   lambda^-_t = lambda_{t-1} / (a_t^2 + p_t lambda_{t-1})
//                   F_t = a_t lambda^-_t / lambda_t,   G_t = Lambda_t / lambda_t.
#include "kdn_params.h"

namespace kdn {

constexpr int kMobThreads = 256;
constexpr int kMobPer = 16;
constexpr int kMobBlock = kMobThreads * kMobPer;

struct Mob {
    float m11, m12, m21, m22;
};

__device__ __forceinline__ Mob mob_identity() { return {1.0f, 0.0f, 0.0f, 1.0f}; }

// Later map L after earlier map E: the matrix product L * E.
__device__ __forceinline__ Mob mob_after(const Mob& L, const Mob& E) {
    return {__builtin_fmaf(L.m11, E.m11, L.m12 * E.m21), __builtin_fmaf(L.m11, E.m12, L.m12 * E.m22),
            __builtin_fmaf(L.m21, E.m11, L.m22 * E.m21), __builtin_fmaf(L.m21, E.m12, L.m22 * E.m22)};
}

// Scale by 2^-e so the largest entry lies in [0.5, 1): exact, map unchanged.
__device__ __forceinline__ Mob mob_norm(const Mob& M) {
    const float mx = fmaxf(fmaxf(M.m11, M.m12), fmaxf(M.m21, M.m22));
    if (!(mx > 0.0f) || !(mx < INFINITY)) return M;
    const int e = __builtin_amdgcn_frexp_expf(mx);
    return {ldexpf(M.m11, -e), ldexpf(M.m12, -e), ldexpf(M.m21, -e), ldexpf(M.m22, -e)};
}

__device__ __forceinline__ Mob mob_step(float a, float p, float L) {
    const float a2 = a * a;
    return {__builtin_fmaf(L, p, 1.0f), L * a2, p, a2};
}

__device__ __forceinline__ float mob_apply(const Mob& M, float l) {
    return __builtin_fmaf(M.m11, l, M.m12) / __builtin_fmaf(M.m21, l, M.m22);
}

__device__ __forceinline__ Mob mob_shfl_up(const Mob& M, int s) {
    return {__shfl_up(M.m11, s), __shfl_up(M.m12, s), __shfl_up(M.m21, s), __shfl_up(M.m22, s)};
}


// Composite of this thread's (up to) 16 consecutive tokens.
__device__ __forceinline__ Mob thread_composite(const MobParams& p, int64_t bh, int64_t t0) {
    Mob P = mob_identity();
    const float* a = p.a + bh * p.T;
    const float* pp = p.p + bh * p.T;
    const float* L = p.Lam + bh * p.T;
#pragma unroll
    for (int u = 0; u < kMobPer; ++u) {
        const int64_t t = t0 + u;
        if (t < p.T) P = mob_after(mob_step(a[t], pp[t], L[t]), P);
        if ((u & 3) == 3) P = mob_norm(P);
    }
    return P;
}

// Inclusive scan over the workgroup's 256 thread composites (thread order =
// token order).  Returns the inclusive prefix; *excl receives the exclusive one.
__device__ Mob block_scan(Mob P, Mob* excl, Mob (&s_w)[kMobThreads / kWave]) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        const Mob Q = mob_shfl_up(P, s);
        if (lane >= s) P = mob_norm(mob_after(P, Q));
    }
    Mob ex = mob_shfl_up(P, 1);
    if (lane == 0) ex = mob_identity();
    if (lane == kWave - 1) s_w[wave] = P;
    __syncthreads();
    Mob before = mob_identity();
    for (int w = 0; w < wave; ++w) before = mob_norm(mob_after(s_w[w], before));
    *excl = mob_norm(mob_after(ex, before));
    return mob_norm(mob_after(P, before));
}

__global__ __launch_bounds__(kMobThreads) void k_mob_reduce(MobParams p) {
    __shared__ Mob s_w[kMobThreads / kWave];
    const int64_t bh = blockIdx.x / p.nblk;
    const int blk = static_cast<int>(blockIdx.x % p.nblk);
    const int64_t t0 = static_cast<int64_t>(blk) * kMobBlock + static_cast<int64_t>(threadIdx.x) * kMobPer;
    Mob excl;
    const Mob inc = block_scan(thread_composite(p, bh, t0), &excl, s_w);
    if (threadIdx.x == kMobThreads - 1) {
        float* o = p.blk + (bh * p.nblk + blk) * 4;
        o[0] = inc.m11; o[1] = inc.m12; o[2] = inc.m21; o[3] = inc.m22;
    }
}

__global__ __launch_bounds__(kMobThreads) void k_mob_apply(MobParams p) {
    __shared__ Mob s_w[kMobThreads / kWave];
    __shared__ Mob s_carry;
    const int64_t bh = blockIdx.x / p.nblk;
    const int blk = static_cast<int>(blockIdx.x % p.nblk);
    const int64_t t0 = static_cast<int64_t>(blk) * kMobBlock + static_cast<int64_t>(threadIdx.x) * kMobPer;

    if (threadIdx.x == 0) {
        Mob C = mob_identity();
        for (int b = 0; b < blk; ++b) {
            const float* m = p.blk + (bh * p.nblk + b) * 4;
            C = mob_norm(mob_after(Mob{m[0], m[1], m[2], m[3]}, C));
        }
        s_carry = C;
    }
    Mob excl;
    block_scan(thread_composite(p, bh, t0), &excl, s_w);  // also orders s_carry
    const Mob start = mob_after(excl, s_carry);

    const float l0 = p.lambda0 ? p.lambda0[bh] : 1.0f;
    float lam = mob_apply(start, l0);
    const float* a = p.a + bh * p.T;
    const float* pp = p.p + bh * p.T;
    const float* L = p.Lam + bh * p.T;
#pragma unroll
    for (int u = 0; u < kMobPer; ++u) {
        const int64_t t = t0 + u;
        if (t >= p.T) break;
        const float at = a[t];
        const float lpred = lam / __builtin_fmaf(pp[t], lam, at * at);
        const float lnew = lpred + L[t];
        if (p.lambda_out) p.lambda_out[bh * p.T + t] = lnew;
        if (p.F) {
            p.F[bh * p.T + t] = at * lpred / lnew;
            p.G[bh * p.T + t] = L[t] / lnew;
        }
        lam = lnew;
    }
}

int mob_block() { return kMobBlock; }

int mobius_launch(const MobParams& p, int64_t BH, hipStream_t st) {
    if (BH == 0 || p.T == 0) return KDN_OK;
    const int64_t grid = BH * p.nblk;
    hipLaunchKernelGGL(k_mob_reduce, dim3(static_cast<uint32_t>(grid)), dim3(kMobThreads), 0, st, p);
    int rc = launch_status();
    if (rc != KDN_OK) return rc;
    hipLaunchKernelGGL(k_mob_apply, dim3(static_cast<uint32_t>(grid)), dim3(kMobThreads), 0, st, p);
    return launch_status();
}

}  // namespace kdn

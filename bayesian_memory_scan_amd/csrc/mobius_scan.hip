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
// Three launches, O(T) work in all:
//   k_mob_reduce: per (head, block of 4096 tokens) the block's composite;
//   k_mob_carry:  per head, one wave turns the block composites, in place,
//                 into each block's carry-in (the ordered product of all
//                 earlier blocks), 64 blocks per step, the running product
//                 carried from step to step;
//   k_mob_apply:  per (head, block) the in-block exclusive scan of per-thread
//                 composites (a DPP wave scan, LDS across the 4 waves) after
//                 the block's carry-in, then each thread walks its 16 tokens
//                 sequentially from its starting precision and writes
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

// The map of the lane that DPP control CTRL names, in the rows ROWS enables;
// other lanes (no source lane, or a row left out) get the identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or(float x, float id) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), CTRL, ROWS, 0xf, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ Mob mob_dpp(const Mob& M) {
    return {dpp_or<CTRL, ROWS>(M.m11, 1.0f), dpp_or<CTRL, ROWS>(M.m12, 0.0f), dpp_or<CTRL, ROWS>(M.m21, 0.0f),
            dpp_or<CTRL, ROWS>(M.m22, 1.0f)};
}

// Inclusive scan of the wave's 64 maps in lane order: lane l ends with
// M_l o ... o M_0.  Four row_shr steps within each row of 16, then the
// last lane of a row is broadcast into the next row (row_bcast:15, rows 1
// and 3) and lane 31 into the upper half (row_bcast:31, rows 2 and 3).
__device__ __forceinline__ Mob mob_wave_scan(Mob P) {
    P = mob_norm(mob_after(P, mob_dpp<0x111, 0xf>(P)));
    P = mob_norm(mob_after(P, mob_dpp<0x112, 0xf>(P)));
    P = mob_norm(mob_after(P, mob_dpp<0x114, 0xf>(P)));
    P = mob_norm(mob_after(P, mob_dpp<0x118, 0xf>(P)));
    P = mob_norm(mob_after(P, mob_dpp<0x142, 0xa>(P)));
    P = mob_norm(mob_after(P, mob_dpp<0x143, 0xc>(P)));
    return P;
}

// The previous lane's map (wave_shr:1); the identity in lane 0.
__device__ __forceinline__ Mob mob_prev_lane(const Mob& M) { return mob_dpp<0x138, 0xf>(M); }

// Lane 63's map in every lane.
__device__ __forceinline__ Mob mob_last_lane(const Mob& M) {
    return {__int_as_float(__builtin_amdgcn_readlane(__float_as_int(M.m11), kWave - 1)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M.m12), kWave - 1)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M.m21), kWave - 1)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M.m22), kWave - 1))};
}


// The 16 consecutive tokens of one thread: float4 loads when the head's rows
// are 16-byte aligned and the run is whole, else scalar loads (padding:
// a = 1, p = 0, Lambda = 0, the identity map).
struct Run16 {
    float a[kMobPer], p[kMobPer], L[kMobPer];
};

__device__ __forceinline__ void load_run(const MobParams& P, int64_t bh, int64_t t0, Run16& r) {
    const float* a = P.a + bh * P.T;
    const float* pp = P.p + bh * P.T;
    const float* L = P.Lam + bh * P.T;
    if ((P.T & 3) == 0 && t0 + kMobPer <= P.T) {
#pragma unroll
        for (int u = 0; u < kMobPer; u += 4) {
            const float4 x = *reinterpret_cast<const float4*>(a + t0 + u);
            const float4 y = *reinterpret_cast<const float4*>(pp + t0 + u);
            const float4 z = *reinterpret_cast<const float4*>(L + t0 + u);
            r.a[u] = x.x; r.a[u + 1] = x.y; r.a[u + 2] = x.z; r.a[u + 3] = x.w;
            r.p[u] = y.x; r.p[u + 1] = y.y; r.p[u + 2] = y.z; r.p[u + 3] = y.w;
            r.L[u] = z.x; r.L[u + 1] = z.y; r.L[u + 2] = z.z; r.L[u + 3] = z.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kMobPer; ++u) {
            const bool in = t0 + u < P.T;
            r.a[u] = in ? a[t0 + u] : 1.0f;
            r.p[u] = in ? pp[t0 + u] : 0.0f;
            r.L[u] = in ? L[t0 + u] : 0.0f;
        }
    }
}

// Composite of a thread's run (later maps on the left).
__device__ __forceinline__ Mob run_composite(const Run16& r) {
    Mob P = mob_identity();
#pragma unroll
    for (int u = 0; u < kMobPer; ++u) {
        P = mob_after(mob_step(r.a[u], r.p[u], r.L[u]), P);
        if ((u & 3) == 3) P = mob_norm(P);
    }
    return P;
}

// Inclusive scan over the workgroup's 256 thread composites (thread order =
// token order).  Returns the inclusive prefix; *excl receives the exclusive one.
__device__ Mob block_scan(Mob P, Mob* excl, Mob (&s_w)[kMobThreads / kWave]) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    P = mob_wave_scan(P);
    const Mob ex = mob_prev_lane(P);
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
    Run16 run;
    load_run(p, bh, t0, run);
    Mob excl;
    const Mob inc = block_scan(run_composite(run), &excl, s_w);
    if (threadIdx.x == kMobThreads - 1) {
        float* o = p.blk + (bh * p.nblk + blk) * 4;
        o[0] = inc.m11; o[1] = inc.m12; o[2] = inc.m21; o[3] = inc.m22;
    }
}

// Block composites -> carry-ins, in place: one wave per head walks its
// blocks 64 at a time (a wave scan per step, the running product of all
// earlier steps carried in a register).
__global__ __launch_bounds__(kWave) void k_mob_carry(MobParams p) {
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    float* base = p.blk + bh * p.nblk * 4;
    Mob C = mob_identity();
    for (int64_t b0 = 0; b0 < p.nblk; b0 += kWave) {
        const bool in = b0 + lane < p.nblk;
        Mob x = mob_identity();
        if (in) {
            const float4 m = *reinterpret_cast<const float4*>(base + (b0 + lane) * 4);
            x = Mob{m.x, m.y, m.z, m.w};
        }
        const Mob inc = mob_wave_scan(x);
        const Mob cin = mob_norm(mob_after(mob_prev_lane(inc), C));
        if (in) *reinterpret_cast<float4*>(base + (b0 + lane) * 4) = make_float4(cin.m11, cin.m12, cin.m21, cin.m22);
        C = mob_norm(mob_after(mob_last_lane(inc), C));
    }
}

__global__ __launch_bounds__(kMobThreads) void k_mob_apply(MobParams p) {
    __shared__ Mob s_w[kMobThreads / kWave];
    const int64_t bh = blockIdx.x / p.nblk;
    const int blk = static_cast<int>(blockIdx.x % p.nblk);
    const int64_t t0 = static_cast<int64_t>(blk) * kMobBlock + static_cast<int64_t>(threadIdx.x) * kMobPer;

    // carry-in of the block (written by k_mob_carry)
    const float4 cm = *reinterpret_cast<const float4*>(p.blk + (bh * p.nblk + blk) * 4);
    const Mob carry{cm.x, cm.y, cm.z, cm.w};
    Run16 run;
    load_run(p, bh, t0, run);
    Mob excl;
    block_scan(run_composite(run), &excl, s_w);
    const Mob start = mob_after(excl, carry);

    const float l0 = p.lambda0 ? p.lambda0[bh] : 1.0f;
    float lam = mob_apply(start, l0);
    float lo[kMobPer], fo[kMobPer], go[kMobPer];
#pragma unroll
    for (int u = 0; u < kMobPer; ++u) {
        const float at = run.a[u];
        const float lpred = lam * fast_rcp(__builtin_fmaf(run.p[u], lam, at * at));
        const float lnew = lpred + run.L[u];
        const float inv = fast_rcp(lnew);
        lo[u] = lnew;
        fo[u] = at * lpred * inv;
        go[u] = run.L[u] * inv;
        lam = lnew;
    }
    const bool whole = (p.T & 3) == 0 && t0 + kMobPer <= p.T;
    float* lout = p.lambda_out ? p.lambda_out + bh * p.T : nullptr;
    float* Fo = p.F ? p.F + bh * p.T : nullptr;
    float* Go = p.F ? p.G + bh * p.T : nullptr;
    if (whole) {
#pragma unroll
        for (int u = 0; u < kMobPer; u += 4) {
            if (lout) *reinterpret_cast<float4*>(lout + t0 + u) = make_float4(lo[u], lo[u + 1], lo[u + 2], lo[u + 3]);
            if (Fo) {
                *reinterpret_cast<float4*>(Fo + t0 + u) = make_float4(fo[u], fo[u + 1], fo[u + 2], fo[u + 3]);
                *reinterpret_cast<float4*>(Go + t0 + u) = make_float4(go[u], go[u + 1], go[u + 2], go[u + 3]);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < kMobPer; ++u) {
            if (t0 + u >= p.T) break;
            if (lout) lout[t0 + u] = lo[u];
            if (Fo) {
                Fo[t0 + u] = fo[u];
                Go[t0 + u] = go[u];
            }
        }
    }
}

int mob_block() { return kMobBlock; }

int mobius_launch(const MobParams& p, int64_t BH, hipStream_t st) {
    if (BH == 0 || p.T == 0) return KDN_OK;
    const int64_t grid = BH * p.nblk;
    hipLaunchKernelGGL(k_mob_reduce, dim3(static_cast<uint32_t>(grid)), dim3(kMobThreads), 0, st, p);
    int rc = launch_status();
    if (rc != KDN_OK) return rc;
    hipLaunchKernelGGL(k_mob_carry, dim3(static_cast<uint32_t>(BH)), dim3(kWave), 0, st, p);
    if ((rc = launch_status()) != KDN_OK) return rc;
    hipLaunchKernelGGL(k_mob_apply, dim3(static_cast<uint32_t>(grid)), dim3(kMobThreads), 0, st, p);
    return launch_status();
}

}  // namespace kdn

// decode.hip -- one-token decode of the diagonal-precision recurrence.
//
// Same update as the scan (Palimpsa, "Learning to Remember, Learn, and Forget
// in Attention-Based Models", Metodologia 1-2) for a single token, applied in
// place to the stored state (constant-memory decoding, Kalman Delta Networks
// abstract):
//   I'  = alpha I + (1 - alpha) I_prior + beta[i] k[j]^2
//   mu' = (alpha I mu + beta[i] v[i] k[j]) / I'
//   o[i] = sum_j q[j] mu'[j][i]
// The step is a streaming read-modify-write of 2 x d_k x d_v floats per head:
// HBM-bound.  One workgroup (up to 512 threads) per head; each thread owns one
// float4 column group and NF key rows, issues all its state loads before any
// arithmetic, and the per-column partial read-outs are summed across row
// groups through LDS.  State loads and stores are non-temporal: the state is
// touched once per call, so it should not displace anything from the caches
// (and a repeated call cannot be served from the last-level cache).
#include "kdn_params.h"

#include <type_traits>

namespace kdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__((DK * DV / 4 < 512 ? DK * DV / 4 : 512))
void k_decode(DecodeParams p) {
    constexpr int NTH = DK * DV / 4 < 512 ? DK * DV / 4 : 512;
    constexpr int CG = DV / 4;            // float4 column groups per row
    constexpr int RG = NTH / CG;          // row groups
    constexpr int NF = DK / RG;           // rows per thread
    static_assert(NTH % CG == 0 && DK % RG == 0, "decode tile shape");

    __shared__ float4 s_part[RG][CG];

    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int r0 = tid / CG;
    const int64_t bh = blockIdx.x;
    const int h = static_cast<int>(bh % p.H);

    auto load = [&](const void* base, int64_t idx) -> float {
        if constexpr (BF16) return bf16_at(static_cast<const uint16_t*>(base), idx);
        else return static_cast<const float*>(base)[idx];
    };

    f32x4* I4 = reinterpret_cast<f32x4*>(p.I + bh * DK * DV);
    f32x4* M4 = reinterpret_cast<f32x4*>(p.mu + bh * DK * DV);

    // Every small per-token input is loaded first, before the state and so
    // before the first state store.  vmcnt counts loads and stores in issue
    // order, and the compiler cannot move a load of k or q above a store of
    // the state (it cannot rule out aliasing), so a load left inside the row
    // loop would wait for the previous row's stores to complete.
    const float dval = load(p.d, bh);
    // beta == NULL: Palimpsa-M gating, beta[i] = d (the source is selected,
    // not branched on, so that the loads issue back to back)
    const void* bsrc = p.beta ? p.beta : p.d;
    const int64_t b0 = p.beta ? bh * DV + cg * 4 : bh;
    const int bst = p.beta ? 1 : 0;
    float bcol[4], bvcol[4], kr[NF], qr[NF];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float b = load(bsrc, b0 + e * bst);
        bcol[e] = b;
        bvcol[e] = b * load(p.v, bh * DV + cg * 4 + e);
    }
#pragma unroll
    for (int n = 0; n < NF; ++n) {
        const int j = r0 + n * RG;
        kr[n] = load(p.k, bh * DK + j);
        qr[n] = load(p.q, bh * DK + j);
    }
    f32x4 Iv[NF], Mv[NF];
#pragma unroll
    for (int n = 0; n < NF; ++n) {
        const int j = r0 + n * RG;
        Iv[n] = __builtin_nontemporal_load(&I4[j * CG + cg]);
        Mv[n] = __builtin_nontemporal_load(&M4[j * CG + cg]);
    }

    const float alpha = fast_exp(-p.A[h] * dval);
    const float c = (1.0f - alpha) * p.I_prior;

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int n = 0; n < NF; ++n) {
        const int j = r0 + n * RG;
        const float kj = kr[n];
        const float qj = qr[n];
        const float k2 = kj * kj;
        float Io[4] = {Iv[n][0], Iv[n][1], Iv[n][2], Iv[n][3]};
        float Mo[4] = {Mv[n][0], Mv[n][1], Mv[n][2], Mv[n][3]};
        float In[4], Mn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            In[e] = __builtin_fmaf(alpha, Io[e], __builtin_fmaf(bcol[e], k2, c));
            const float eta = __builtin_fmaf(alpha * Io[e], Mo[e], bvcol[e] * kj);
            Mn[e] = eta * fast_rcp(In[e]);
            acc[e] = __builtin_fmaf(qj, Mn[e], acc[e]);
        }
        // the new state is not read again by this call: stream it past the caches
        __builtin_nontemporal_store(f32x4{In[0], In[1], In[2], In[3]}, &I4[j * CG + cg]);
        __builtin_nontemporal_store(f32x4{Mn[0], Mn[1], Mn[2], Mn[3]}, &M4[j * CG + cg]);
    }

    s_part[r0][cg] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (tid < CG) {
        float4 s = s_part[0][tid];
        for (int g = 1; g < RG; ++g) {
            const float4 x = s_part[g][tid];
            s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
        }
        reinterpret_cast<float4*>(p.o + bh * DV)[tid] = s;
    }
}

template <int DK, bool BF16>
static int launch_dv(const DecodeParams& p, int64_t dv, int64_t grid, hipStream_t st) {
    auto go = [&](auto kern, int nth) {
        hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(nth), 0, st, p);
    };
    switch (dv) {
        case 16: go(k_decode<DK, 16, BF16>, DK * 16 / 4 < 512 ? DK * 16 / 4 : 512); break;
        case 32: go(k_decode<DK, 32, BF16>, DK * 32 / 4 < 512 ? DK * 32 / 4 : 512); break;
        case 64: go(k_decode<DK, 64, BF16>, DK * 64 / 4 < 512 ? DK * 64 / 4 : 512); break;
        case 128: go(k_decode<DK, 128, BF16>, DK * 128 / 4 < 512 ? DK * 128 / 4 : 512); break;
        default: return KDN_EUNSUPPORTED;
    }
    return launch_status();
}

template <bool BF16>
static int launch_decode_t(const DecodeParams& p, int64_t dk, int64_t dv, int64_t grid, hipStream_t st) {
    switch (dk) {
        case 16: return launch_dv<16, BF16>(p, dv, grid, st);
        case 32: return launch_dv<32, BF16>(p, dv, grid, st);
        case 64: return launch_dv<64, BF16>(p, dv, grid, st);
        case 128: return launch_dv<128, BF16>(p, dv, grid, st);
        default: return KDN_EUNSUPPORTED;
    }
}

int decode_launch(const DecodeParams& p, int64_t B, int64_t dk, int64_t dv, bool bf16, hipStream_t st) {
    const int64_t grid = B * p.H;
    if (grid == 0) return KDN_OK;
    return bf16 ? launch_decode_t<true>(p, dk, dv, grid, st) : launch_decode_t<false>(p, dk, dv, grid, st);
}

}  // namespace kdn

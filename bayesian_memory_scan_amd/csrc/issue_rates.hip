// issue_rates.hip -- gfx950 VALU issue-rate probe (libkdnprobe.so).
//
// Measurement only: this library is not part of libkdnscan and no scan calls
// it.  It times, on the device, how fast one CU issues the instruction mixes
// that the diagonal-precision scan's inner loop is built from, so that the
// kernel design rests on measured rates rather than on a model:
//
//   * single-instruction chains (8 independent chains per lane, no memory
//     traffic): v_fmac_f32 with VGPR, SGPR and DPP operands, v_mul_f32,
//     v_add_f32, v_rcp_f32, and v_rcp_f32 interleaved with four fmacs;
//   * the per-entry work of the scan (precision update, information-mean
//     update, quotient, read-out) for R key rows x CC value columns per lane,
//     with the quotient taken three ways: one reciprocal per entry ("direct"),
//     one per two key rows ("pair": a/x + b/y = (a y + b x)/(x y)) and one per
//     four ("quad"), with operands either in registers ("alu") or read from
//     LDS per token the way the scan stages them ("lds", plus the read-out's
//     permlane swap and LDS write).
//
// Occupancy is set by the static LDS each workgroup holds: a 256-thread
// workgroup puts one wave on each SIMD, and the grid is 256 * WPS workgroups
// whose LDS lets exactly WPS of them share a CU, so every SIMD runs WPS waves
// for the whole kernel.  Every kernel writes its results, so nothing is dead,
// and every loop runs a fixed trip count: all waves exit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;
constexpr int kRing = 4;   // tokens in the LDS operand ring

// LDS per workgroup (bytes) that lets exactly wps workgroups share a CU's
// 160 KiB: more than 160/(wps+1) KiB, at most 160/wps.
template <int WPS>
constexpr int lds_bytes() {
    return WPS == 1 ? 96 * 1024 : WPS == 2 ? 72 * 1024 : WPS == 4 ? 36 * 1024 : 18 * 1024;
}

__device__ __forceinline__ void opaque(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ void stamp(uint64_t* clk, uint64_t t0, uint64_t r0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = __builtin_amdgcn_s_memtime() - t0;
        clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

// Single-instruction chains.  KIND: 0 fmac (VGPR operands), 1 fmac with an
// SGPR multiplicand, 2 fmac with a DPP row-broadcast multiplicand, 3 mul,
// 4 add, 5 rcp, 6 one rcp + four independent fmacs.
template <int KIND, int WPS>
__global__ __launch_bounds__(kThreads, WPS) void k_single(float* out, float b, float c, int iters,
                                                      uint64_t* clk) {
    __shared__ float pad[lds_bytes<WPS>() / 4];
    float a[kChains], f[kChains][4];
#pragma unroll
    for (int n = 0; n < kChains; ++n) {
        a[n] = 1.0f + 1e-7f * static_cast<float>(threadIdx.x + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[n][e] = 0.5f + 1e-8f * static_cast<float>(n + e);
    }
    float src = b + 1e-9f * static_cast<float>(threadIdx.x);
    opaque(src);
    pad[threadIdx.x] = src;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int n = 0; n < kChains; ++n) {
            if constexpr (KIND == 0) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a[n]) : "v"(src), "v"(c));
            if constexpr (KIND == 1) asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a[n]) : "s"(b), "v"(c));
            if constexpr (KIND == 2)
                asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:3 row_mask:0xf bank_mask:0xf"
                             : "+v"(a[n]) : "v"(src), "v"(c));
            if constexpr (KIND == 3) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(a[n]) : "v"(c));
            if constexpr (KIND == 4) asm volatile("v_add_f32 %0, %0, %1" : "+v"(a[n]) : "v"(c));
            if constexpr (KIND == 5) asm volatile("v_rcp_f32 %0, %0" : "+v"(a[n]));
            if constexpr (KIND == 6) {
                asm volatile("v_rcp_f32 %0, %0" : "+v"(a[n]));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(f[n][e]) : "v"(src), "v"(c));
            }
        }
    }
    stamp(clk, t0, r0);
    float s = pad[(threadIdx.x + 1) % kThreads];
#pragma unroll
    for (int n = 0; n < kChains; ++n) {
        s += a[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) s += f[n][e];
    }
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

// The scan's per-entry work for R key rows x CC value columns per lane.
//   MODE 0 (direct): m = eta * rcp(I) per entry, acc += q m.
//   MODE 1 (pair):   per two rows a, b of a column, N = q_a eta_a I_b + q_b eta_b I_a,
//                    D = I_a I_b, acc += N * rcp(D).
//   MODE 2 (quad):   pairs (a,b), (c,d) combined the same way once more.
// LDS: operands come from an LDS ring laid out as the scan stages a chunk
// (s k, s k^2, q per key row; (beta, beta v) per column), one token ahead,
// and each token's per-column partial read-out is summed with the lane 32
// apart (v_permlane32_swap) and written to LDS.
template <int MODE, int R, int CC, bool LDS, int WPS>
__global__ __launch_bounds__(kThreads, WPS) void k_mix(float* out, int iters, uint64_t* clk) {
    static_assert(R % 4 == 0 && (CC == 1 || CC == 2 || CC == 4), "lane tile");
    constexpr int ROWS = 8 * R;        // key rows of the workgroup: 4 waves x 2 halves x R
    constexpr int COLS = 32 * CC;      // value columns: 32 lanes x CC
    constexpr int RING_FLOATS = kRing * (3 * ROWS + 2 * COLS);
    constexpr int OUT_FLOATS = kRing * 4 * 32 * CC;
    static_assert((RING_FLOATS + OUT_FLOATS) * 4 <= lds_bytes<WPS>(), "LDS ring fits the pad");
    __shared__ float lds[lds_bytes<WPS>() / 4];
    float* ks = lds;
    float* k2s = ks + kRing * ROWS;
    float* qs = k2s + kRing * ROWS;
    float* bvs = qs + kRing * ROWS;           // [kRing][COLS][2]
    float* opart = bvs + kRing * 2 * COLS;    // [kRing][4 waves][32 * CC]

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wv = tid / 64;
    const int half = lane / 32;
    const int cp = lane % 32;
    const int j0 = wv * 2 * R + half * R;

    for (int e = tid; e < RING_FLOATS; e += kThreads) {
        const int seg = e / (kRing * ROWS);
        lds[e] = seg == 0 ? 0.09f : seg == 1 ? 0.008f : seg == 2 ? 0.5f : ((e & 1) ? 0.3f : 0.5f);
    }
    __syncthreads();

    float I[R][CC], eta[R][CC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            I[r][c] = 1.0f + 1e-3f * static_cast<float>(r + c + lane);
            eta[r][c] = 0.1f * static_cast<float>(r - c);
        }

    struct Ops {
        float k[R], k2[R], q[R], bt[CC], bv[CC];
    };
    auto load = [&](int slot) __attribute__((always_inline)) {
        Ops o;
        if constexpr (LDS) {
#pragma unroll
            for (int h = 0; h < R / 4; ++h) {
                const float4 a = *reinterpret_cast<const float4*>(ks + slot * ROWS + j0 + 4 * h);
                const float4 b = *reinterpret_cast<const float4*>(k2s + slot * ROWS + j0 + 4 * h);
                const float4 c = *reinterpret_cast<const float4*>(qs + slot * ROWS + j0 + 4 * h);
                o.k[4 * h] = a.x; o.k[4 * h + 1] = a.y; o.k[4 * h + 2] = a.z; o.k[4 * h + 3] = a.w;
                o.k2[4 * h] = b.x; o.k2[4 * h + 1] = b.y; o.k2[4 * h + 2] = b.z; o.k2[4 * h + 3] = b.w;
                o.q[4 * h] = c.x; o.q[4 * h + 1] = c.y; o.q[4 * h + 2] = c.z; o.q[4 * h + 3] = c.w;
            }
            const float* bp = bvs + (slot * COLS + cp * CC) * 2;
            if constexpr (CC == 1) {
                const float2 u = *reinterpret_cast<const float2*>(bp);
                o.bt[0] = u.x; o.bv[0] = u.y;
            } else {
#pragma unroll
                for (int h = 0; h < CC / 2; ++h) {
                    const float4 u = *reinterpret_cast<const float4*>(bp + 4 * h);
                    o.bt[2 * h] = u.x; o.bv[2 * h] = u.y; o.bt[2 * h + 1] = u.z; o.bv[2 * h + 1] = u.w;
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                o.k[r] = 0.09f; o.k2[r] = 0.008f; o.q[r] = 0.5f;
                opaque(o.k[r]); opaque(o.k2[r]); opaque(o.q[r]);
            }
#pragma unroll
            for (int c = 0; c < CC; ++c) {
                o.bt[c] = 0.5f; o.bv[c] = 0.3f;
                opaque(o.bt[c]); opaque(o.bv[c]);
            }
        }
        return o;
    };

    float dP = 0.004f;
    float sink = 0.0f;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    Ops cur = load(0);
    for (int it = 0; it < iters; it += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const Ops nxt = load((u + 1) % kRing);
            opaque(dP);
            float acc[CC];
#pragma unroll
            for (int c = 0; c < CC; ++c) {
                if constexpr (MODE == 0) {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        I[r][c] = __builtin_fmaf(cur.k2[r], cur.bt[c], I[r][c]) + dP;
                        eta[r][c] = __builtin_fmaf(cur.k[r], cur.bv[c], eta[r][c]);
                        const float m = eta[r][c] * __builtin_amdgcn_rcpf(I[r][c]);
                        acc[c] = r == 0 ? cur.q[r] * m : __builtin_fmaf(cur.q[r], m, acc[c]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        I[r][c] = __builtin_fmaf(cur.k2[r], cur.bt[c], I[r][c]) + dP;
                        eta[r][c] = __builtin_fmaf(cur.k[r], cur.bv[c], eta[r][c]);
                    }
                    constexpr int G = MODE == 1 ? 2 : 4;
#pragma unroll
                    for (int g = 0; g < R; g += G) {
                        // pair (a, b) = (g, g+1): N = q_a eta_a I_b + q_b eta_b I_a, D = I_a I_b
                        float n0 = cur.q[g] * (eta[g][c] * I[g + 1][c]);
                        n0 = __builtin_fmaf(cur.q[g + 1], eta[g + 1][c] * I[g][c], n0);
                        float d0 = I[g][c] * I[g + 1][c];
                        if constexpr (G == 4) {
                            float n1 = cur.q[g + 2] * (eta[g + 2][c] * I[g + 3][c]);
                            n1 = __builtin_fmaf(cur.q[g + 3], eta[g + 3][c] * I[g + 2][c], n1);
                            const float d1 = I[g + 2][c] * I[g + 3][c];
                            n0 = __builtin_fmaf(n1, d0, n0 * d1);
                            d0 = d0 * d1;
                        }
                        const float rq = __builtin_amdgcn_rcpf(d0);
                        acc[c] = g == 0 ? n0 * rq : __builtin_fmaf(n0, rq, acc[c]);
                    }
                }
            }
            if constexpr (LDS) {
                float* op = opart + (u * 4 + wv) * 32 * CC;
                if constexpr (CC == 1) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0]),
                                                                     __float_as_uint(acc[0]), false, false);
                    if (half == 0) op[cp] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                } else {
#pragma unroll
                    for (int c = 0; c < CC; c += 2) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[c]),
                                                                         __float_as_uint(acc[c + 1]), false, false);
                        op[cp * CC + c + half] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < CC; ++c) sink += acc[c];
            }
            cur = nxt;
        }
    }
    stamp(clk, t0, r0);
    float s = sink;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CC; ++c) s += I[r][c] + eta[r][c];
    if constexpr (LDS) {
        __syncthreads();
        s += opart[tid % OUT_FLOATS];
    }
    out[static_cast<int64_t>(blockIdx.x) * kThreads + tid] = s;
}

typedef void (*single_fn)(float*, float, float, int, uint64_t*);
typedef void (*mix_fn)(float*, int, uint64_t*);

struct Entry {
    const char* name;
    int kind;        // 0: single-instruction chain, 1: scan mix
    int per_iter;    // lane-instructions (chains) or entry-steps (mixes) per loop trip
    const void* fn[4];   // 1, 2, 4, 8 waves per SIMD
};

#define SINGLE(NAME, K, PER)                                                                   \
    {NAME, 0, PER,                                                                             \
     {reinterpret_cast<const void*>(&k_single<K, 1>), reinterpret_cast<const void*>(&k_single<K, 2>), \
      reinterpret_cast<const void*>(&k_single<K, 4>), reinterpret_cast<const void*>(&k_single<K, 8>)}}
#define MIX(NAME, M, R, CC, L)                                                                  \
    {NAME, 1, (R) * (CC),                                                                       \
     {reinterpret_cast<const void*>(&k_mix<M, R, CC, L, 1>),                                    \
      reinterpret_cast<const void*>(&k_mix<M, R, CC, L, 2>),                                    \
      reinterpret_cast<const void*>(&k_mix<M, R, CC, L, 4>),                                    \
      reinterpret_cast<const void*>(&k_mix<M, R, CC, L, 8>)}}

const Entry kEntries[] = {
    SINGLE("fmac", 0, kChains),
    SINGLE("fmac_sgpr", 1, kChains),
    SINGLE("fmac_dpp", 2, kChains),
    SINGLE("mul", 3, kChains),
    SINGLE("add", 4, kChains),
    SINGLE("rcp", 5, kChains),
    SINGLE("rcp+4fmac", 6, 5 * kChains),
    MIX("direct 4x2 alu", 0, 4, 2, false),
    MIX("pair 4x2 alu", 1, 4, 2, false),
    MIX("quad 4x2 alu", 2, 4, 2, false),
    MIX("direct 4x2 lds", 0, 4, 2, true),
    MIX("pair 4x2 lds", 1, 4, 2, true),
    MIX("quad 4x2 lds", 2, 4, 2, true),
    MIX("direct 4x1 lds", 0, 4, 1, true),
    MIX("quad 4x1 lds", 2, 4, 1, true),
    MIX("quad 4x4 lds", 2, 4, 4, true),
    MIX("quad 8x2 lds", 2, 8, 2, true),
    MIX("quad 8x1 lds", 2, 8, 1, true),
};
constexpr int kNumEntries = sizeof(kEntries) / sizeof(kEntries[0]);

}  // namespace

extern "C" {

int kdn_probe_count(void) { return kNumEntries; }

const char* kdn_probe_name(int i) { return i >= 0 && i < kNumEntries ? kEntries[i].name : nullptr; }

// Lane-instructions (chains) or entry-steps (mixes) per lane per loop trip.
int kdn_probe_per_iter(int i) { return i >= 0 && i < kNumEntries ? kEntries[i].per_iter : 0; }

// Runs probe i with wps waves per SIMD (1, 2, 4 or 8) for `iters` loop trips
// per lane: one untimed launch, then one timed by HIP events.  Writes the
// timed launch's milliseconds, workgroup 0's shader clocks and 100 MHz
// real-time ticks over its loop, and the kernel's VGPR count.  Returns 0, or
// a negative value on bad arguments or a HIP error.
int kdn_probe_run(int i, int wps, int iters, float* ms, uint64_t* clocks, uint64_t* ticks, int* vgprs) {
    if (i < 0 || i >= kNumEntries || iters <= 0 || iters % kRing != 0) return -1;
    const int slot = wps == 1 ? 0 : wps == 2 ? 1 : wps == 4 ? 2 : wps == 8 ? 3 : -1;
    if (slot < 0) return -1;
    const Entry& e = kEntries[i];
    const int blocks = 256 * wps;
    float* out = nullptr;
    uint64_t* clk = nullptr;
    if (hipMalloc(&out, sizeof(float) * blocks * kThreads) != hipSuccess) return -2;
    if (hipMalloc(&clk, 2 * sizeof(uint64_t)) != hipSuccess) {
        (void)hipFree(out);
        return -2;
    }
    hipFuncAttributes attr{};
    (void)hipFuncGetAttributes(&attr, e.fn[slot]);
    if (vgprs) *vgprs = attr.numRegs;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    int rc = 0;
    for (int rep = 0; rep < 2 && rc == 0; ++rep) {
        if (rep == 1) (void)hipEventRecord(e0, nullptr);
        if (e.kind == 0)
            hipLaunchKernelGGL(reinterpret_cast<single_fn>(const_cast<void*>(e.fn[slot])), dim3(blocks),
                               dim3(kThreads), 0, nullptr, out, 1.0000001f, 1e-8f, iters, clk);
        else
            hipLaunchKernelGGL(reinterpret_cast<mix_fn>(const_cast<void*>(e.fn[slot])), dim3(blocks),
                               dim3(kThreads), 0, nullptr, out, iters, clk);
        if (hipGetLastError() != hipSuccess) rc = -3;
        if (rep == 1) (void)hipEventRecord(e1, nullptr);
        if (hipDeviceSynchronize() != hipSuccess) rc = -3;
    }
    if (rc == 0) {
        (void)hipEventElapsedTime(ms, e0, e1);
        uint64_t h[2] = {0, 0};
        if (hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) rc = -3;
        *clocks = h[0];
        *ticks = h[1];
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(out);
    (void)hipFree(clk);
    return rc;
}

}  // extern "C"

// kdn_lane.h -- wave-level helpers for gfx950: DPP row broadcasts, the
// cross-lane sums used by the scans, and the XCD-aware workgroup numbering.
#pragma once

#include <type_traits>

#include "kdn_internal.h"

namespace kdn {

// v_fmac_f32 with its first multiplicand broadcast from lane N of each row of
// 16 lanes (DPP row_newbcast): acc += bcast_N(src) * other.  One VGPR holding
// a value per lane of a row then feeds 16 multiply-adds without LDS traffic.
template <int N>
__device__ __forceinline__ void fmac_bcast(float& acc, float src, float other) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(src), "v"(other), "n"(N));
}

// A VALU write of a VGPR needs two wait states before a DPP instruction may
// read it as its (permuted) source.  The compiler inserts them for its own
// DPP instructions but cannot see inside the fmac_bcast asm, so every value
// fed to fmac_bcast that a VALU instruction produced passes through here: the
// s_nop provides the wait states and ties the value's last write before it.
// The build also scans the generated code for any remaining hazard.
__device__ __forceinline__ float dpp_src(float x) {
    asm volatile("s_nop 1" : "+v"(x));
    return x;
}

// x *= s in place (the result stays in x's register).  Used inside uniform
// branches on loop-carried state: a plain multiply lets the register
// allocator pick a new register in one branch and then copy every value
// back at the merge.
__device__ __forceinline__ void scale_inplace(float& x, float s) {
    asm("v_mul_f32 %0, %1, %0" : "+v"(x) : "s"(s));
}

// A wave-uniform value copied into a VGPR.  VALU instructions with an SGPR
// operand issue at half the rate of all-VGPR ones on gfx950, so a scalar
// read by many instructions is moved once.
__device__ __forceinline__ float vgpr_copy(float s) {
    float v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
    return v;
}

// Compile-time loop N, N+1, ..., END-1 (register arrays need constant indices).
template <int N, int END>
struct Unroll {
    template <typename F>
    __device__ __forceinline__ static void run(F&& f) {
        f(std::integral_constant<int, N>{});
        Unroll<N + 1, END>::run(f);
    }
};
template <int END>
struct Unroll<END, END> {
    template <typename F>
    __device__ __forceinline__ static void run(F&&) {}
};

// Workgroups are dealt to the 8 XCDs round-robin by blockIdx.  Renumber them
// so that consecutive logical ids run on one XCD: the column tiles of a head
// (adjacent ids) then share that XCD's L2 and read the key side from HBM once.
__device__ __forceinline__ int64_t xcd_local_id() {
    constexpr uint32_t kXcd = 8;
    const uint32_t n = gridDim.x;
    const uint32_t b = blockIdx.x;
    const uint32_t full = n / kXcd * kXcd;
    if (b >= full) return b;
    return static_cast<int64_t>(b % kXcd) * (full / kXcd) + b / kXcd;
}

// Value of lane N of this lane's row of 16 (DPP row_newbcast), as a plain
// operand; the compiler folds it into the consuming v_mul_f32.
template <int N>
__device__ __forceinline__ float bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, true));
}

__device__ __forceinline__ float uniform(float x) {
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(x)));
}

// A wave-uniform 64-bit integer moved to scalar registers (integer division
// leaves its results in VGPRs).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint64_t u = static_cast<uint64_t>(x);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// DPP lane permutations inside a row of 16 lanes, each an involution:
// row_mirror pairs l with 15-l, row_half_mirror l with 7-l (within 8),
// quad_perm [3,2,1,0] l with 3-l (within 4), quad_perm [1,0,3,2] l with l^1.
constexpr int kDppMirror = 0x140;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppQuadReverse = 0x1b;
constexpr int kDppQuadSwap1 = 0xb1;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// v_permlane32_swap / v_permlane16_swap (gfx950) followed by an add:
// returns, in the lanes of the lower half (of the wave / of each 32), a summed
// with its partner lane's a, and in the upper half b summed with its partner's b.
__device__ __forceinline__ float swap32_add(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_add(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One butterfly level inside a row of 16 on a pair (a, b): lanes whose bit
// BIT is clear keep a summed with their partner's a, the others b with their
// partner's b.  The partner (given by CTRL) has BIT flipped.
template <int CTRL, int BIT>
__device__ __forceinline__ float pair_level(float a, float b, int lane) {
    const bool hi = (lane >> BIT) & 1;
    const float keep = hi ? b : a;
    const float send = hi ? a : b;
    return keep + dpp<CTRL>(send);
}

// Last four butterfly levels of a 64-lane sum of 32 values, after the two
// permlane levels have left 8 partial sums per lane (x[m] holds, in lanes
// with bit 4 clear, value m and otherwise value m + 8 of its half).
__device__ __forceinline__ float wave_sum32_tail(const float (&x)[8], int lane) {
    float y[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) y[m] = pair_level<kDppMirror, 3>(x[m], x[m + 4], lane);
    float z[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) z[m] = pair_level<kDppHalfMirror, 2>(y[m], y[m + 2], lane);
    const float r = pair_level<kDppQuadReverse, 1>(z[0], z[1], lane);
    return r + dpp<kDppQuadSwap1>(r);
}

// Sum 32 values per lane over all 64 lanes of the wave.  On return lane l
// holds the total of value v[(l >> 5) * 16 + ((l >> 1) & 15)] (lanes l and
// l^1 hold the same total).  70 VALU operations for 32 sums.
__device__ __forceinline__ float wave_sum32(const float (&v)[32], int lane) {
    float w[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) w[m] = swap32_add(v[m], v[m + 16]);
    float x[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) x[m] = swap16_add(w[m], w[m + 8]);
    return wave_sum32_tail(x, lane);
}

// Sum two values over all 64 lanes: lanes 0-31 return the total of a,
// lanes 32-63 the total of b.
__device__ __forceinline__ float wave_sum2(float a, float b) {
    float x = swap32_add(a, b);
    x = swap16_add(x, x);
    x += dpp<kDppMirror>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppQuadReverse>(x);
    return x + dpp<kDppQuadSwap1>(x);
}

// Maximum over the 64 lanes of the wave, returned in every lane.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kDppQuadSwap1>(x));
    x = fmaxf(x, dpp<kDppQuadReverse>(x));
    x = fmaxf(x, dpp<kDppHalfMirror>(x));
    x = fmaxf(x, dpp<kDppMirror>(x));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Buffer resource over `bytes` bytes from `base` (raw, untyped, gfx9 format
// word).  Loads past the end return 0 and stores past the end are dropped, so
// a ragged chunk needs no branches: the wait counters stay exact and the next
// chunk's loads stay in flight.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// N contiguous floats at byte offset `off` (16-byte aligned for N >= 4,
// 8-byte for N == 2).
template <int N>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[N]) {
    if constexpr (N >= 4) {
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * e, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[e + i] = __uint_as_float(u[i]);
        }
    } else if constexpr (N == 2) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        x[0] = __uint_as_float(u[0]);
        x[1] = __uint_as_float(u[1]);
    } else {
        x[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
}

template <int N>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&x)[N]) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    if constexpr (N >= 4) {
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const u32x4 u = {__float_as_uint(x[e]), __float_as_uint(x[e + 1]), __float_as_uint(x[e + 2]),
                             __float_as_uint(x[e + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(u, r, off + 4 * e, 0, 0);
        }
    } else if constexpr (N == 2) {
        const u32x2 u = {__float_as_uint(x[0]), __float_as_uint(x[1])};
        __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[0]), r, off, 0, 0);
    }
}


// N contiguous 16-bit (bf16) or 32-bit (fp32) elements of type E at byte
// offset `off`, widened to fp32 (bf16 is the top half of an fp32).  The run
// is aligned to its own size.
template <typename E, int N>
__device__ __forceinline__ void buf_load_widen(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[N]) {
    if constexpr (sizeof(E) == 4) {
        buf_load<N>(r, off, x);
    } else if constexpr (N >= 8) {
#pragma unroll
        for (int e = 0; e < N; e += 8) {
            const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, off + 2 * e, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[e + 2 * i] = __uint_as_float(u[i] << 16);
                x[e + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
            }
        }
    } else if constexpr (N == 4) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else if constexpr (N == 2) {
        const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xffff0000u);
    } else {
        x[0] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
    }
}

// N contiguous floats (16-byte aligned for N >= 4, 8-byte for N == 2).
template <int N>
__device__ __forceinline__ void store_run(float* dst, const float (&x)[N]) {
    if constexpr (N >= 4) {
#pragma unroll
        for (int e = 0; e < N; e += 4)
            *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(x[0], x[1]);
    } else {
        dst[0] = x[0];
    }
}

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_prefix16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    return x;
}

}  // namespace kdn

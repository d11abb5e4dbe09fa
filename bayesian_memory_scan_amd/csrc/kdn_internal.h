// kdn_internal.h -- helpers shared by the libkdnscan translation units.
// gfx950 (CDNA4) only: wave64, 64 KiB-per-workgroup static LDS limit lifted
// to 160 KiB per CU, fp32 VALU without packed math.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/kdnscan.h"

namespace kdn {

constexpr int kWave = 64;
constexpr int kNumCU = 256;  // MI355X compute units (8 XCDs x 32)

// Element-wise passes: 256-thread workgroups walking their range with a grid
// stride, so the grid stays far below the 2^32 - 1 work-item limit of one
// dispatch whatever the element count.
constexpr int kElemThreads = 256;
constexpr int64_t kElemMaxGroups = 65536;   // 16.8 M threads: 32 waves on every SIMD

inline uint32_t elem_groups(int64_t n) {
    const int64_t g = (n + kElemThreads - 1) / kElemThreads;
    return static_cast<uint32_t>(g < kElemMaxGroups ? g : kElemMaxGroups);
}

__device__ __forceinline__ int64_t elem_first() {
    return static_cast<int64_t>(blockIdx.x) * kElemThreads + threadIdx.x;
}
__device__ __forceinline__ int64_t elem_stride() {
    return static_cast<int64_t>(gridDim.x) * kElemThreads;
}

// bf16 -> fp32 is exact: the bf16 bits are the top half of the float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Raw hardware reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Load one 16-byte vector of elements from global memory.
__device__ __forceinline__ uint4 ld16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Widen a 16-byte vector (8 bf16 or 4 f32) into floats; returns the count.
template <bool BF16>
__device__ __forceinline__ void widen(const uint4& u, float* out) {
    if constexpr (BF16) {
        out[0] = bf16_lo(u.x); out[1] = bf16_hi(u.x);
        out[2] = bf16_lo(u.y); out[3] = bf16_hi(u.y);
        out[4] = bf16_lo(u.z); out[5] = bf16_hi(u.z);
        out[6] = bf16_lo(u.w); out[7] = bf16_hi(u.w);
    } else {
        out[0] = __uint_as_float(u.x); out[1] = __uint_as_float(u.y);
        out[2] = __uint_as_float(u.z); out[3] = __uint_as_float(u.w);
    }
}

// A 16-byte vector holding VW copies of element idx (bf16 bits or f32): the
// input gate of Palimpsa-M gating, where beta_t[i] = d_t for every i.
template <bool BF16>
__device__ __forceinline__ uint4 splat16(const void* base, int64_t idx) {
    if constexpr (BF16) {
        const uint32_t b = static_cast<const uint16_t*>(base)[idx];
        const uint32_t w = b | (b << 16);
        return make_uint4(w, w, w, w);
    } else {
        const uint32_t b = __float_as_uint(static_cast<const float*>(base)[idx]);
        return make_uint4(b, b, b, b);
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool head_size_ok(int64_t n) { return n == 16 || n == 32 || n == 64 || n == 128; }

// Records the error of the last failed launch (per thread) for
// kdn_last_hip_error().
void note_hip_error(hipError_t e);

inline int launch_status() {
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return KDN_OK;
    note_hip_error(e);
    return KDN_EHIP;
}

// A caller's timing event (a hipEvent_t, or NULL for none), recorded on the
// call's stream.
inline int record_event(void* ev, hipStream_t st) {
    if (ev == nullptr) return KDN_OK;
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(ev), st);
    if (e == hipSuccess) return KDN_OK;
    note_hip_error(e);
    return KDN_EHIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace kdn

// Device helpers shared by the matrix-core kernels (refine band, sigmoid
// chunk score, chunk attention mass).  Included by .hip sources only.
#pragma once

#include "lsa_internal.h"

namespace lsa_dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Block barrier for data shared through LDS only: it waits for the wave's
// LDS operations but lets its global loads and stores stay in flight (the
// workgroup release of a __syncthreads() waits for all of them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two ulps of fp32 per operation: Higham's gamma(n) = n u / (1 - n u) taken
// with u = 2^-22, which also covers an accumulation that truncates.
constexpr float kU2 = 2.384185791015625e-07f;
__host__ __device__ constexpr float gam(int n) { return n * kU2 / (1.0f - n * kU2); }

// 8 fp8 e4m3fn bytes -> 8 bf16 (exact: every e4m3 value is a bf16 value;
// the conversion scale is 1)
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return r;
}

// Element offset of the 8 dims lane group lq holds in MFMA k-step ks.  Any
// order of the dims gives the same dot products as long as both operands
// use it; fp8 rows are read 16 bytes (two k-steps) per lane.
template <int KDT>
__device__ __forceinline__ int kdim(int ks, int lq) {
    if constexpr (KDT == LSA_FP8_E4M3FN) return (ks >> 1) * 64 + lq * 16 + (ks & 1) * 8;
    else return ks * 32 + lq * 8;
}

__device__ __forceinline__ float sumsq_bf16x8(uint4 v) {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xffff0000u);
        s = __builtin_fmaf(lo, lo, s);
        s = __builtin_fmaf(hi, hi, s);
    }
    return s;
}

// x + x of lane ^ 16 and x + x of lane ^ 32 (permlane swaps, no LDS)
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace lsa_dev

// Device-side building blocks shared by the gfx950 kernels: vector types for
// the bf16 matrix-core (MFMA) operands, conversions and wave-level helpers.
//
// MFMA operand layouts used throughout (wave64, verified on gfx950):
//   v_mfma_f32_32x32x16_bf16  D[32][32] += A[32][16] * B[16][32]
//     A: lane l holds row l%32, k = 8*(l/32) + e for its 8 elements e
//     B: lane l holds col l%32, k = 8*(l/32) + e
//     D: lane l holds col l%32, rows 8*(r/4) + 4*(l/32) + r%4 in register r
// Because A and B index k the same way, any permutation of the contraction
// dimension that is applied to both operands leaves the product unchanged;
// the kernels use that to make every lane's operand a contiguous 16-byte
// load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Raw 16- and 8-byte payloads.  Native vector types (not HIP's uint4 struct)
// so that arrays of them stay in registers instead of private memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Fourth word of a raw buffer resource (32-bit data format, no swizzle):
// loads through such a resource past its size return zeros without touching
// memory.
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Device-coherent 8-byte store and load of two floats: partial results that
// one workgroup leaves for another inside a launch bypass the per-XCD caches,
// so no cache needs writing back or invalidating.  A workgroup waits for its
// own stores (s_waitcnt vmcnt(0)) before it takes the ticket that hands them
// over.
__device__ __forceinline__ void coherent_st64(uint64_t* p, float lo, float hi) {
    const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, lo) |
                       ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 coherent_ld64(const uint64_t* p) {
    const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__builtin_bit_cast(float, (uint32_t)v), __builtin_bit_cast(float, (uint32_t)(v >> 32)));
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)), with the device erff.
__device__ __forceinline__ float gelu_erf(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// GELU with erf from Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (Hastings' approximation): for x >= 0
//     erf(x) ~= 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//     t = 1 / (1 + p x),
// with |error| <= 1.5e-7, and erf(-x) = -erf(x).  Branch-free; used where
// the result feeds a bf16 pipeline.
//
// Written as GELU(z) = max(z, 0) - |z| * (poly / 2) * exp(-z^2 / 2), which is
// z Phi(z) for either sign of z, with the factors 1/sqrt(2) and 1/2 folded
// into the constants: 11 VALU operations and two transcendentals.
__device__ __forceinline__ float gelu_fast(float z) {
    constexpr float p = 0.3275911f * 0.70710678118654752f;
    constexpr float a1 = 0.5f * 0.254829592f, a2 = 0.5f * -0.284496736f, a3 = 0.5f * 1.421413741f;
    constexpr float a4 = 0.5f * -1.453152027f, a5 = 0.5f * 1.061405429f;
    constexpr float e_scale = -0.5f * 1.4426950408889634f;  // exp(-a^2/2) = 2^(a^2 e_scale)
    const float a = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(fmaf(p, a, 1.0f));
    const float half_poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
    const float e = __builtin_amdgcn_exp2f(a * a * e_scale);
    return fmaf(-a * half_poly, e, fmaxf(z, 0.0f));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace tg

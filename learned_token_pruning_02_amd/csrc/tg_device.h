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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ uint4 as_uint4(bf16x8 v) {
    return __builtin_bit_cast(uint4, v);
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

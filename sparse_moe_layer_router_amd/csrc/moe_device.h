// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand (8 values per lane)
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // 16x16 MFMA accumulator (4 per lane)
typedef __attribute__((ext_vector_type(16))) float f32x16_t;   // 32x32 MFMA accumulator (16 per lane)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16-byte load / store unit
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;  // 8-byte unit

#define MOE_WAVE 64

namespace moe {

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bfloat16, round to nearest, ties to even, NaN stays NaN (quiet), denormals kept: the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32), two values per instruction.
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_hw_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw_t){lo, hi}, bf16x2_hw_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }

// Streaming 16-byte load for data read exactly once (expert weights): non-temporal hint.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4_t*)p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Sum over the 64 lanes of a wave with a fixed butterfly order (deterministic); every lane gets it.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
  return v;
}

// SiLU(z) = z * sigmoid(z). The hardware reciprocal (about 1 ulp) replaces the IEEE division: the
// result is rounded to bf16 or summed in fp32 next, and the division's correction sequence made
// the GEMM epilogue several times longer. 1 + exp(-z) >= 1, and its reciprocal is 0 when it
// overflows (z below about -88), so the result is -0 there, as the division gives.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (MOE_WAVE - 1)); }

}  // namespace moe

// One-byte weight codes -> bf16, in registers: the decode step of the INT8 and FP8 (E4M3) expert
// weights (inference-optimisation chapter, model-compression part: one byte per weight halves the
// bytes decode reads; the layer uses the code's value times the row scale, and the scale is applied
// to the fp32 accumulators, not here). Shared by the weight-streaming kernels and the dequantizer,
// so a check of the dequantizer over every code checks what the layer multiplies.
#pragma once

#include "kernels.h"
#include "moe_device.h"

namespace moe {

// Eight int8 codes (two little-endian words) -> the eight bf16 values, byte i of lo in the low half
// of word i / 2. Exact: |q| <= 127 has at most 7 significant bits, so the float's low 16 bits are
// zero and its high half is the bf16 value; one byte permute packs the high halves of a pair.
__device__ __forceinline__ u32x4_t i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = i < 2 ? lo : hi;
    const int b = (i & 1) * 2;  // byte index of the pair's first code
    const float f0 = (float)((int32_t)(w << (24 - 8 * b)) >> 24);
    const float f1 = (float)((int32_t)(w << (16 - 8 * b)) >> 24);
    r[i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return r;
}

// Eight E4M3 codes -> the eight bf16 values, the same order, by gfx950's packed conversion (two
// codes of one 16-bit half of a word per instruction, OCP E4M3: bias 7, subnormals, S.1111.111 NaN),
// with the conversion's scale at 1. Exact: every finite E4M3 value (at most 4 significant bits,
// exponents -9..8) is a bf16 value.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return u32x4_t{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1), __builtin_bit_cast(uint32_t, v2),
                 __builtin_bit_cast(uint32_t, v3)};
}

// The eight bf16 values of eight one-byte codes of the layout (INT8 or E4M3; the bf16 layouts never
// reach it).
template <int LAYOUT>
__device__ __forceinline__ u32x4_t codes_to_bf16x8(uint32_t lo, uint32_t hi) {
  if (LAYOUT == kFp8Frag) return e4m3x8_to_bf16x8(lo, hi);
  return i8x8_to_bf16x8(lo, hi);
}

}  // namespace moe

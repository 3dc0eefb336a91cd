// One-time INT8 or FP8 quantization of expert weights (MOE_LAYOUT_INT8_FRAG, MOE_LAYOUT_FP8_FRAG).
//
// Inference-optimisation chapter (fangpin.github.io, LLM-from-scratch ch. 6), model-compression
// part, second route ("make every byte cheaper"): decode reads every selected weight once, so one
// byte per weight instead of two halves the traffic; the affine code is x_q = round(x / s) + z.
// Sparse-MoE overview article (adg.csdn.net), section 4.3: INT8 expert weights for the same reason.
//
// Here: symmetric (z = 0), one scale per output channel (matrix row): s = max|w_row| / 127 and
// q = rint(w / s), both in float32 with IEEE division, so the codes are reproducible bit for bit.
// FP8: s = max|w_row| / 448 and the code is the E4M3 value nearest to w / s (OCP 8-bit float, "fn"
// variant: bias 7, 3 mantissa bits, subnormals, largest finite 448), ties to the even code,
// magnitudes from 464 up saturating to 448.
// Codes are stored in the fragment order the streaming kernels read: every 1 KB is a 16-row x
// 64-column block; lane l of a wave holds row l % 16, columns 8 * (l / 16) .. +8 of the block's
// first 32 columns followed by the same 8 columns of its second 32, i.e. the bf16 16x16x32 MFMA
// A-operand chunks of two consecutive K steps. The float32 row scales follow all the codes.
#include "codes.h"
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

// one wave per row: the largest magnitude, then the scale (0 for an all-zero row)
template <bool FP8>
__global__ void __launch_bounds__(256)
quant_row_scale_kernel(const uint16_t* __restrict__ src, float* __restrict__ scale, long long n_rows, int cols) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int lane = lane_id();
  const uint16_t* r = src + (size_t)row * cols;
  float m = 0.f;
  for (int c = lane * 8; c < cols; c += 64 * 8) {
    const u32x4_t v = ld16(r + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[q] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[q] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) scale[row] = m / (FP8 ? 448.0f : 127.0f);
}

// float32 -> E4M3 code: the nearest value, ties to the even code, on the float's own bits. At or
// above 464 (and for NaN) the code saturates to 448 (0x7E); below 2^-6 the value is rounded on the
// subnormal grid of 2^-9 (8 steps = 2^-6, the first normal code). Otherwise the float32 mantissa is
// rounded to 3 bits (add half minus one plus the lowest kept bit, then shift), a carry moving to
// the next exponent. The sign bit is the input's.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a < 464.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  const uint32_t ab = __float_as_uint(a);
  uint32_t e = (ab >> 23) - 120u;  // E4M3 biased exponent: (exp - 127) + 7, in 1..15
  const uint32_t m23 = ab & 0x7FFFFFu;
  uint32_t m = (m23 + 0x7FFFFu + ((m23 >> 20) & 1u)) >> 20;
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  return sign | (e << 3) | m;
}

template <bool FP8>
__device__ __forceinline__ uint32_t quant4(uint32_t a, uint32_t b, float s) {
  // four bf16 values (two per word) -> four one-byte codes, little-endian
  const float v[4] = {bf16_to_f32(a & 0xFFFFu), bf16_to_f32(a >> 16), bf16_to_f32(b & 0xFFFFu), bf16_to_f32(b >> 16)};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t code = 0;
    if (FP8) {
      code = s > 0.f ? f32_to_e4m3(v[i] / s) : 0u;
    } else {
      float q = s > 0.f ? rintf(v[i] / s) : 0.f;
      q = fminf(fmaxf(q, -127.f), 127.f);
      code = (uint32_t)(int32_t)q & 0xFFu;
    }
    out |= code << (8 * i);
  }
  return out;
}

// one thread per 16-byte output chunk: chunk o is lane (o % 64) of 1 KB block (o / 64)
template <bool FP8>
__global__ void __launch_bounds__(256)
quant_pack_kernel(const uint16_t* __restrict__ src, const float* __restrict__ scale, int8_t* __restrict__ dst,
                  long long n_mats, int rows, int cols) {
  const long long per_mat = (long long)rows * cols / 16;
  const long long total = n_mats * per_mat;
  const int kb_per_band = cols / 64;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const long long m = o / per_mat;
    const long long q = o - m * per_mat;
    const long long blk = q / 64;
    const int lane = (int)(q % 64);
    const long long band = blk / kb_per_band;
    const int kb = (int)(blk % kb_per_band);
    const long long r = band * 16 + (lane & 15);
    const int c = kb * 64 + (lane >> 4) * 8;
    const uint16_t* sr = src + (size_t)m * rows * cols + (size_t)r * cols;
    const float s = scale[(size_t)m * rows + r];
    const u32x4_t lo = ld16(sr + c), hi = ld16(sr + c + 32);
    const u32x4_t out = {quant4<FP8>(lo[0], lo[1], s), quant4<FP8>(lo[2], lo[3], s), quant4<FP8>(hi[0], hi[1], s),
                         quant4<FP8>(hi[2], hi[3], s)};
    *(u32x4_t*)(dst + (size_t)m * rows * cols + (size_t)q * 16) = out;
  }
}

// The inverse view: one thread per 16-byte chunk of codes (the same chunk numbering), decoded by
// the streaming kernels' own code -> bf16 step, then times the row scale in float32, written to the
// row-major float32 matrix (8 + 8 consecutive columns).
template <int LAYOUT>
__global__ void __launch_bounds__(256)
dequant_kernel(const int8_t* __restrict__ codes, const float* __restrict__ scale, float* __restrict__ dst,
               long long n_mats, int rows, int cols) {
  const long long per_mat = (long long)rows * cols / 16;
  const long long total = n_mats * per_mat;
  const int kb_per_band = cols / 64;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const long long m = o / per_mat;
    const long long q = o - m * per_mat;
    const long long blk = q / 64;
    const int lane = (int)(q % 64);
    const long long r = (blk / kb_per_band) * 16 + (lane & 15);
    const int c = (int)(blk % kb_per_band) * 64 + (lane >> 4) * 8;
    const u32x4_t w = *(const u32x4_t*)(codes + (size_t)m * rows * cols + (size_t)q * 16);
    const float s = scale[(size_t)m * rows + r];
    const u32x4_t v[2] = {codes_to_bf16x8<LAYOUT>(w[0], w[1]), codes_to_bf16x8<LAYOUT>(w[2], w[3])};
    float* out = dst + (size_t)m * rows * cols + (size_t)r * cols + c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4_t a, b;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        a[2 * j] = bf16_to_f32(v[h][j] & 0xFFFFu) * s;
        a[2 * j + 1] = bf16_to_f32(v[h][j] >> 16) * s;
        b[2 * j] = bf16_to_f32(v[h][j + 2] & 0xFFFFu) * s;
        b[2 * j + 1] = bf16_to_f32(v[h][j + 2] >> 16) * s;
      }
      *(f32x4_t*)(out + 32 * h) = a;
      *(f32x4_t*)(out + 32 * h + 4) = b;
    }
  }
}

size_t quantized_weight_bytes(long long n_mats, int rows, int cols) {
  return (size_t)n_mats * rows * cols + (size_t)n_mats * rows * sizeof(float);
}

hipError_t launch_quantize_weights(const void* src, void* dst, long long n_mats, int rows, int cols, bool fp8,
                                   hipStream_t stream) {
  int8_t* codes = (int8_t*)dst;
  float* scale = (float*)(codes + (size_t)n_mats * rows * cols);
  const long long n_rows = n_mats * (long long)rows;
  if (fp8)
    hipLaunchKernelGGL(quant_row_scale_kernel<true>, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream,
                       (const uint16_t*)src, scale, n_rows, cols);
  else
    hipLaunchKernelGGL(quant_row_scale_kernel<false>, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream,
                       (const uint16_t*)src, scale, n_rows, cols);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long chunks = n_mats * (long long)rows * cols / 16;
  long long blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (fp8)
    hipLaunchKernelGGL(quant_pack_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)src,
                       (const float*)scale, codes, n_mats, rows, cols);
  else
    hipLaunchKernelGGL(quant_pack_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)src,
                       (const float*)scale, codes, n_mats, rows, cols);
  return hipGetLastError();
}

hipError_t launch_dequantize_weights(const void* src, int layout, float* dst, long long n_mats, int rows, int cols,
                                     hipStream_t stream) {
  const int8_t* codes = (const int8_t*)src;
  const float* scale = (const float*)(codes + (size_t)n_mats * rows * cols);
  const long long chunks = n_mats * (long long)rows * cols / 16;
  long long blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (layout == kFp8Frag)
    hipLaunchKernelGGL(dequant_kernel<kFp8Frag>, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scale, dst,
                       n_mats, rows, cols);
  else
    hipLaunchKernelGGL(dequant_kernel<kInt8Frag>, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scale, dst,
                       n_mats, rows, cols);
  return hipGetLastError();
}

}  // namespace moe

// One-time INT8 quantization of expert weights (MOE_LAYOUT_INT8_FRAG).
//
// Inference-optimisation chapter (fangpin.github.io, LLM-from-scratch ch. 6), model-compression
// part, second route ("make every byte cheaper"): decode reads every selected weight once, so one
// byte per weight instead of two halves the traffic; the affine code is x_q = round(x / s) + z.
// Sparse-MoE overview article (adg.csdn.net), section 4.3: INT8 expert weights for the same reason.
//
// Here: symmetric (z = 0), one scale per output channel (matrix row): s = max|w_row| / 127 and
// q = rint(w / s), both in float32 with IEEE division, so the codes are reproducible bit for bit.
// Codes are stored in the fragment order the streaming kernels read: every 1 KB is a 16-row x
// 64-column block; lane l of a wave holds row l % 16, columns 8 * (l / 16) .. +8 of the block's
// first 32 columns followed by the same 8 columns of its second 32, i.e. the bf16 16x16x32 MFMA
// A-operand chunks of two consecutive K steps. The float32 row scales follow all the codes.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

// one wave per row: the largest magnitude, then the scale (0 for an all-zero row)
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
  if (lane == 0) scale[row] = m / 127.0f;
}

__device__ __forceinline__ uint32_t quant4(uint32_t a, uint32_t b, float s) {
  // four bf16 values (two per word) -> four int8 codes, little-endian
  const float v[4] = {bf16_to_f32(a & 0xFFFFu), bf16_to_f32(a >> 16), bf16_to_f32(b & 0xFFFFu), bf16_to_f32(b >> 16)};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q = s > 0.f ? rintf(v[i] / s) : 0.f;
    q = fminf(fmaxf(q, -127.f), 127.f);
    out |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * i);
  }
  return out;
}

// one thread per 16-byte output chunk: chunk o is lane (o % 64) of 1 KB block (o / 64)
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
    const u32x4_t out = {quant4(lo[0], lo[1], s), quant4(lo[2], lo[3], s), quant4(hi[0], hi[1], s),
                         quant4(hi[2], hi[3], s)};
    *(u32x4_t*)(dst + (size_t)m * rows * cols + (size_t)q * 16) = out;
  }
}

size_t quantized_weight_bytes(long long n_mats, int rows, int cols) {
  return (size_t)n_mats * rows * cols + (size_t)n_mats * rows * sizeof(float);
}

hipError_t launch_quantize_weights(const void* src, void* dst, long long n_mats, int rows, int cols,
                                   hipStream_t stream) {
  int8_t* codes = (int8_t*)dst;
  float* scale = (float*)(codes + (size_t)n_mats * rows * cols);
  const long long n_rows = n_mats * (long long)rows;
  hipLaunchKernelGGL(quant_row_scale_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t*)src, scale, n_rows, cols);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long long chunks = n_mats * (long long)rows * cols / 16;
  long long blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(quant_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)src,
                     (const float*)scale, codes, n_mats, rows, cols);
  return hipGetLastError();
}

}  // namespace moe

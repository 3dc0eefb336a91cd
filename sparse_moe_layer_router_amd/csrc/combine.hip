// Combine: back to token order and weighted merge.
//
// Sparse-MoE overview article (adg.csdn.net), section 2.2 step 4: the layer output is the
// weighted sum of the selected experts' outputs; MoE-kernels page (blog.llmgo.top), section 1.1:
// the shared expert's output is added for every token; data-movement page, section 4: expert
// outputs are converted back to token order, weighted and merged.
//
// One block per token; each thread owns 8 consecutive features (one 16-byte bf16 load per row),
// gathers the token's k expert rows through inv_perm in fixed slot order, accumulates in fp32
// starting from the shared-expert row, and rounds once.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

template <int DT>
__global__ void __launch_bounds__(256)
combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ inv_perm, const float* __restrict__ w,
               const void* __restrict__ shared, void* __restrict__ out, int T, int k, int d) {
  const int t = blockIdx.x;
  const long long rows = (long long)T * k;
  for (int i = threadIdx.x * 8; i < d; i += 256 * 8) {
    float acc[8];
    if (shared) {
      if (DT == kBF16) {
        u32x4_t s = ld16((const uint16_t*)shared + (size_t)t * d + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) { acc[2 * q] = bf16_to_f32(s[q] & 0xFFFFu); acc[2 * q + 1] = bf16_to_f32(s[q] >> 16); }
      } else {
        const float* s = (const float*)shared + (size_t)t * d + i;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = s[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    }
    for (int j = 0; j < k; ++j) {
      long long r = inv_perm[(size_t)t * k + j];
      r = r < 0 ? 0 : (r >= rows ? rows - 1 : r);  // never read outside y, whatever the indices hold
      const float wj = w[(size_t)t * k + j];
      if (DT == kBF16) {
        u32x4_t v = ld16((const uint16_t*)y + (size_t)r * d + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += wj * bf16_to_f32(v[q] & 0xFFFFu);
          acc[2 * q + 1] += wj * bf16_to_f32(v[q] >> 16);
        }
      } else {
        const float* v = (const float*)y + (size_t)r * d + i;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wj * v[q];
      }
    }
    if (DT == kBF16) {
      u32x4_t o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      *(u32x4_t*)((uint16_t*)out + (size_t)t * d + i) = o;
    } else {
      float* o = (float*)out + (size_t)t * d + i;
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = acc[q];
    }
  }
}

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                          const void* shared_out, void* out, int T, int k, int d, hipStream_t stream) {
  if (dtype == kBF16)
    hipLaunchKernelGGL(combine_kernel<kBF16>, dim3(T), dim3(256), 0, stream, y_perm, inv_perm, topk_w, shared_out,
                       out, T, k, d);
  else
    hipLaunchKernelGGL(combine_kernel<kF32>, dim3(T), dim3(256), 0, stream, y_perm, inv_perm, topk_w, shared_out,
                       out, T, k, d);
  return hipGetLastError();
}

const char* combine_kernel_name(int dtype) { return dtype == kBF16 ? "combine_kernel<1>" : "combine_kernel<0>"; }

}  // namespace moe

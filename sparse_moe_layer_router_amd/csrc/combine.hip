// Combine: back to token order and weighted merge.
//
// Sparse-MoE overview article (adg.csdn.net), section 2.2 step 4: the layer output is the
// weighted sum of the selected experts' outputs; MoE-kernels page (blog.llmgo.top), section 1.1:
// the shared expert's output is added for every token; data-movement page, section 4: expert
// outputs are converted back to token order, weighted and merged.
//
// One block per token, a thread per 8 consecutive features (one 16-byte bf16 load per row); a
// block has up to 1024 threads for a few tokens and 256 for many, looping over the features. The
// token's k slots (inv_perm, weight) are read once into registers; for k <= 8 (kernels for k <= 2,
// 4 and 8) all k expert rows of a feature chunk (and the shared-expert row) are loaded before the
// first is used, so their latencies overlap. Accumulation is fp32 in fixed slot order starting from
// the shared-expert row, rounded once. Expert rows are loaded and bf16 outputs stored with the
// non-temporal hint: each is touched once here.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

namespace {

// NT: non-temporal load (the expert output rows are read exactly once)
template <int DT, bool NT = false>
__device__ __forceinline__ void load_row8(const void* base, size_t off, float (&v)[8]) {
  if (DT == kBF16) {
    const u32x4_t s = NT ? ld16_stream((const uint16_t*)base + off) : ld16((const uint16_t*)base + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) { v[2 * q] = bf16_to_f32(s[q] & 0xFFFFu); v[2 * q + 1] = bf16_to_f32(s[q] >> 16); }
  } else {
    const float* s = (const float*)base + off;
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = s[q];
  }
}

template <int DT>
__device__ __forceinline__ void store_row8(void* base, size_t off, const float (&acc)[8]) {
  if (DT == kBF16) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    __builtin_nontemporal_store(o, (u32x4_t*)((uint16_t*)base + off));
  } else {
    float* o = (float*)base + off;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = acc[q];
  }
}

}  // namespace

// KMAX > 0: k <= KMAX, slots held in registers and rows loaded together; KMAX = 0: any k.
template <int DT, int KMAX>
__global__ void __launch_bounds__(1024)
combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ inv_perm, const float* __restrict__ w,
               const void* __restrict__ shared, void* __restrict__ out, int T, int k, int d) {
  const int t = blockIdx.x;
  const long long rows = (long long)T * k;
  constexpr int KR = KMAX > 0 ? KMAX : 1;
  long long rr[KR];
  float wr[KR];
  // The slots come in with one vector load (lane j reads slot j) and are then broadcast from their
  // lanes. Slots past k repeat slot k - 1 (the same row, never added), so every row load below is
  // unconditional and the compiler issues them back to back: behind a branch per slot it waited for
  // each load before issuing the next.
  if (KMAX > 0) {
    const int lane = lane_id();
    const int js = lane < k ? lane : k - 1;
    int32_t rl = inv_perm[(size_t)t * k + js];
    rl = rl < 0 ? 0 : (rl >= rows ? (int32_t)(rows - 1) : rl);  // never read outside y, whatever the indices hold
    const float wl = w[(size_t)t * k + js];
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int src = j < k ? j : k - 1;
      rr[j] = __shfl(rl, src, 64);
      wr[j] = __shfl(wl, src, 64);
    }
  }
  for (int i = threadIdx.x * 8; i < d; i += blockDim.x * 8) {
    float acc[8];
    if (KMAX > 0) {
      float v[KR][8];
#pragma unroll
      for (int j = 0; j < KR; ++j) load_row8<DT, true>(y, (size_t)rr[j] * d + i, v[j]);
      if (shared) {
        load_row8<DT>(shared, (size_t)t * d + i, acc);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < KR; ++j)
        if (j < k)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += wr[j] * v[j][q];
    } else {
      if (shared) {
        load_row8<DT>(shared, (size_t)t * d + i, acc);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
      }
      for (int j = 0; j < k; ++j) {
        long long r = inv_perm[(size_t)t * k + j];
        r = r < 0 ? 0 : (r >= rows ? rows - 1 : r);
        const float wj = w[(size_t)t * k + j];
        float v[8];
        load_row8<DT, true>(y, (size_t)r * d + i, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += wj * v[q];
      }
    }
    store_row8<DT>(out, (size_t)t * d + i, acc);
  }
}

namespace {
template <int DT>
void launch_dt(const void* y_perm, const int32_t* inv_perm, const float* topk_w, const void* shared_out, void* out,
               int T, int k, int d, hipStream_t stream) {
  // few tokens: one pass over the features per block, as many lanes as chunks; many tokens: 256
  // threads per block, looping over the features, so that more blocks fit on a CU at once
  const int chunks = (d + 7) / 8;
  const int threads = T >= 1024 ? 256 : (chunks >= 1024 ? 1024 : (chunks + 63) / 64 * 64);
  if (k <= 2)
    hipLaunchKernelGGL((combine_kernel<DT, 2>), dim3(T), dim3(threads), 0, stream, y_perm, inv_perm, topk_w,
                       shared_out, out, T, k, d);
  else if (k <= 4)
    hipLaunchKernelGGL((combine_kernel<DT, 4>), dim3(T), dim3(threads), 0, stream, y_perm, inv_perm, topk_w,
                       shared_out, out, T, k, d);
  else if (k <= 8)
    hipLaunchKernelGGL((combine_kernel<DT, 8>), dim3(T), dim3(threads), 0, stream, y_perm, inv_perm, topk_w,
                       shared_out, out, T, k, d);
  else
    hipLaunchKernelGGL((combine_kernel<DT, 0>), dim3(T), dim3(threads), 0, stream, y_perm, inv_perm, topk_w,
                       shared_out, out, T, k, d);
}
}  // namespace

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                          const void* shared_out, void* out, int T, int k, int d, hipStream_t stream) {
  if (dtype == kBF16)
    launch_dt<kBF16>(y_perm, inv_perm, topk_w, shared_out, out, T, k, d, stream);
  else
    launch_dt<kF32>(y_perm, inv_perm, topk_w, shared_out, out, T, k, d, stream);
  return hipGetLastError();
}

const char* combine_kernel_name(int dtype, int k) {
  const bool b = dtype == kBF16;
  if (k <= 2) return b ? "combine_kernel<1, 2>" : "combine_kernel<0, 2>";
  if (k <= 4) return b ? "combine_kernel<1, 4>" : "combine_kernel<0, 4>";
  if (k <= 8) return b ? "combine_kernel<1, 8>" : "combine_kernel<0, 8>";
  return b ? "combine_kernel<1, 0>" : "combine_kernel<0, 0>";
}

}  // namespace moe

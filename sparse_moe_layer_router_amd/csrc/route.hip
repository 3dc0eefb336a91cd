// Router: scoring (logits = x . W_g^T + bias) and a wavefront-level top-k with softmax over the k.
//
// Sparse-MoE overview article (adg.csdn.net), section 2.2: each token is scored against every
// expert by a small linear layer, the E scores are ordered and the K best kept, and the K kept
// scores are softmax-normalised into weights that sum to one.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

// ------------------------------------------------------------------------------------- logits
// One wave per (token, expert): lanes stride the d axis 8 elements at a time, fp32 accumulate,
// deterministic butterfly reduction. Four experts per 256-thread block.
template <int DT>
__global__ void __launch_bounds__(256)
route_logits_valu(const void* __restrict__ x, const void* __restrict__ w, const float* __restrict__ bias,
                  float* __restrict__ logits, int T, int E, int d) {
  const int t = blockIdx.x;
  const int e = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (e >= E) return;
  float acc = 0.f;
  if (DT == kBF16) {
    const uint16_t* xr = (const uint16_t*)x + (size_t)t * d;
    const uint16_t* wr = (const uint16_t*)w + (size_t)e * d;
    for (int i = lane * 8; i < d; i += 64 * 8) {
      u32x4_t a = ld16(xr + i), b = ld16(wr + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc += bf16_to_f32(a[q] & 0xFFFFu) * bf16_to_f32(b[q] & 0xFFFFu);
        acc += bf16_to_f32(a[q] >> 16) * bf16_to_f32(b[q] >> 16);
      }
    }
  } else {
    const float* xr = (const float*)x + (size_t)t * d;
    const float* wr = (const float*)w + (size_t)e * d;
    for (int i = lane * 8; i < d; i += 64 * 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += xr[i + q] * wr[i + q];
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) logits[(size_t)t * E + e] = acc + (bias ? bias[e] : 0.f);
}

// ------------------------------------------------------------------------------------- top-k
// One wave per token. Lane l holds logits l, l+64, ... (E <= 1024 -> at most 16 per lane). Each
// of the k rounds takes the lane-local best not yet taken, then a butterfly arg-max over the
// wave with the order (value descending, index ascending); the winner is marked taken. The
// winning values stay in registers (slot s lives in lane s % 64) for the softmax.
constexpr int kMaxPerLane = 16;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
                  float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[kMaxPerLane];
  uint32_t taken = 0;
  const int nper = (E + 63) / 64;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    int e = lane + 64 * j;
    const bool ok = j < nper && e < E;
    const float val = ok ? row[e] : 0.f;
    v[j] = (val != val) ? -__builtin_inff() : val;  // NaN orders like -inf so k ids are always chosen
    if (!ok) taken |= 1u << j;
  }
  float sel[kMaxPerLane];  // selected value of slot s = lane + 64*j
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) sel[j] = 0.f;

  for (int s = 0; s < k; ++s) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      int e = lane + 64 * j;
      if (!((taken >> j) & 1u) && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if ((s & 63) == lane) {
      sel[s >> 6] = bv;  // s >> 6 < 16 because k <= E <= 1024
      topk_idx[(size_t)t * k + s] = bi;
    }
  }
  // softmax over the k selected, shifted by the largest (slot 0, held by lane 0)
  const float m = __shfl(sel[0], 0, 64);
  float ex[kMaxPerLane];
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    int s = lane + 64 * j;
    ex[j] = (s < k) ? expf(sel[j] - m) : 0.f;
    part += ex[j];
  }
  const float total = wave_sum(part);
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    int s = lane + 64 * j;
    if (s < k) topk_w[(size_t)t * k + s] = ex[j] / total;
  }
}

// ------------------------------------------------------------------------------------ launchers
hipError_t launch_route_logits(int dtype, const void* x, const void* w_router, const float* bias, float* logits,
                               int T, int E, int d, hipStream_t stream) {
  if (dtype == kBF16 && T >= kRouterGemmMinTokens) return launch_router_gemm(x, w_router, bias, logits, T, E, d, stream);
  dim3 grid(T, (E + 3) / 4), block(256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(route_logits_valu<kBF16>, grid, block, 0, stream, x, w_router, bias, logits, T, E, d);
  else
    hipLaunchKernelGGL(route_logits_valu<kF32>, grid, block, 0, stream, x, w_router, bias, logits, T, E, d);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream) {
  hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

const char* route_logits_kernel_name(int dtype, int T, int) {
  if (dtype == kBF16 && T >= kRouterGemmMinTokens) return "grouped_gemm_kernel<2, 0>";
  return dtype == kBF16 ? "route_logits_valu<1>" : "route_logits_valu<0>";
}
const char* route_topk_kernel_name() { return "route_topk_kernel"; }

}  // namespace moe

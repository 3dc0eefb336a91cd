// Measurement probes: a streaming read of HBM and a register-only bf16 MFMA loop, the two roofs the
// layer's kernels are compared with on the running part (inference-optimisation chapter, roofline
// section). Declared in include/moe_calib.h.
#include <hip/hip_runtime.h>

#include "../../include/moe_calib.h"
#include "moe_device.h"

namespace {

constexpr int kReadThreads = 256;
constexpr int kMfmaThreads = 512;
constexpr int kMfmaLdsBytes = 96 * 1024;   // more than half the LDS of a CU: one workgroup per CU

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <bool NT>
__device__ __forceinline__ u32x4_t load16(const u32x4_t* p) {
  if (NT) return __builtin_nontemporal_load(p);
  return *p;
}

// Workgroup b owns a contiguous share of the n16 16-byte units (a whole number of 1 KB chunks); its
// four waves read the share 1 KB per load (lane l the l-th 16 bytes), wave w the chunks w, w + 4,
// w + 8, ..., eight loads in flight per round, so the four waves of a workgroup read adjacent
// kilobytes at any moment. Of the patterns tried, a few long streams per compute unit (here two
// workgroups per unit, 2 MB per wave at 4 GiB) read fastest: on random data 2% above 8 K waves that
// each stream their own 512 KB. Every unit index stays below the share's end, which is at most n16.
template <bool NT>
__global__ void __launch_bounds__(kReadThreads) calib_read_kernel(const u32x4_t* __restrict__ buf, size_t n16,
                                                                  uint32_t* __restrict__ sink) {
  constexpr size_t kWaves = kReadThreads / 64, kStep = kWaves * 64;  // units between a wave's chunks
  const int lane = threadIdx.x & 63;
  const size_t share = ((n16 + gridDim.x - 1) / gridDim.x + 63) / 64 * 64;
  const size_t beg = (size_t)blockIdx.x * share < n16 ? (size_t)blockIdx.x * share : n16;
  const size_t end = beg + share < n16 ? beg + share : n16;
  uint32_t acc = 0;
  size_t i = beg + (size_t)(threadIdx.x >> 6) * 64 + lane;
  for (; i + 7 * kStep < end; i += 8 * kStep) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = load16<NT>(buf + i + j * kStep);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= fold(v[j]);
  }
  for (; i < end; i += kStep) acc ^= fold(load16<NT>(buf + i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  __shared__ uint32_t part[kWaves];
  if (lane == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Each wave: two operand fragments per lane loaded once, then iters x 8 independent 32x32x16 MFMAs,
// consecutive instructions taking the two fragments in swapped roles.
__global__ void __launch_bounds__(kMfmaThreads, 1) calib_mfma_kernel(const u32x4_t* __restrict__ ops, int iters,
                                                                     float* __restrict__ sink,
                                                                     uint64_t* __restrict__ clocks) {
  __shared__ float lds[kMfmaLdsBytes / 4];
  const int gl = blockIdx.x * kMfmaThreads + threadIdx.x;
  const u32x4_t a0 = ops[2 * gl], a1 = ops[2 * gl + 1];
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = (j & 1) ? moe::mfma32x32x16(a1, a0, acc[j]) : moe::mfma32x32x16(a0, a1, acc[j]);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  s = moe::wave_sum(s);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    lds[wave] = s;
    if (clocks) {
      uint64_t* c = clocks + 4 * ((size_t)blockIdx.x * (kMfmaThreads / 64) + wave);
      c[0] = t0;
      c[1] = r0;
      c[2] = t1;
      c[3] = r1;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int w = 0; w < kMfmaThreads / 64; ++w) tot += lds[w];
    sink[blockIdx.x] = tot;
  }
}

}  // namespace

extern "C" moe_status moe_calib_read_stream(const void* buf, size_t bytes, uint32_t* sink, int nontemporal,
                                            void* stream) {
  if (!buf || !sink || bytes == 0) return MOE_ERR_INVALID_ARG;
  if (bytes % 16 || (uintptr_t)buf % 16 || (uintptr_t)sink % 4) return MOE_ERR_ALIGNMENT;
  const size_t n16 = bytes / 16;
  if (nontemporal)
    hipLaunchKernelGGL(calib_read_kernel<true>, dim3(MOE_CALIB_READ_BLOCKS), dim3(kReadThreads), 0,
                       (hipStream_t)stream, (const u32x4_t*)buf, n16, sink);
  else
    hipLaunchKernelGGL(calib_read_kernel<false>, dim3(MOE_CALIB_READ_BLOCKS), dim3(kReadThreads), 0,
                       (hipStream_t)stream, (const u32x4_t*)buf, n16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status moe_calib_mfma(const void* operands, int32_t iters, float* sink, uint64_t* clocks,
                                     void* stream) {
  if (!operands || !sink || iters < 1) return MOE_ERR_INVALID_ARG;
  if ((uintptr_t)operands % 16 || (uintptr_t)sink % 4 || (uintptr_t)clocks % 8) return MOE_ERR_ALIGNMENT;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(MOE_CALIB_MFMA_BLOCKS), dim3(kMfmaThreads), 0, (hipStream_t)stream,
                     (const u32x4_t*)operands, iters, sink, clocks);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

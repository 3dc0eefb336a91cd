// One-time re-layout of expert weights into the fragment-tiled order (MOE_LAYOUT_FRAG16).
//
// Each 1 KB of the packed matrix is one 16-row x 32-column block in the A-operand lane order of
// the 16x16x32 bf16 MFMA, so a wave reading a weight for a matrix-core instruction reads 1 KB of
// contiguous memory instead of 16 separate 64-byte row pieces.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

// one thread per 16-byte output chunk: chunk o is lane (o % 64) of block (o / 64)
__global__ void __launch_bounds__(256)
pack_frag16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, long long n_mats, int rows,
                   int cols) {
  const long long per_mat = (long long)rows * cols / 8;  // 16-byte chunks per matrix
  const long long total = n_mats * per_mat;
  const int kb_per_band = cols / 32;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const long long m = o / per_mat;
    const long long q = o - m * per_mat;
    const long long blk = q / 64;
    const int lane = (int)(q % 64);
    const long long band = blk / kb_per_band;
    const int kb = (int)(blk % kb_per_band);
    const long long r = band * 16 + (lane & 15);
    const int c = kb * 32 + (lane >> 4) * 8;
    const u32x4_t v = ld16(src + (size_t)m * rows * cols + (size_t)r * cols + c);
    *(u32x4_t*)(dst + (size_t)m * rows * cols + (size_t)q * 8) = v;
  }
}

hipError_t launch_pack_weights(const void* src, void* dst, long long n_mats, int rows, int cols, hipStream_t stream) {
  const long long chunks = n_mats * (long long)rows * cols / 8;
  long long blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_frag16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)src,
                     (uint16_t*)dst, n_mats, rows, cols);
  return hipGetLastError();
}

}  // namespace moe

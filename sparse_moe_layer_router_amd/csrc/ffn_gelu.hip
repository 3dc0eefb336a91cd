// Two-layer GELU experts, the optional expert form of the sparse-MoE overview article
// (adg.csdn.net), section 4.1 layer code: every routed expert is Linear(d -> H) with a bias, GELU,
// Linear(H -> d) with a bias, applied to its own bucket of dispatched rows (MoE-kernels page,
// section 4.2: one launch over ragged groups given by an offsets array, empty experts skipped).
// GELU is the exact form z * Phi(z) = z * erfc(-z / sqrt 2) / 2.
//
// Both layers are one weight-streaming kernel (bf16, MFMA 16x16x32), the scheme of the SwiGLU
// decode kernels with a single matrix: block (nb, g) owns 64 consecutive output rows of group g's
// weight (4 waves x 16 rows); a wave streams its 16 weight rows once per pass, front to back, and
// applies each 16 x 32 fragment to 16 NTT tokens of the bucket (the B operand, from L2). The first
// layer gathers x rows through perm_src and stores GELU(acc + b1) as bf16 hidden rows [rows, H];
// the second reads those rows and stores acc + b2 as bf16 output rows [rows, d]. Accumulation is
// fp32 inside the MFMA; the bias is added in fp32 before the activation and the single rounding.
// A bucket of n rows streams its expert's weights ceil(n / 16 NTT) times, so this is the decode-regime
// form; layers with many rows per expert run the tiled grouped GEMM instead (ffn_gemm.hip, GELU
// modes). With one token tile the B loads are issued for every lane (rows past the bucket read its
// first row) and zeroed at the MFMA, so no load waits behind a per-lane branch; with two tiles the
// second is mostly past the bucket and its loads stay masked.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int kGeluRowsPerBlock = 64;  // 4 waves x 16 weight rows
constexpr int kGeluUnroll = 8;         // k-steps of 32 issued back to back

__device__ __forceinline__ float gelu_exact(float z) { return 0.5f * z * erfcf(-0.70710678118654752f * z); }

// Lane's weight source for the 16 rows [r0, r0 + 16) of a [rows, K] matrix; k-step s (32 columns)
// is at base + s * step elements. Row-major: row r0 + lane % 16 (rows past the matrix read the
// last row and are never stored), columns 8 (lane / 16) .. + 8 of the step; fragment-tiled: block
// (r0 / 16, s), one contiguous kilobyte per wave.
template <int LAYOUT>
__device__ __forceinline__ const uint16_t* weight_base(const void* wv, int r0, int rows, int K, int lane, int* step) {
  const uint16_t* w = (const uint16_t*)wv;
  if (LAYOUT == kFrag16) {
    *step = 512;
    return w + (size_t)(r0 / 16) * (K / 32) * 512 + lane * 8;
  }
  *step = 32;
  const int r = r0 + (lane & 15) < rows ? r0 + (lane & 15) : rows - 1;
  return w + (size_t)r * K + (lane >> 4) * 8;
}

}  // namespace

// UP: hid[r] = GELU(W1[g] . x[src(r)] + b1[g]);  !UP: y[r] = W2[g] . hid[r] + b2[g]
template <int NTT, int LAYOUT, bool UP>
__global__ void __launch_bounds__(256)
ffn_gelu_stream(const GeluGroups p) {
  const int g = blockIdx.y;
  long long a = p.offsets[g], b = p.offsets[g + 1];
  a = a < 0 ? 0 : (a > p.rows ? p.rows : a);  // never address outside the row buffers
  b = b < a ? a : (b > p.rows ? p.rows : b);
  const int n = (int)(b - a);
  if (n <= 0) return;
  const int N = UP ? p.H : p.d, K = UP ? p.d : p.H;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int n0 = blockIdx.x * kGeluRowsPerBlock + wave * 16;
  if (n0 >= N) return;
  const size_t wsz = (size_t)p.H * p.d;
  int ws = 0;
  const uint16_t* aw = weight_base<LAYOUT>((const uint16_t*)(UP ? p.w1 : p.w2) + (size_t)g * wsz, n0, N, K, lane, &ws);
  const float* bias = UP ? (p.b1 ? p.b1 + (size_t)g * p.H : nullptr) : (p.b2 ? p.b2 + (size_t)g * p.d : nullptr);
  const int ar = lane & 15, kq = lane >> 4;
  uint16_t* out = (uint16_t*)(UP ? p.hid : p.y);

  for (int tt = 0; tt < n; tt += 16 * NTT) {
    const uint16_t* bx[NTT];
    bool bok[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int rr = tt + j * 16 + ar;
      bok[j] = rr < n;
      long long src = a + (bok[j] ? rr : 0);
      if (UP && p.perm_src) {
        src = p.perm_src[src] / p.k;
        src = src < 0 ? 0 : (src >= p.T ? p.T - 1 : src);  // never read outside x
      }
      bx[j] = (const uint16_t*)(UP ? p.x : p.hid) + (size_t)src * K + kq * 8;
    }
    f32x4_t acc[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) acc[j] = f32x4_t{0, 0, 0, 0};
    const u32x4_t zero = {0, 0, 0, 0};
    int k0 = 0;
    for (; k0 + 32 * kGeluUnroll <= K; k0 += 32 * kGeluUnroll) {
      u32x4_t w[kGeluUnroll], x[kGeluUnroll][NTT];
#pragma unroll
      for (int s = 0; s < kGeluUnroll; ++s) w[s] = ld16_stream(aw + (size_t)(k0 / 32 + s) * ws);
#pragma unroll
      for (int s = 0; s < kGeluUnroll; ++s)
#pragma unroll
        for (int j = 0; j < NTT; ++j) x[s][j] = NTT == 1 || bok[j] ? ld16(bx[j] + k0 + 32 * s) : zero;
#pragma unroll
      for (int s = 0; s < kGeluUnroll; ++s)
#pragma unroll
        for (int j = 0; j < NTT; ++j) acc[j] = mfma16x16x32(w[s], bok[j] ? x[s][j] : zero, acc[j]);
    }
    for (; k0 < K; k0 += 32) {  // tail: K is a multiple of 8, so a lane's 8 columns are all in or all out
      const bool kok = k0 + kq * 8 < K;
      const u32x4_t w = kok ? ld16_stream(aw + (size_t)(k0 / 32) * ws) : zero;
#pragma unroll
      for (int j = 0; j < NTT; ++j) acc[j] = mfma16x16x32(w, (kok && bok[j]) ? ld16(bx[j] + k0) : zero, acc[j]);
    }
    // lane holds output columns c .. c + 3 (weight rows) of token row tt + 16 j + lane % 16
    const int c = n0 + kq * 4;
    if (c < N) {
      f32x4_t bc = {0.f, 0.f, 0.f, 0.f};
      if (bias) bc = f32x4_t{bias[c], bias[c + 1], bias[c + 2], bias[c + 3]};
#pragma unroll
      for (int j = 0; j < NTT; ++j) {
        const int rr = tt + j * 16 + ar;
        if (rr < n) {
          f32x4_t v = acc[j] + bc;
          if (UP) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_exact(v[e]);
          }
          *(u32x2_t*)(out + (size_t)(a + rr) * N + c) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
  }
}

namespace {
// two 16-token tiles per pass above 16 tokens (the weights of a bucket are streamed half as often)
int gelu_ntt(const GeluGroups& g) { return g.T > 16 ? 2 : 1; }

template <bool UP>
hipError_t launch_gelu(const GeluGroups& g, hipStream_t stream) {
  const int N = UP ? g.H : g.d;
  const dim3 grid((N + kGeluRowsPerBlock - 1) / kGeluRowsPerBlock, g.E);
  const bool two = gelu_ntt(g) == 2;
  if (g.layout == kFrag16 && two)
    hipLaunchKernelGGL((ffn_gelu_stream<2, kFrag16, UP>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFrag16)
    hipLaunchKernelGGL((ffn_gelu_stream<1, kFrag16, UP>), grid, dim3(256), 0, stream, g);
  else if (two)
    hipLaunchKernelGGL((ffn_gelu_stream<2, kRowMajor, UP>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((ffn_gelu_stream<1, kRowMajor, UP>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gelu_up(const GeluGroups& g, hipStream_t stream) { return launch_gelu<true>(g, stream); }
hipError_t launch_gelu_down(const GeluGroups& g, hipStream_t stream) { return launch_gelu<false>(g, stream); }

const char* gelu_kernel_name(const GeluGroups& g, bool up) {
  static const char* const names[2][2][2] = {
      {{"ffn_gelu_stream<1, 0, false>", "ffn_gelu_stream<1, 0, true>"},
       {"ffn_gelu_stream<1, 1, false>", "ffn_gelu_stream<1, 1, true>"}},
      {{"ffn_gelu_stream<2, 0, false>", "ffn_gelu_stream<2, 0, true>"},
       {"ffn_gelu_stream<2, 1, false>", "ffn_gelu_stream<2, 1, true>"}}};
  return names[gelu_ntt(g) == 2][g.layout == kFrag16][up ? 1 : 0];
}

}  // namespace moe

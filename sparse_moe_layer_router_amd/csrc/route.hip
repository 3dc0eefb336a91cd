// Router: scoring (logits = x . W_g^T + bias) and a wavefront-level top-k with softmax over the k.
//
// Sparse-MoE overview article (adg.csdn.net), section 2.2: each token is scored against every
// expert by a small linear layer, the E scores are ordered and the K best kept, and the K kept
// scores are softmax-normalised into weights that sum to one.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

// ------------------------------------------------------------------------------------- logits
// One wave per (token, expert): lanes stride the d axis 8 elements at a time, fp32 accumulate,
// deterministic butterfly reduction. Four experts per 256-thread block. The bf16 loads of kChunks
// consecutive strides are issued together before any of them is used, so a row of d = 7168 costs
// two memory round trips instead of fourteen (the sums keep the same order).
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
    constexpr int kChunks = 8;
    const uint16_t* xr = (const uint16_t*)x + (size_t)t * d;
    const uint16_t* wr = (const uint16_t*)w + (size_t)e * d;
    const u32x4_t zero = {0, 0, 0, 0};
    for (int i0 = lane * 8; i0 < d; i0 += 64 * 8 * kChunks) {
      u32x4_t a[kChunks], b[kChunks];
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int i = i0 + 64 * 8 * c;  // d is a multiple of 8: a lane's chunk is all in or all out
        a[c] = i < d ? ld16(xr + i) : zero;
        b[c] = i < d ? ld16(wr + i) : zero;
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        if (i0 + 64 * 8 * c >= d) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc += bf16_to_f32(a[c][q] & 0xFFFFu) * bf16_to_f32(b[c][q] & 0xFFFFu);
          acc += bf16_to_f32(a[c][q] >> 16) * bf16_to_f32(b[c][q] >> 16);
        }
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

// bf16: one block of four waves per tile of 16 experts x 16 tokens, as 16x16x32 MFMAs over d
// (A = 16 router rows, B = 16 token rows, lane l reading row l % 16 at k-chunk l / 16 of each
// 32-wide step, 16 bytes per lane). Every router row and token row is read once per tile, not once
// per (token, expert) pair. The four waves take consecutive quarters of the 32-wide k-steps and
// their partial sums are added in wave order through LDS (fixed order: the result does not depend
// on timing). Rows past E repeat a valid row and tokens past T read zeros; neither is stored. Lane
// l ends with experts 4 (l / 16) + i, i < 4, of token l % 16.
__global__ void __launch_bounds__(256)
route_logits_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias,
                  float* __restrict__ logits, int T, int E, int d) {
  constexpr int kU = 8;  // k-steps loaded back to back
  __shared__ f32x4_t part[3][64];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int ar = lane & 15, kq = lane >> 4;
  const int er = e0 + ar < E ? e0 + ar : E - 1;
  const bool tok = t0 + ar < T;
  const uint16_t* wa = w + (size_t)er * d + kq * 8;
  const uint16_t* xb = x + (size_t)(tok ? t0 + ar : 0) * d + kq * 8;
  const int nk = (d + 31) / 32, per = (nk + 3) / 4;
  const int kb = wave * per * 32, ke = (wave + 1) * per * 32 < d ? (wave + 1) * per * 32 : d;
  const u32x4_t zero = {0, 0, 0, 0};
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int k0 = kb;
  for (; k0 + 32 * kU <= ke; k0 += 32 * kU) {
    u32x4_t a[kU], b[kU];
#pragma unroll
    for (int s = 0; s < kU; ++s) a[s] = ld16(wa + k0 + 32 * s);
#pragma unroll
    for (int s = 0; s < kU; ++s) b[s] = tok ? ld16(xb + k0 + 32 * s) : zero;
#pragma unroll
    for (int s = 0; s < kU; ++s) acc = mfma16x16x32(a[s], b[s], acc);
  }
  for (; k0 < ke; k0 += 32) {  // d is a multiple of 8: a lane's 8-element chunk is all in or all out
    const bool kok = k0 + kq * 8 < d;
    const u32x4_t a = kok ? ld16(wa + k0) : zero;
    const u32x4_t b = (kok && tok) ? ld16(xb + k0) : zero;
    acc = mfma16x16x32(a, b, acc);
  }
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const f32x4_t p = part[q][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += p[i];
  }
  const int t = t0 + ar;
  if (t >= T) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + kq * 4 + i;
    if (e < E) logits[(size_t)t * E + e] = acc[i] + (bias ? bias[e] : 0.f);
  }
}

// ------------------------------------------------------------------------------------- top-k
// One wave per token. Lane l holds logits l, l+64, ... (NPER = ceil(E/64) <= 16 per lane). Each of
// the k rounds takes the lane-local best not yet taken, then the wave's largest value (a DPP
// max-reduction inside rows of 16 lanes, then across rows) and, among the lanes holding it, the
// smallest expert id (the same reduction on ids): the order is value descending, id ascending.
// The winner is marked taken; slot s's value and id stay in lane s % 64 for the softmax.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// max / min over the 64 lanes, result in every lane (DPP row ops, then row broadcasts, then lane 63)
template <bool MAX>
__device__ __forceinline__ int dpp_step(int v, int moved) {
  if (MAX) return __float_as_int(fmaxf(__int_as_float(v), __int_as_float(moved)));
  return v < moved ? v : moved;
}
template <bool MAX>
__device__ __forceinline__ int wave_reduce(int v) {
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));  // row_bcast:15 -> rows 1, 3
  v = dpp_step<MAX>(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));  // row_bcast:31 -> rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k and weights of one token's logits row by one wave. SIG = 0: ranks the logits (any logit
// bias is already inside them), weights = softmax over the k. SIG = 1: ranks sigmoid(l) + bias[e]
// (bias may be NULL), weights = the selected sigmoid(l) over their sum. Writes topk_idx/topk_w of
// the token (and, when lds_ids is not NULL, a copy of the ids into LDS).
template <int NPER, int SIG>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, const float* __restrict__ bias,
                                           int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* lds_ids,
                                           int lane) {
  float v[NPER];  // the score that decides the selection
  float a[NPER];  // sigmoid routing: the unbiased affinity that enters the weights
  uint32_t taken = 0;
  // every lane's scores (and biases) are loaded before any is used: from a clamped index, so the
  // loads need no branch and share one memory round trip
  float raw[NPER], rb[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int e = lane + 64 * j;
    raw[j] = row[e < E ? e : E - 1];
    rb[j] = (SIG && bias) ? bias[e < E ? e : E - 1] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int e = lane + 64 * j;
    const bool ok = e < E;
    const float val = ok ? raw[j] : 0.f;
    const bool nan = val != val;
    if (SIG) {
      a[j] = nan ? 0.f : 1.0f / (1.0f + expf(-val));
      v[j] = nan ? -__builtin_inff() : a[j] + (ok ? rb[j] : 0.f);
    } else {
      v[j] = nan ? -__builtin_inff() : val;  // NaN orders like -inf so k ids are always chosen
    }
    if (!ok) taken |= 1u << j;
  }
  float sel[NPER];  // weight source of slot s = lane + 64*j: its logit (softmax) or affinity (sigmoid)
#pragma unroll
  for (int j = 0; j < NPER; ++j) sel[j] = 0.f;

  for (int s = 0; s < k; ++s) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;  // no candidate left in this lane
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int e = lane + 64 * j;
      if (!((taken >> j) & 1u) && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
    const float m = __int_as_float(wave_reduce<true>(__float_as_int(bv)));
    const int win = wave_reduce<false>((bi != 0x7FFFFFFF && bv == m) ? bi : 0x7FFFFFFF);
    float src = m;
    if (SIG) {  // the winner's affinity, from the lane that holds it
      float mine = 0.f;
#pragma unroll
      for (int j = 0; j < NPER; ++j)
        if (j == (win >> 6)) mine = a[j];
      src = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), win & 63));
    }
    if ((win & 63) == lane) taken |= 1u << (win >> 6);
    if ((s & 63) == lane) {
      sel[s >> 6] = src;  // s >> 6 < NPER because k <= E
      idx_out[s] = win;
      if (lds_ids) lds_ids[s] = win;
    }
  }
  float ex[NPER];
  float part = 0.f;
  if (SIG) {
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      ex[j] = (lane + 64 * j < k) ? sel[j] : 0.f;
      part += ex[j];
    }
  } else {
    // softmax over the k selected, shifted by the largest (slot 0, held by lane 0)
    const float mx = __shfl(sel[0], 0, 64);
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      ex[j] = (lane + 64 * j < k) ? expf(sel[j] - mx) : 0.f;
      part += ex[j];
    }
  }
  const float total = wave_sum(part);
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int s = lane + 64 * j;
    if (s < k) w_out[s] = ex[j] / total;
  }
}

template <int NPER, int SIG>
__global__ void __launch_bounds__(256)
route_topk_kernel(const float* __restrict__ logits, int T, int E, int k, const float* __restrict__ bias,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<NPER, SIG>(logits + (size_t)t * E, E, k, bias, topk_idx + (size_t)t * k, topk_w + (size_t)t * k, nullptr,
                        lane_id());
}

// ------------------------------------------------------------------------------ small batches
// Decode-sized batches: one block of 16 waves does the top-k of every token (one wave per token,
// the routine above; at most 16 tokens), then the whole dispatch of the T*k slots from LDS: histogram, exclusive
// offsets, and the stable (expert, flat slot) permutation by one wave walking the slots in
// order, 64 at a time, lanes with equal expert ids ranked by ballots over the id bits. Same
// results, bit for bit, as route_topk_kernel followed by the three permute kernels.
constexpr int kTailWaves = 16;
static_assert(kSmallTailMaxTokens <= kTailWaves, "one token per wave");

template <int NPER, int SIG>
__global__ void __launch_bounds__(kTailWaves * 64)
route_tail_small_kernel(const float* __restrict__ logits, int T, int E, int k, const float* __restrict__ bias,
                        int32_t* __restrict__ topk_idx,
                        float* __restrict__ topk_w, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                        int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_perm) {
  __shared__ int32_t ids[kSmallTailMaxRows];
  __shared__ int32_t cur[1024];  // per-expert counts, then the next free row of each expert
  __shared__ int32_t wave_tot[kTailWaves];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kTailWaves)
    topk_token<NPER, SIG>(logits + (size_t)t * E, E, k, bias, topk_idx + (size_t)t * k, topk_w + (size_t)t * k,
                          ids + t * k, lane);
  for (int e = threadIdx.x; e < E; e += kTailWaves * 64) cur[e] = 0;
  __syncthreads();
  const int rows = T * k;
  for (int p = threadIdx.x; p < rows; p += kTailWaves * 64) atomicAdd(&cur[ids[p]], 1);
  __syncthreads();
  // exclusive scan of the counts over experts (one expert per thread, E <= 1024)
  const int e = threadIdx.x;
  const int32_t c = e < E ? cur[e] : 0;
  int32_t incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const int32_t excl = before + incl - c;
  if (e < E) {
    counts[e] = c;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + c;
    cur[e] = excl;
  }
  __syncthreads();
  if (wave != 0) return;
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < rows; c0 += 64) {
    const int p = c0 + lane;
    const int id = p < rows ? ids[p] : -1;
    const bool valid = id >= 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = valid && ((id >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int n = __popcll(same);
    const int32_t pos = valid ? cur[id] + rank : 0;
    __builtin_amdgcn_wave_barrier();  // every lane has read cur[] before the group's first lane bumps it
    if (valid && rank == 0) cur[id] += n;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      perm_src[pos] = p;
      inv_perm[p] = pos;
    }
  }
}

// ------------------------------------------------------------------------------------ launchers
hipError_t launch_route_logits(int dtype, const void* x, const void* w_router, const float* bias, float* logits,
                               int T, int E, int d, hipStream_t stream) {
  if (dtype == kBF16 && T >= kRouterGemmMinTokens) return launch_router_gemm(x, w_router, bias, logits, T, E, d, stream);
  if (dtype == kBF16 && T > kRouterValuMaxTokens) {
    hipLaunchKernelGGL(route_logits_mfma, dim3((E + 15) / 16, (T + 15) / 16), dim3(256), 0, stream,
                       (const uint16_t*)x, (const uint16_t*)w_router, bias, logits, T, E, d);
    return hipGetLastError();
  }
  dim3 grid(T, (E + 3) / 4), block(256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(route_logits_valu<kBF16>, grid, block, 0, stream, x, w_router, bias, logits, T, E, d);
  else
    hipLaunchKernelGGL(route_logits_valu<kF32>, grid, block, 0, stream, x, w_router, bias, logits, T, E, d);
  return hipGetLastError();
}

// candidates per lane for E experts: 1, 2, 4, 8 or 16
static int nper_of(int E) {
  int n = 1;
  while (64 * n < E) n *= 2;
  return n;
}

#define MOE_NPER_SWITCH(E, F, S) \
  switch (nper_of(E)) {          \
    case 1: F(1, S); break;      \
    case 2: F(2, S); break;      \
    case 4: F(4, S); break;      \
    case 8: F(8, S); break;      \
    default: F(16, S); break;    \
  }

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int routing, const float* score_bias,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream) {
#define MOE_TOPK(N, S)                                                                                 \
  hipLaunchKernelGGL((route_topk_kernel<N, S>), dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, \
                     score_bias, topk_idx, topk_w)
  if (routing == kRoutingSigmoid) {
    MOE_NPER_SWITCH(E, MOE_TOPK, 1)
  } else {
    MOE_NPER_SWITCH(E, MOE_TOPK, 0)
  }
#undef MOE_TOPK
  return hipGetLastError();
}

const char* route_logits_kernel_name(int dtype, int T, int) {
  if (dtype == kBF16 && T >= kRouterGemmMinTokens) return "grouped_gemm_kernel<2, 0>";
  if (dtype == kBF16 && T > kRouterValuMaxTokens) return "route_logits_mfma";
  return dtype == kBF16 ? "route_logits_valu<1>" : "route_logits_valu<0>";
}

bool route_tail_fused(int T, int k) { return T <= kSmallTailMaxTokens && (long long)T * k <= kSmallTailMaxRows; }

hipError_t launch_route_tail_small(const float* logits, int T, int E, int k, int routing, const float* score_bias,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* perm_src, int32_t* inv_perm, hipStream_t stream) {
#define MOE_TAIL(N, S)                                                                                           \
  hipLaunchKernelGGL((route_tail_small_kernel<N, S>), dim3(1), dim3(kTailWaves * 64), 0, stream, logits, T, E, k, \
                     score_bias, topk_idx, topk_w, counts, offsets, perm_src, inv_perm)
  if (routing == kRoutingSigmoid) {
    MOE_NPER_SWITCH(E, MOE_TAIL, 1)
  } else {
    MOE_NPER_SWITCH(E, MOE_TAIL, 0)
  }
#undef MOE_TAIL
  return hipGetLastError();
}

static const char* const kTopkNames[2][5] = {
    {"route_topk_kernel<1, 0>", "route_topk_kernel<2, 0>", "route_topk_kernel<4, 0>", "route_topk_kernel<8, 0>",
     "route_topk_kernel<16, 0>"},
    {"route_topk_kernel<1, 1>", "route_topk_kernel<2, 1>", "route_topk_kernel<4, 1>", "route_topk_kernel<8, 1>",
     "route_topk_kernel<16, 1>"}};
static const char* const kTailNames[2][5] = {
    {"route_tail_small_kernel<1, 0>", "route_tail_small_kernel<2, 0>", "route_tail_small_kernel<4, 0>",
     "route_tail_small_kernel<8, 0>", "route_tail_small_kernel<16, 0>"},
    {"route_tail_small_kernel<1, 1>", "route_tail_small_kernel<2, 1>", "route_tail_small_kernel<4, 1>",
     "route_tail_small_kernel<8, 1>", "route_tail_small_kernel<16, 1>"}};
static int nper_slot(int E) {
  int n = nper_of(E), i = 0;
  while ((1 << i) < n) ++i;
  return i;
}
const char* route_topk_kernel_name(int E, int routing) {
  return kTopkNames[routing == kRoutingSigmoid ? 1 : 0][nper_slot(E)];
}
const char* route_tail_small_kernel_name(int E, int routing) {
  return kTailNames[routing == kRoutingSigmoid ? 1 : 0][nper_slot(E)];
}

}  // namespace moe

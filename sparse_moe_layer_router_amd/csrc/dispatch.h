// Host-side launchers of the routing, dispatch, combine and weight-packing kernels. Every launcher
// enqueues on `stream` and returns the launch status; shapes were validated by the caller
// (moe_abi.cpp).
#pragma once

#include "kernels.h"

namespace moe {

// ---- routing -------------------------------------------------------------------------------
hipError_t launch_route_logits(int dtype, const void* x, const void* w_router, const float* bias,
                               float* logits, int T, int E, int d, hipStream_t stream);
// routing rule (moe_routing): softmax over the top-k logits, or sigmoid scores with a selection-only
// bias (score_bias [E] or NULL; unused by the softmax rule, whose bias is added to the logits)
enum Routing { kRoutingSoftmax = 0, kRoutingSigmoid = 1 };
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int routing, const float* score_bias,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream);
const char* route_logits_kernel_name(int dtype, int T, int E);
const char* route_topk_kernel_name(int E, int routing);

// Decode-sized batches (T <= 16 tokens, one per wave of the block; T*k <= 4096 slots): top-k,
// softmax and the whole dispatch (counts, offsets, perm_src, inv_perm) in one single-block launch
// after the logits. Each top-k is a chain of cross-lane exchanges, so more tokens per wave would
// serialize them; larger batches keep the one-wave-per-token kernel and the three permute kernels.
constexpr int kSmallTailMaxTokens = 16;
constexpr int kSmallTailMaxRows = 4096;
bool route_tail_fused(int T, int k);
hipError_t launch_route_tail_small(const float* logits, int T, int E, int k, int routing, const float* score_bias,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                                   int32_t* perm_src, int32_t* inv_perm, hipStream_t stream);
const char* route_tail_small_kernel_name(int E, int routing);

// ---- permutation ---------------------------------------------------------------------------
// Rows are cut into tiles of `tile` flat slots; `tile_counts` holds [n_tiles, E] int32.
int permute_tile_size(long long rows);
size_t permute_scratch_bytes(long long rows, int E);
hipError_t launch_permute_count(const int32_t* topk_idx, long long rows, int E, int tile, int32_t* tile_counts,
                                hipStream_t stream);
hipError_t launch_permute_scan(int32_t* tile_counts, long long rows, int E, int tile, int32_t* counts,
                               int32_t* offsets, hipStream_t stream);
hipError_t launch_permute_scatter(const int32_t* topk_idx, long long rows, int E, int tile,
                                  const int32_t* tile_counts, int32_t* perm_src, int32_t* inv_perm,
                                  hipStream_t stream);

// load statistics: load[e] = counts[e] / slots, aux = coef * sum_e (load[e] - 1/E)^2 (either output may be NULL)
hipError_t launch_load_stats(const int32_t* counts, int E, long long slots, float coef, float* load, float* aux,
                             hipStream_t stream);

// ---- combine ---------------------------------------------------------------------------------
hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                          const void* shared_out, void* out, int T, int k, int d, hipStream_t stream);
const char* combine_kernel_name(int dtype, int k);

// ---- two-layer GELU experts (bf16; row-major or fragment-tiled weights) ----------------------
// Routed groups 0..E-1 take rows [offsets[g], offsets[g+1]) of the dispatched order (source token
// perm_src[r] / k, or row r of x when perm_src is NULL). hid[r] = GELU(W1[g] x + b1[g]) (bf16,
// [rows, H] row-major), y[r] = W2[g] hid[r] + b2[g] (bf16, [rows, d]); a NULL bias is zero.
struct GeluGroups {
  int layout;              // kRowMajor or kFrag16
  int d, E, k, H, T;
  long long rows;          // T*k
  const int32_t* offsets;  // [E+1]
  const int32_t* perm_src; // [rows] or NULL
  const void* x;           // [T, d] (or [rows, d] when perm_src is NULL)
  const void* w1;          // [E, H, d]
  const float* b1;         // [E, H] or NULL
  const void* w2;          // [E, d, H]
  const float* b2;         // [E, d] or NULL
  void* hid;               // [rows, H]
  void* y;                 // [rows, d]
};
hipError_t launch_gelu_up(const GeluGroups& g, hipStream_t stream);
hipError_t launch_gelu_down(const GeluGroups& g, hipStream_t stream);
const char* gelu_kernel_name(const GeluGroups& g, bool up);

// ---- weight packing (MOE_LAYOUT_FRAG16) and INT8 / FP8 quantization (MOE_LAYOUT_INT8_FRAG / FP8_FRAG) ----
hipError_t launch_pack_weights(const void* src, void* dst, long long n_mats, int rows, int cols, hipStream_t stream);
size_t quantized_weight_bytes(long long n_mats, int rows, int cols);
hipError_t launch_quantize_weights(const void* src, void* dst, long long n_mats, int rows, int cols, bool fp8,
                                   hipStream_t stream);
hipError_t launch_dequantize_weights(const void* src, int layout, float* dst, long long n_mats, int rows, int cols,
                                     hipStream_t stream);

}  // namespace moe

// Host-side launchers of the expert (FFN) kernels and the types they share with the rest of the
// library. Every launcher enqueues on `stream` and returns the launch status; shapes were
// validated by the caller (moe_abi.cpp). Routing, dispatch, combine and weight packing are
// declared in dispatch.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Largest expert count the kernels handle (the C ABI rejects more).
constexpr int kMaxExperts = 1024;

enum Dtype { kF32 = 0, kBF16 = 1 };

// ---- grouped SwiGLU experts ------------------------------------------------------------------
// A set of expert groups: routed groups 0..E-1 take rows [offsets[g], offsets[g+1]) of the
// dispatched order (source token perm_src[r] / k, or r when perm_src is NULL); the optional
// shared group (index E) takes rows [shared_row0, shared_row0 + T) with source token r - row0.
enum WeightLayout { kRowMajor = 0, kFrag16 = 1, kInt8Frag = 2, kFp8Frag = 3 };
// One-byte weight codes (INT8 or FP8 E4M3) in the same fragment order, with float32 row scales.
__host__ __device__ constexpr bool byte_codes(int layout) { return layout == kInt8Frag || layout == kFp8Frag; }

// Offset (elements) of element (r, c) of a [rows, cols] matrix in the fragment-tiled layout:
// 16 x 32 blocks along each 16-row band; inside a block, 64 lanes x 8 consecutive columns in the
// A-operand order of the 16x16x32 MFMA (lane = r%16 + 16 * ((c%32)/8)).
__host__ __device__ inline size_t frag16_offset(size_t r, size_t c, size_t cols) {
  return ((r / 16) * (cols / 32) + c / 32) * 512 + ((r % 16) + 16 * ((c % 32) / 8)) * 8 + c % 8;
}


struct FfnGroups {
  int dtype;
  int layout;                  // WeightLayout of the expert weights
  int d;                       // model width
  int E;                       // routed groups
  int k;                       // slots per token (perm_src divisor)
  int H;                       // routed hidden size
  long long rows;              // routed rows (T*k)
  const int32_t* offsets;      // [E+1]
  const int32_t* perm_src;     // [rows] or NULL
  const void* x;               // [T, d] (or [rows, d] when perm_src is NULL)
  const void* w_gate;          // [E, H, d]
  const void* w_up;            // [E, H, d]
  const void* w_down;          // [E, d, H]
  // shared expert (Hs == 0: none)
  int Hs;
  int T;
  const void* ws_gate;         // [Hs, d]
  const void* ws_up;           // [Hs, d]
  const void* ws_down;         // [d, Hs]
  // outputs
  void* hid;                   // hidden activations (dtype): routed [rows, H], then shared [T, Hs]; on the
                               // grouped-GEMM path in the packed layout described below instead
  void* y;                     // routed outputs [rows, d], then shared outputs [T, d] (dtype)
  float mean_rows_per_group;   // host-side regime hint (T*k / E)
  long long rbands;            // grouped-GEMM path: routed band capacity of the packed hidden activations
  // Two-layer GELU experts on the grouped-GEMM path (gelu = 1): w_gate holds W1 [E, H, d], w_down
  // W2 [E, d, H], w_up is unused, Hs = 0; hid = GELU(W1 x + b1), y = W2 hid + b2 (a NULL bias is zero)
  int gelu;
  const float* b1;             // [E, H] or NULL
  const float* b2;             // [E, d] or NULL
};

// Grouped-GEMM path: the hidden activations are packed into 16-row x 32-column blocks
// (frag16_offset order, columns padded to a multiple of 32 with zeros), the layout the down pass
// loads as contiguous kilobytes. Every routed group starts on a 16-row band: group g owns bands
// [pband[g], pband[g] + ceil(n_g / 16)) of the routed region, which holds `rbands` bands; the
// shared group's T rows follow in a region of their own.
__host__ __device__ inline long long gemm_pad32(long long v) { return (v + 31) / 32 * 32; }
__host__ __device__ inline long long gemm_routed_bands(long long rows, int E) { return (rows + 15) / 16 + E; }
__host__ __device__ inline long long gemm_hid_elems(long long rows, int E, int T, int H, int Hs) {
  return gemm_routed_bands(rows, E) * 16 * gemm_pad32(H) + (Hs > 0 ? (long long)(T + 15) / 16 * 16 * gemm_pad32(Hs) : 0);
}

// Which kernels run the experts, chosen from shapes only (no device data):
//   kPathF32    float32 layers: plain VALU kernels;
//   kPathStream bf16, few rows per expert (decode): weight-streaming MFMA GEMV, every weight read once;
//   kPathGemm   bf16, many rows per expert (prefill): tiled MFMA grouped GEMM with a tile schedule.
enum FfnPath { kPathF32 = 0, kPathStream = 1, kPathGemm = 2 };
constexpr float kGemmMinRowsPerExpert = 32.f;
FfnPath ffn_path(const FfnGroups& g);

hipError_t launch_ffn_gate_up_stream(const FfnGroups& g, hipStream_t stream);
hipError_t launch_ffn_down_stream(const FfnGroups& g, hipStream_t stream);
hipError_t launch_ffn_gate_up_f32(const FfnGroups& g, hipStream_t stream);
hipError_t launch_ffn_down_f32(const FfnGroups& g, hipStream_t stream);

// grouped GEMM: `sched` holds gemm_schedule_ints(E) int32 (tile prefix sums of both passes, the
// routed groups' first bands of the packed hidden activations, and each pass's per-XCD tile ranges)
size_t gemm_schedule_ints(int E);
hipError_t launch_gemm_schedule(const FfnGroups& g, int32_t* sched, hipStream_t stream);
hipError_t launch_gemm_gate_up(const FfnGroups& g, const int32_t* sched, hipStream_t stream);
hipError_t launch_gemm_down(const FfnGroups& g, const int32_t* sched, hipStream_t stream);

// dense router GEMM (bf16, large T): logits = x . w^T + bias
constexpr int kRouterGemmMinTokens = 2048;
// bf16 router logits: one wave per (token, expert) up to this many tokens, MFMA tiles of 16 x 16 above
constexpr int kRouterValuMaxTokens = 16;
hipError_t launch_router_gemm(const void* x, const void* w, const float* bias, float* logits, int T, int E, int d,
                              hipStream_t stream);

const char* ffn_schedule_kernel_name(const FfnGroups& g);
const char* ffn_gate_up_kernel_name(const FfnGroups& g);
const char* ffn_down_kernel_name(const FfnGroups& g);

}  // namespace moe

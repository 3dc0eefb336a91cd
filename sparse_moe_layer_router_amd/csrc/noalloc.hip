// moe_layer_forward without a workspace argument, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
// layer's intermediates (logits, ids, weights, permutation, tile schedule, hidden activations,
// expert outputs) live in one file-scope device array of fixed size instead of a caller buffer.
//
// Each GPU holds its own copy of the array for the life of the process. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the device symbol): the first
// call on a device, with that device current, looks up that device's address of the array with
// hipGetSymbolAddress and keeps it; every launch takes that address. Nothing in the array needs
// to start at zero: the layer writes every byte it reads earlier in the same call. All calls on
// one GPU share the array, so calls that overlap on one GPU (two streams, two threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "the header states the same limit");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// The calling thread's current device, which must also be the device of `stream`.
moe_status current_device(hipStream_t stream, int* dev) {
  if (hipGetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
  if (*dev < 0 || *dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_ERR_HIP;
    if (sdev != *dev) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

// This device's address of `scratch`, looked up once per device (with that device current).
moe_status scratch_of(int dev, void** out) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
  });
  if (g_lookup[dev] != hipSuccess || !g_scratch[dev]) return MOE_ERR_HIP;
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* w_router,
                                                const float* logit_bias, const void* w_gate, const void* w_up,
                                                const void* w_down, const void* w_shared_gate,
                                                const void* w_shared_up, const void* w_shared_down, void* out,
                                                int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                                float* logits_out, void* stream) {
  const size_t need = moe_workspace_bytes(s);
  if (need == 0) return MOE_ERR_INVALID_ARG;  // invalid shape (every valid shape needs some bytes)
  if (s->T == 0) return MOE_OK;
  if (need > kScratchBytes) return MOE_ERR_TOO_LARGE;
  int dev = -1;
  moe_status st = current_device((hipStream_t)stream, &dev);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_of(dev, &ws);
  if (st != MOE_OK) return st;
  return moe_layer_forward(s, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                           w_shared_down, out, topk_idx_out, topk_w_out, counts_out, logits_out, ws, kScratchBytes,
                           stream);
}

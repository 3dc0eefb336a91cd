// C ABI of the MoE layer: host-side validation, workspace layout and kernel orchestration.
// Nothing here allocates, synchronizes or copies device memory; every launch goes on the caller's
// stream. Validation completes before the first launch, so an error enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/moe.h"
#include "dispatch.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t logits, topk_idx, topk_w, counts, offsets, perm_src, inv_perm, tile_counts, sched, hid, y, total;
};

size_t elem_size(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

Layout layout_of(const moe_shape& s) {
  const size_t T = (size_t)s.T, E = (size_t)s.n_experts, k = (size_t)s.top_k;
  const size_t rows = T * k, d = (size_t)s.d_model, H = (size_t)s.d_hidden, Hs = (size_t)s.d_shared_hidden;
  const size_t es = elem_size(s.dtype);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  L.logits = take(T * E * 4);
  L.topk_idx = take(rows * 4);
  L.topk_w = take(rows * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm_src = take(rows * 4);
  L.inv_perm = take(rows * 4);
  L.tile_counts = take(moe::permute_scratch_bytes((long long)rows, (int)E));
  L.sched = take(moe::gemm_schedule_ints((int)E) * 4);
  // the grouped-GEMM path keeps its hidden activations in the packed layout
  moe::FfnGroups shape_only{};
  shape_only.dtype = s.dtype;
  shape_only.layout = s.weight_layout;
  shape_only.mean_rows_per_group = (float)((double)s.T * s.top_k / s.n_experts);
  const bool gemm = moe::ffn_path(shape_only) == moe::kPathGemm;
  size_t hid_elems = rows * H + (Hs ? T * Hs : 0);
  if (gemm) {
    const size_t packed = (size_t)moe::gemm_hid_elems((long long)rows, (int)E, (int)T, (int)H, (int)Hs);
    hid_elems = packed > hid_elems ? packed : hid_elems;
  }
  L.hid = take(hid_elems * es);
  L.y = take((rows + (Hs ? T : 0)) * d * es);
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->T < 0 || s->d_model < 1 || s->n_experts < 1 || s->top_k < 1 || s->d_hidden < 1 || s->d_shared_hidden < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
  if (s->n_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((long long)s->T * s->top_k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (s->d_model % 8 || s->d_hidden % 8 || s->d_shared_hidden % 8) return MOE_ERR_ALIGNMENT;
  if (s->weight_layout != MOE_LAYOUT_ROWMAJOR && s->weight_layout != MOE_LAYOUT_FRAG16 &&
      s->weight_layout != MOE_LAYOUT_INT8_FRAG && s->weight_layout != MOE_LAYOUT_FP8_FRAG)
    return MOE_ERR_UNSUPPORTED;
  if (s->routing != MOE_ROUTING_SOFTMAX && s->routing != MOE_ROUTING_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (s->weight_layout == MOE_LAYOUT_FRAG16) {
    // every expert matrix ([H, d], [d, H], [Hs, d], [d, Hs]) must tile into 16 x 32 blocks
    if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (s->d_model % 32 || s->d_hidden % 32 || s->d_shared_hidden % 32) return MOE_ERR_ALIGNMENT;
  }
  if (s->weight_layout == MOE_LAYOUT_INT8_FRAG || s->weight_layout == MOE_LAYOUT_FP8_FRAG) {
    // every expert matrix tiles into 16 x 64 blocks of codes
    if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (s->d_model % 64 || s->d_hidden % 64 || s->d_shared_hidden % 64) return MOE_ERR_ALIGNMENT;
  }
  return MOE_OK;
}

// required device pointer with the given alignment
moe_status need(const void* p, size_t a) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return aligned(p, a) ? MOE_OK : MOE_ERR_ALIGNMENT;
}
// optional device pointer (NULL allowed)
moe_status maybe(const void* p, size_t a) { return (!p || aligned(p, a)) ? MOE_OK : MOE_ERR_ALIGNMENT; }

#define MOE_TRY(expr)                      \
  do {                                     \
    moe_status st_ = (expr);               \
    if (st_ != MOE_OK) return st_;         \
  } while (0)

#define MOE_LAUNCH(expr)                   \
  do {                                     \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

moe_status check_workspace(const moe_shape& s, void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, kAlign)) return MOE_ERR_ALIGNMENT;
  return ws_bytes >= layout_of(s).total ? MOE_OK : MOE_ERR_WORKSPACE;
}

// Stage event recording for the timed variant.
struct Events {
  void* const* ev;
  hipStream_t stream;
  bool mark(int stage, int end) const {
    if (!ev) return true;
    void* e = ev[2 * stage + end];
    if (!e) return true;
    return hipEventRecord((hipEvent_t)e, stream) == hipSuccess;
  }
};

#define MOE_MARK(E_, stage, end)            \
  do {                                      \
    if (!(E_).mark((stage), (end))) return MOE_ERR_HIP; \
  } while (0)

char* at(void* base, size_t off) { return (char*)base + off; }

moe_status route_impl(const moe_shape& s, const void* x, const void* w_router, const float* bias, float* logits,
                      int32_t* idx, float* w, const Events& ev, hipStream_t stream) {
  const bool sig = s.routing == MOE_ROUTING_SIGMOID;
  MOE_MARK(ev, MOE_STAGE_ROUTE_LOGITS, 0);
  MOE_LAUNCH(moe::launch_route_logits(s.dtype, x, w_router, sig ? nullptr : bias, logits, s.T, s.n_experts,
                                      s.d_model, stream));
  MOE_MARK(ev, MOE_STAGE_ROUTE_LOGITS, 1);
  MOE_MARK(ev, MOE_STAGE_ROUTE_TOPK, 0);
  MOE_LAUNCH(moe::launch_route_topk(logits, s.T, s.n_experts, s.top_k, s.routing, sig ? bias : nullptr, idx, w,
                                    stream));
  MOE_MARK(ev, MOE_STAGE_ROUTE_TOPK, 1);
  return MOE_OK;
}

moe_status permute_impl(const moe_shape& s, const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                        int32_t* inv_perm, int32_t* tile_counts, const Events& ev, hipStream_t stream) {
  const long long rows = (long long)s.T * s.top_k;
  const int tile = moe::permute_tile_size(rows);
  MOE_MARK(ev, MOE_STAGE_PERMUTE_COUNT, 0);
  MOE_LAUNCH(moe::launch_permute_count(idx, rows, s.n_experts, tile, tile_counts, stream));
  MOE_MARK(ev, MOE_STAGE_PERMUTE_COUNT, 1);
  MOE_MARK(ev, MOE_STAGE_PERMUTE_SCAN, 0);
  MOE_LAUNCH(moe::launch_permute_scan(tile_counts, rows, s.n_experts, tile, counts, offsets, stream));
  MOE_MARK(ev, MOE_STAGE_PERMUTE_SCAN, 1);
  MOE_MARK(ev, MOE_STAGE_PERMUTE_SCATTER, 0);
  MOE_LAUNCH(moe::launch_permute_scatter(idx, rows, s.n_experts, tile, tile_counts, perm_src, inv_perm, stream));
  MOE_MARK(ev, MOE_STAGE_PERMUTE_SCATTER, 1);
  return MOE_OK;
}

moe::FfnGroups groups_for(const moe_shape& s, const void* x, const int32_t* perm_src, const int32_t* offsets,
                          const void* wg, const void* wu, const void* wd, const void* sg, const void* su,
                          const void* sd, void* hid, void* y) {
  moe::FfnGroups g{};
  g.dtype = s.dtype;
  g.layout = s.weight_layout;
  g.d = s.d_model;
  g.E = s.n_experts;
  g.k = s.top_k;
  g.H = s.d_hidden;
  g.rows = (long long)s.T * s.top_k;
  g.offsets = offsets;
  g.perm_src = perm_src;
  g.x = x;
  g.w_gate = wg;
  g.w_up = wu;
  g.w_down = wd;
  g.Hs = s.d_shared_hidden;
  g.T = s.T;
  g.ws_gate = sg;
  g.ws_up = su;
  g.ws_down = sd;
  g.hid = hid;
  g.y = y;
  g.mean_rows_per_group = (float)((double)s.T * s.top_k / s.n_experts);
  g.rbands = moe::gemm_routed_bands(g.rows, g.E);
  return g;
}

moe::GeluGroups gelu_groups_for(const moe_shape& s, const void* x, const int32_t* perm_src, const int32_t* offsets,
                                const void* w1, const float* b1, const void* w2, const float* b2, void* hid,
                                void* y) {
  moe::GeluGroups g{};
  g.layout = s.weight_layout;
  g.d = s.d_model;
  g.E = s.n_experts;
  g.k = s.top_k;
  g.H = s.d_hidden;
  g.T = s.T;
  g.rows = (long long)s.T * s.top_k;
  g.offsets = offsets;
  g.perm_src = perm_src;
  g.x = x;
  g.w1 = w1;
  g.b1 = b1;
  g.w2 = w2;
  g.b2 = b2;
  g.hid = hid;
  g.y = y;
  return g;
}

// The GELU experts as grouped-GEMM groups: W1 in the gate slot, W2 in the down slot, no shared expert.
moe::FfnGroups gelu_gemm_groups(const moe_shape& s, const void* x, const int32_t* perm_src, const int32_t* offsets,
                                const void* w1, const float* b1, const void* w2, const float* b2, void* hid, void* y) {
  moe_shape routed = s;
  routed.d_shared_hidden = 0;
  moe::FfnGroups g = groups_for(routed, x, perm_src, offsets, w1, nullptr, w2, nullptr, nullptr, nullptr, hid, y);
  g.gelu = 1;
  g.b1 = b1;
  g.b2 = b2;
  return g;
}

moe_status ffn_impl(const moe::FfnGroups& g, int32_t* sched, const Events& ev, hipStream_t stream) {
  const moe::FfnPath path = moe::ffn_path(g);
  MOE_MARK(ev, MOE_STAGE_FFN_SCHEDULE, 0);
  if (path == moe::kPathGemm) {
    MOE_LAUNCH(moe::launch_gemm_schedule(g, sched, stream));
  }
  MOE_MARK(ev, MOE_STAGE_FFN_SCHEDULE, 1);
  MOE_MARK(ev, MOE_STAGE_FFN_GATE_UP, 0);
  switch (path) {
    case moe::kPathF32: MOE_LAUNCH(moe::launch_ffn_gate_up_f32(g, stream)); break;
    case moe::kPathStream: MOE_LAUNCH(moe::launch_ffn_gate_up_stream(g, stream)); break;
    case moe::kPathGemm: MOE_LAUNCH(moe::launch_gemm_gate_up(g, sched, stream)); break;
  }
  MOE_MARK(ev, MOE_STAGE_FFN_GATE_UP, 1);
  MOE_MARK(ev, MOE_STAGE_FFN_DOWN, 0);
  switch (path) {
    case moe::kPathF32: MOE_LAUNCH(moe::launch_ffn_down_f32(g, stream)); break;
    case moe::kPathStream: MOE_LAUNCH(moe::launch_ffn_down_stream(g, stream)); break;
    case moe::kPathGemm: MOE_LAUNCH(moe::launch_gemm_down(g, sched, stream)); break;
  }
  MOE_MARK(ev, MOE_STAGE_FFN_DOWN, 1);
  return MOE_OK;
}

moe_status layer_impl(const moe_shape* sp, const void* x, const void* w_router, const float* bias, const void* wg,
                      const void* wu, const void* wd, const void* sg, const void* su, const void* sd, void* out,
                      int32_t* idx_out, float* w_out, int32_t* counts_out, float* logits_out, void* ws,
                      size_t ws_bytes, void* stream_p, void* const* events) {
  MOE_TRY(check_shape(sp));
  const moe_shape& s = *sp;
  if (s.T == 0) return MOE_OK;  // nothing to read or write: empty tensors may have NULL pointers
  const size_t va = 16;
  MOE_TRY(need(x, va));
  MOE_TRY(need(w_router, va));
  MOE_TRY(maybe(bias, 4));
  MOE_TRY(need(wg, va));
  MOE_TRY(need(wu, va));
  MOE_TRY(need(wd, va));
  if (s.d_shared_hidden > 0) {
    MOE_TRY(need(sg, va));
    MOE_TRY(need(su, va));
    MOE_TRY(need(sd, va));
  }
  MOE_TRY(need(out, va));
  MOE_TRY(maybe(idx_out, 4));
  MOE_TRY(maybe(w_out, 4));
  MOE_TRY(maybe(counts_out, 4));
  MOE_TRY(maybe(logits_out, 4));
  MOE_TRY(check_workspace(s, ws, ws_bytes));

  hipStream_t stream = (hipStream_t)stream_p;
  const Events ev{events, stream};
  const Layout L = layout_of(s);
  float* logits = logits_out ? logits_out : (float*)at(ws, L.logits);
  int32_t* idx = idx_out ? idx_out : (int32_t*)at(ws, L.topk_idx);
  float* w = w_out ? w_out : (float*)at(ws, L.topk_w);
  int32_t* counts = counts_out ? counts_out : (int32_t*)at(ws, L.counts);
  int32_t* offsets = (int32_t*)at(ws, L.offsets);
  int32_t* perm_src = (int32_t*)at(ws, L.perm_src);
  int32_t* inv_perm = (int32_t*)at(ws, L.inv_perm);
  int32_t* tiles = (int32_t*)at(ws, L.tile_counts);
  void* hid = at(ws, L.hid);
  void* y = at(ws, L.y);

  if (moe::route_tail_fused(s.T, s.top_k)) {
    // decode-sized batch: top-k, softmax and the dispatch in one launch after the logits
    const bool sig = s.routing == MOE_ROUTING_SIGMOID;
    MOE_MARK(ev, MOE_STAGE_ROUTE_LOGITS, 0);
    MOE_LAUNCH(moe::launch_route_logits(s.dtype, x, w_router, sig ? nullptr : bias, logits, s.T, s.n_experts,
                                        s.d_model, stream));
    MOE_MARK(ev, MOE_STAGE_ROUTE_LOGITS, 1);
    MOE_MARK(ev, MOE_STAGE_ROUTE_TOPK, 0);
    MOE_LAUNCH(moe::launch_route_tail_small(logits, s.T, s.n_experts, s.top_k, s.routing, sig ? bias : nullptr, idx,
                                            w, counts, offsets, perm_src, inv_perm, stream));
    MOE_MARK(ev, MOE_STAGE_ROUTE_TOPK, 1);
    for (int st = MOE_STAGE_PERMUTE_COUNT; st <= MOE_STAGE_PERMUTE_SCATTER; ++st) {
      MOE_MARK(ev, st, 0);
      MOE_MARK(ev, st, 1);
    }
  } else {
    MOE_TRY(route_impl(s, x, w_router, bias, logits, idx, w, ev, stream));
    MOE_TRY(permute_impl(s, idx, counts, offsets, perm_src, inv_perm, tiles, ev, stream));
  }
  const moe::FfnGroups g = groups_for(s, x, perm_src, offsets, wg, wu, wd, sg, su, sd, hid, y);
  MOE_TRY(ffn_impl(g, (int32_t*)at(ws, L.sched), ev, stream));
  const void* shared_out =
      s.d_shared_hidden > 0 ? (const void*)((const char*)y + (size_t)s.T * s.top_k * s.d_model * elem_size(s.dtype))
                            : nullptr;
  MOE_MARK(ev, MOE_STAGE_COMBINE, 0);
  MOE_LAUNCH(moe::launch_combine(s.dtype, y, inv_perm, w, shared_out, out, s.T, s.top_k, s.d_model, stream));
  MOE_MARK(ev, MOE_STAGE_COMBINE, 1);
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return layout_of(*s).total;
}

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case MOE_ERR_ALIGNMENT: return "misaligned size or pointer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_TOO_LARGE: return "shape needs more than the fixed no-allocation scratch";
  }
  return "unknown status";
}

moe_status moe_pack_weights(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols, void* stream) {
  if (n_mats < 0 || rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (rows % 16 || cols % 32) return MOE_ERR_ALIGNMENT;
  if (n_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
  MOE_TRY(need(src, 16));
  MOE_TRY(need(dst, 16));
  const uintptr_t bytes = (uintptr_t)n_mats * (uintptr_t)rows * (uintptr_t)cols * 2;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  MOE_LAUNCH(moe::launch_pack_weights(src, dst, n_mats, rows, cols, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_load_stats(const moe_shape* s, const int32_t* expert_counts, float coef, float* load_out,
                          float* aux_loss_out, void* stream) {
  MOE_TRY(check_shape(s));
  if (s->T == 0) return MOE_OK;
  MOE_TRY(need(expert_counts, 4));
  MOE_TRY(maybe(load_out, 4));
  MOE_TRY(maybe(aux_loss_out, 4));
  MOE_LAUNCH(moe::launch_load_stats(expert_counts, s->n_experts, (long long)s->T * s->top_k, coef, load_out,
                                    aux_loss_out, (hipStream_t)stream));
  return MOE_OK;
}

namespace {
moe_status quantize_impl(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols, bool fp8,
                         void* stream) {
  if (n_mats < 0 || rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (rows % 16 || cols % 64) return MOE_ERR_ALIGNMENT;
  if (n_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
  MOE_TRY(need(src, 16));
  MOE_TRY(need(dst, 16));
  const uintptr_t in = (uintptr_t)n_mats * (uintptr_t)rows * (uintptr_t)cols * 2;
  const uintptr_t out = moe::quantized_weight_bytes(n_mats, rows, cols);
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + out && b < a + in) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  MOE_LAUNCH(moe::launch_quantize_weights(src, dst, n_mats, rows, cols, fp8, (hipStream_t)stream));
  return MOE_OK;
}
}  // namespace

moe_status moe_quantize_weights(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols,
                                void* stream) {
  return quantize_impl(src, dst, n_mats, rows, cols, false, stream);
}

moe_status moe_quantize_weights_fp8(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols,
                                    void* stream) {
  return quantize_impl(src, dst, n_mats, rows, cols, true, stream);
}

moe_status moe_dequantize_weights(const void* src, int32_t weight_layout, float* dst, int64_t n_mats, int32_t rows,
                                  int32_t cols, void* stream) {
  if (weight_layout != MOE_LAYOUT_INT8_FRAG && weight_layout != MOE_LAYOUT_FP8_FRAG) return MOE_ERR_UNSUPPORTED;
  if (n_mats < 0 || rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (rows % 16 || cols % 64) return MOE_ERR_ALIGNMENT;
  if (n_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
  MOE_TRY(need(src, 16));
  MOE_TRY(need(dst, 16));
  const uintptr_t in = moe::quantized_weight_bytes(n_mats, rows, cols);
  const uintptr_t out = (uintptr_t)n_mats * (uintptr_t)rows * (uintptr_t)cols * 4;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + out && b < a + in) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  MOE_LAUNCH(moe::launch_dequantize_weights(src, weight_layout, dst, n_mats, rows, cols, (hipStream_t)stream));
  return MOE_OK;
}

size_t moe_quantized_weight_bytes(int64_t n_mats, int32_t rows, int32_t cols) {
  if (n_mats < 0 || rows < 0 || cols < 0) return 0;
  return moe::quantized_weight_bytes(n_mats, rows, cols);
}

moe_status moe_route(const moe_shape* s, const void* x, const void* w_router, const float* logit_bias,
                     float* logits_out, int32_t* topk_idx, float* topk_w, void* workspace, size_t ws_bytes,
                     void* stream) {
  MOE_TRY(check_shape(s));
  if (s->T == 0) return MOE_OK;
  MOE_TRY(need(x, 16));
  MOE_TRY(need(w_router, 16));
  MOE_TRY(maybe(logit_bias, 4));
  MOE_TRY(maybe(logits_out, 4));
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(topk_w, 4));
  if (!logits_out) MOE_TRY(check_workspace(*s, workspace, ws_bytes));
  float* logits = logits_out ? logits_out : (float*)at(workspace, layout_of(*s).logits);
  return route_impl(*s, x, w_router, logit_bias, logits, topk_idx, topk_w, Events{nullptr, nullptr},
                    (hipStream_t)stream);
}

moe_status moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* perm_src, int32_t* inv_perm, void* workspace, size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(s));
  if (s->T == 0) return MOE_OK;
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(maybe(expert_counts, 4));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(perm_src, 4));
  MOE_TRY(need(inv_perm, 4));
  MOE_TRY(check_workspace(*s, workspace, ws_bytes));
  int32_t* tiles = (int32_t*)at(workspace, layout_of(*s).tile_counts);
  return permute_impl(*s, topk_idx, expert_counts, expert_offsets, perm_src, inv_perm, tiles,
                      Events{nullptr, nullptr}, (hipStream_t)stream);
}

moe_status moe_grouped_ffn(const moe_shape* s, const void* x, const int32_t* perm_src, const int32_t* expert_offsets,
                           const void* w_gate, const void* w_up, const void* w_down, void* y, void* workspace,
                           size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(s));
  if (s->T == 0) return MOE_OK;
  MOE_TRY(need(x, 16));
  MOE_TRY(maybe(perm_src, 4));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(y, 16));
  MOE_TRY(check_workspace(*s, workspace, ws_bytes));
  moe_shape routed = *s;
  routed.d_shared_hidden = 0;  // this entry point runs the routed groups only
  const Layout L = layout_of(*s);
  const moe::FfnGroups g = groups_for(routed, x, perm_src, expert_offsets, w_gate, w_up, w_down, nullptr, nullptr,
                                      nullptr, at(workspace, L.hid), y);
  return ffn_impl(g, (int32_t*)at(workspace, L.sched), Events{nullptr, nullptr}, (hipStream_t)stream);
}

moe_status moe_grouped_ffn_gelu(const moe_shape* s, const void* x, const int32_t* perm_src,
                                const int32_t* expert_offsets, const void* w1, const float* b1, const void* w2,
                                const float* b2, void* y, void* workspace, size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(s));
  if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->weight_layout != MOE_LAYOUT_ROWMAJOR && s->weight_layout != MOE_LAYOUT_FRAG16) return MOE_ERR_UNSUPPORTED;
  if (s->T == 0) return MOE_OK;
  MOE_TRY(need(x, 16));
  MOE_TRY(maybe(perm_src, 4));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(w1, 16));
  MOE_TRY(maybe(b1, 4));
  MOE_TRY(need(w2, 16));
  MOE_TRY(maybe(b2, 4));
  MOE_TRY(need(y, 16));
  MOE_TRY(check_workspace(*s, workspace, ws_bytes));
  const Layout L = layout_of(*s);
  const moe::FfnGroups fg = gelu_gemm_groups(*s, x, perm_src, expert_offsets, w1, b1, w2, b2, at(workspace, L.hid), y);
  if (moe::ffn_path(fg) == moe::kPathGemm)  // many rows per expert: the tiled grouped GEMM
    return ffn_impl(fg, (int32_t*)at(workspace, L.sched), Events{nullptr, nullptr}, (hipStream_t)stream);
  const moe::GeluGroups g = gelu_groups_for(*s, x, perm_src, expert_offsets, w1, b1, w2, b2, at(workspace, L.hid), y);
  MOE_LAUNCH(moe::launch_gelu_up(g, (hipStream_t)stream));
  MOE_LAUNCH(moe::launch_gelu_down(g, (hipStream_t)stream));
  return MOE_OK;
}

const char* moe_gelu_kernel_name(const moe_shape* s, int layer) {
  if (check_shape(s) != MOE_OK || s->dtype != MOE_BF16 || (layer != 0 && layer != 1)) return "";
  if (s->weight_layout != MOE_LAYOUT_ROWMAJOR && s->weight_layout != MOE_LAYOUT_FRAG16) return "";
  const moe::FfnGroups fg = gelu_gemm_groups(*s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                             nullptr, nullptr);
  if (moe::ffn_path(fg) == moe::kPathGemm)
    return layer == 0 ? moe::ffn_gate_up_kernel_name(fg) : moe::ffn_down_kernel_name(fg);
  const moe::GeluGroups g = gelu_groups_for(*s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                            nullptr, nullptr);
  return moe::gelu_kernel_name(g, layer == 0);
}

moe_status moe_combine(const moe_shape* s, const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                       const void* shared_out, void* out, void* stream) {
  MOE_TRY(check_shape(s));
  if (s->T == 0) return MOE_OK;
  MOE_TRY(need(y_perm, 16));
  MOE_TRY(need(inv_perm, 4));
  MOE_TRY(need(topk_w, 4));
  MOE_TRY(maybe(shared_out, 16));
  MOE_TRY(need(out, 16));
  MOE_LAUNCH(moe::launch_combine(s->dtype, y_perm, inv_perm, topk_w, shared_out, out, s->T, s->top_k, s->d_model,
                                 (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_shape* s, const void* x, const void* w_router, const float* logit_bias,
                             const void* w_gate, const void* w_up, const void* w_down, const void* w_shared_gate,
                             const void* w_shared_up, const void* w_shared_down, void* out, int32_t* topk_idx_out,
                             float* topk_w_out, int32_t* counts_out, float* logits_out, void* workspace,
                             size_t ws_bytes, void* stream) {
  return layer_impl(s, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up, w_shared_down, out,
                    topk_idx_out, topk_w_out, counts_out, logits_out, workspace, ws_bytes, stream, nullptr);
}

moe_status moe_layer_forward_timed(const moe_shape* s, const void* x, const void* w_router, const float* logit_bias,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* w_shared_gate, const void* w_shared_up, const void* w_shared_down,
                                   void* out, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                                   float* logits_out, void* workspace, size_t ws_bytes, void* stream,
                                   void* const* events) {
  return layer_impl(s, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up, w_shared_down, out,
                    topk_idx_out, topk_w_out, counts_out, logits_out, workspace, ws_bytes, stream, events);
}

const char* moe_stage_kernel_name(const moe_shape* s, int stage) {
  if (check_shape(s) != MOE_OK) return "";
  const moe::FfnGroups g = groups_for(*s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      nullptr, nullptr, nullptr);
  switch (stage) {
    case MOE_STAGE_ROUTE_LOGITS: return moe::route_logits_kernel_name(s->dtype, s->T, s->n_experts);
    case MOE_STAGE_ROUTE_TOPK:
      return moe::route_tail_fused(s->T, s->top_k) ? moe::route_tail_small_kernel_name(s->n_experts, s->routing)
                                               : moe::route_topk_kernel_name(s->n_experts, s->routing);
    case MOE_STAGE_PERMUTE_COUNT: return moe::route_tail_fused(s->T, s->top_k) ? "" : "permute_count_kernel";
    case MOE_STAGE_PERMUTE_SCAN: return moe::route_tail_fused(s->T, s->top_k) ? "" : "permute_scan_kernel";
    case MOE_STAGE_PERMUTE_SCATTER: return moe::route_tail_fused(s->T, s->top_k) ? "" : "permute_scatter_kernel";
    case MOE_STAGE_FFN_SCHEDULE: return moe::ffn_schedule_kernel_name(g);
    case MOE_STAGE_FFN_GATE_UP: return moe::ffn_gate_up_kernel_name(g);
    case MOE_STAGE_FFN_DOWN: return moe::ffn_down_kernel_name(g);
    case MOE_STAGE_COMBINE: return moe::combine_kernel_name(s->dtype, s->top_k);
  }
  return "";
}

}  // extern "C"

/*
 * moe.h -- C ABI of the sparse Mixture-of-Experts FFN layer forward on one MI355X (gfx950).
 *
 * One layer forward is: router scoring, top-k selection, weighting of the k selected experts
 * (softmax over their logits, or their normalised sigmoid scores),
 * dispatch of (token, slot) pairs into expert-contiguous order, the routed SwiGLU experts over
 * their buckets plus an always-on shared expert, and the weighted-sum combine back into token
 * order. Pages this follows:
 *   - Sparse-MoE overview article (adg.csdn.net), section 2.2 "router mechanism": Top-K routing as
 *     scoring -> selection -> softmax weighting -> weighted combination; section 4.1 layer code.
 *   - "MoE inference kernels: expert parallelism, dynamic routing gates and all-to-all overlap"
 *     (blog.llmgo.top): section 1.1 shared + fine-grained routed experts; section 1.2 W_gate, W_up,
 *     W_down per expert; section 4.2 one grouped GEMM over ragged groups given by an offsets array,
 *     empty experts skipped; section 4.3 token permutation (flatten ids, sort, bincount, offsets).
 *   - "Computation and Data Movement for Inference", sections 4 and 15: route records sorted by
 *     expert so one weight load serves a bucket; outputs restored to token order, weighted, merged.
 *
 * Conventions for every entry point
 *   - Device pointers unless stated. The caller allocates and owns every buffer, including the
 *     workspace; the library never allocates or frees memory and keeps no pointer past the call.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream). Nothing synchronizes the host and nothing is copied device-to-host. Results are
 *     valid once `stream` reaches the point of the call.
 *   - Row-major layouts. Weights are stored [out, in] like a linear layer's weight:
 *     w_router [E, d]; w_gate, w_up [E, H, d]; w_down [E, d, H]; shared weights [Hs, d], [Hs, d],
 *     [d, Hs]. x, y and out are [rows, d]. `dtype` applies to x, all weights, y and out; routing
 *     weights, logits and the logit bias are always float32; indices are int32.
 *   - Expert weights may instead be passed in the fragment-tiled layout MOE_LAYOUT_FRAG16 made
 *     by moe_pack_weights (bf16 only; every expert matrix's row count a multiple of 16 and column
 *     count a multiple of 32): the matrix-core operand order, so every 1 KB of a weight is one
 *     contiguous 16-row x 32-column MFMA operand. The router weight is always row-major.
 *   - Validation happens on the host before anything is enqueued; on any error nothing is
 *     enqueued. Limits: 0 <= T, T * top_k < 2^31, 1 <= top_k <= n_experts <= 1024, d_model,
 *     d_hidden >= 8 and multiples of 8, d_shared_hidden 0 or a multiple of 8, 16-byte aligned
 *     x / weight / y / out pointers and 4-byte aligned int32 / float32 pointers. T == 0 (with a
 *     valid shape) returns MOE_OK at once: nothing is read, checked or enqueued, so empty tensors
 *     may pass NULL. Experts that receive no token cost no work.
 *   - Deterministic: identical inputs give bitwise-identical outputs (no floating-point atomics).
 *   - Not thread-hostile: the library has no mutable global state.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, bad sizes, k outside [1, E] ... */
  MOE_ERR_UNSUPPORTED = 2, /* dtype or size outside the supported range */
  MOE_ERR_ALIGNMENT = 3,   /* d_model / hidden sizes or pointers not aligned as required */
  MOE_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 5,         /* a kernel launch or event record failed */
  MOE_ERR_TOO_LARGE = 6    /* the shape needs more than moe_layer_forward_noalloc's fixed scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Storage layout of the expert weight matrices (w_gate, w_up, w_down and the shared ones). */
typedef enum {
  MOE_LAYOUT_ROWMAJOR = 0, /* [out, in] row-major, like a linear layer's weight */
  MOE_LAYOUT_FRAG16 = 1,   /* fragment-tiled, see moe_pack_weights */
  MOE_LAYOUT_INT8_FRAG = 2, /* INT8 codes with one float32 scale per output row, see
                               moe_quantize_weights (bf16 layers; the codes become bf16 in
                               registers, in the weight-streaming kernels below 32 rows per
                               expert and in the grouped GEMM above, as for bf16 weights) */
  MOE_LAYOUT_FP8_FRAG = 3   /* FP8 E4M3 codes with one float32 scale per output row, in the same
                               byte order, see moe_quantize_weights_fp8 (as INT8 otherwise) */
} moe_weight_layout;

/* How the router turns logits into the k experts and their weights. */
typedef enum {
  MOE_ROUTING_SOFTMAX = 0, /* top-k of the logits (+ logit bias), softmax over the k (overview
                              article section 2.2) */
  MOE_ROUTING_SIGMOID = 1  /* top-k of sigmoid(logit) + bias, weights = the selected experts'
                              sigmoid(logit) normalised to sum 1; the bias steers the selection
                              only (MoE-kernels page section 2.2, DeepSeek-V3 routing without an
                              auxiliary loss) */
} moe_routing;

/* Layer sizes (host pointer). */
typedef struct {
  int32_t T;               /* tokens in this batch */
  int32_t d_model;         /* d */
  int32_t n_experts;       /* E routed experts */
  int32_t top_k;           /* k experts per token */
  int32_t d_hidden;        /* H, hidden size of each routed expert */
  int32_t d_shared_hidden; /* Hs, hidden size of the shared expert; 0 = no shared expert */
  int32_t dtype;           /* moe_dtype */
  int32_t weight_layout;   /* moe_weight_layout of the expert weights */
  int32_t routing;         /* moe_routing */
} moe_shape;

/*
 * moe_pack_weights -- re-lay n_mats row-major bf16 matrices [n_mats, rows, cols] into the
 * fragment-tiled layout MOE_LAYOUT_FRAG16 (same size). rows % 16 == 0, cols % 32 == 0. Element
 * (r, c) of a matrix moves to
 *     ((r / 16) * (cols / 32) + c / 32) * 512  +  ((r % 16) + 16 * ((c % 32) / 8)) * 8  +  c % 8
 * i.e. the matrix is cut into 16 x 32 blocks stored one after another along each 16-row band,
 * and inside a block lane l = (r % 16) + 16 * ((c % 32) / 8) of a wave holds 8 consecutive
 * columns: the A-operand order of the 16x16x32 bf16 MFMA. src and dst must not overlap; both
 * 16-byte aligned. A one-time preparation step (weight load), not part of the layer forward.
 */
moe_status moe_pack_weights(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols, void* stream);

/*
 * moe_quantize_weights -- INT8 copy of n_mats row-major bf16 matrices [n_mats, rows, cols] for
 * MOE_LAYOUT_INT8_FRAG (inference-optimisation chapter, model-compression part, "make every byte
 * cheaper": x_q = round(x / s) + z; here z = 0 and one scale per output row; overview article
 * section 4.3: INT8 expert weights). For every row r of every matrix m:
 *     s[m][r] = max_c |w[m][r][c]| / 127           (float32; 0 for an all-zero row)
 *     q[m][r][c] = rint(w[m][r][c] / s[m][r])      (float32 division, ties to even, in [-127, 127])
 * and the layer uses w ~ q * s. dst holds n_mats * rows * cols int8 codes in fragment order
 * (each 1 KB: a 16-row x 64-column block; lane l = r % 16 + 16 * ((c % 32) / 8) of a wave holds
 * 8 codes of columns c..c+7 of the block's first 32 columns, then the same 8 of its second 32;
 * code (r, c) at byte ((r/16) * (cols/64) + c/64) * 1024 + lane * 16 + ((c % 64) / 32) * 8 + c % 8),
 * followed by the float32 scales [n_mats, rows]. dst needs moe_quantized_weight_bytes() bytes.
 * rows % 16 == 0, cols % 64 == 0; src and dst 16-byte aligned and not overlapping. A one-time
 * preparation step (weight load), not part of the layer forward.
 */
moe_status moe_quantize_weights(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols,
                                void* stream);

/*
 * moe_quantize_weights_fp8 -- the same as moe_quantize_weights with FP8 codes, for
 * MOE_LAYOUT_FP8_FRAG (the same "1-byte weights" route of the inference-optimisation chapter; the
 * pages fix no FP8 format, the format here is the OCP 8-bit float E4M3 "fn": 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest finite
 * 448). For every row r of every matrix m:
 *     s[m][r] = max_c |w[m][r][c]| / 448            (float32; 0 for an all-zero row)
 *     q[m][r][c] = E4M3(w[m][r][c] / s[m][r])      (float32 division; the nearest E4M3 value, ties
 *                                                    to the even code, 464 and above saturate to 448;
 *                                                    never the NaN pattern)
 * and the layer uses w ~ value(q) * s. Byte layout, buffer size (moe_quantized_weight_bytes) and
 * argument rules as for moe_quantize_weights.
 */
moe_status moe_quantize_weights_fp8(const void* src, void* dst, int64_t n_mats, int32_t rows, int32_t cols,
                                    void* stream);

/*
 * moe_dequantize_weights -- the float32 weights an MOE_LAYOUT_INT8_FRAG or MOE_LAYOUT_FP8_FRAG buffer
 * (src, as written by moe_quantize_weights / moe_quantize_weights_fp8) stands for, row-major
 * [n_mats, rows, cols]: dst[m][r][c] = value(q[m][r][c]) * s[m][r], one float32 multiplication,
 * where value() is the code's integer (INT8) or E4M3 value (the NaN codes 0x7F / 0xFF, which the
 * quantizers never write, give NaN). The code -> value step is the one the weight-streaming kernels
 * run before their multiplications, so this shows exactly which weights the layer uses (inspection,
 * export, checks). weight_layout other than those two: MOE_ERR_UNSUPPORTED. rows % 16 == 0,
 * cols % 64 == 0; src and dst 16-byte aligned and not overlapping. Not part of the layer forward.
 */
moe_status moe_dequantize_weights(const void* src, int32_t weight_layout, float* dst, int64_t n_mats, int32_t rows,
                                  int32_t cols, void* stream);

/* Bytes of an MOE_LAYOUT_INT8_FRAG or MOE_LAYOUT_FP8_FRAG buffer of n_mats [rows, cols] matrices:
 * codes plus scales. */
size_t moe_quantized_weight_bytes(int64_t n_mats, int32_t rows, int32_t cols);

/* Bytes of workspace that every entry point below accepts for shape `s` (0 if `s` is invalid). */
size_t moe_workspace_bytes(const moe_shape* s);

/* Short English description of a status code (static string). */
const char* moe_status_string(moe_status st);

/*
 * moe_route -- scoring, selection and weighting for every token.
 * Overview article section 2.2 steps 1-3; MoE-kernels page sections 2.2 and 4.3 (gate, top-k).
 *   logits[t, e] = sum_i x[t, i] * w_router[e, i], accumulated in float32.
 *   MOE_ROUTING_SOFTMAX: l = logits (+ logit_bias[e]);
 *     topk_idx[t, 0..k-1] = the k largest l, ordered by value descending, ties to the lower e;
 *     topk_w[t, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected (sums to 1).
 *   MOE_ROUTING_SIGMOID: a_e = sigmoid(logits[t, e]) = 1 / (1 + exp(-logits[t, e]));
 *     topk_idx[t, 0..k-1] = the k largest a_e + logit_bias[e] (same order and tie rule);
 *     topk_w[t, j] = a_j / sum_i a_i over the k selected (the bias does not enter the weights).
 * x [T, d] (dtype); w_router [E, d] (dtype); logit_bias [E] float32 or NULL (softmax: added to
 * the logits before both selection and softmax; sigmoid: added to the sigmoid scores for the
 * selection only); logits_out [T, E] float32 or NULL (softmax: the logits with the bias added;
 * sigmoid: the plain logits); topk_idx [T, k] int32 and topk_w [T, k] float32 are required outputs.
 * Scores are compared as floats with a NaN score taken as -inf, so every token gets k distinct ids
 * in [0, E) whatever the logits hold (a NaN ties with -inf, and the tie goes to the lower id).
 * Softmax weights of selected -inf or NaN scores are 0 while at least one selected score is
 * finite; with none finite the weights are unspecified.
 */
moe_status moe_route(const moe_shape* s, const void* x, const void* w_router, const float* logit_bias,
                     float* logits_out, int32_t* topk_idx, float* topk_w, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * moe_permute -- dispatch bookkeeping (MoE-kernels page section 4.3; data-movement page section 4).
 *   expert_counts[e]  = number of (t, j) with topk_idx[t, j] == e          int32 [E]
 *   expert_offsets    = exclusive running sum, offsets[0] = 0, offsets[E] = T*k   int32 [E+1]
 *   perm_src[r]       = flat slot t*k + j of dispatched row r; the rows of expert e are
 *                       [offsets[e], offsets[e+1]) in increasing t                int32 [T*k]
 *   inv_perm[t*k + j] = r, the inverse permutation                               int32 [T*k]
 * topk_idx [T, k] int32 with every entry in [0, E) (entries outside give unspecified results but
 * never out-of-bounds accesses). expert_counts may be NULL.
 */
moe_status moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* perm_src, int32_t* inv_perm, void* workspace,
                       size_t ws_bytes, void* stream);

/*
 * moe_load_stats -- load statistics of a routing (overview article section 4.1, the layer code's
 * auxiliary balance loss):
 *   load_out[e]     = expert_counts[e] / (T * k)                                   float32 [E]
 *   aux_loss_out[0] = coef * sum_e (load_out[e] - 1/E)^2   (the page uses coef = 0.01) float32 [1]
 * expert_counts [E] int32 as written by moe_permute / moe_layer_forward; load_out and
 * aux_loss_out may each be NULL. float32, fixed summation order (deterministic).
 */
moe_status moe_load_stats(const moe_shape* s, const int32_t* expert_counts, float coef, float* load_out,
                          float* aux_loss_out, void* stream);

/*
 * moe_grouped_ffn -- every expert over its own contiguous bucket of rows, in one pass
 * (MoE-kernels page sections 1.2 and 4.2):
 *   for each e and each row r in [expert_offsets[e], expert_offsets[e+1]):
 *     src = perm_src ? perm_src[r] / k : r
 *     h = SiLU(w_gate[e] . x[src]) * (w_up[e] . x[src]),  SiLU(z) = z * sigmoid(z)
 *     y[r] = w_down[e] . h
 * With perm_src == NULL, x is read as [T*k, d] rows in bucket order (for the shared expert pass
 * {E=1, k=1, H=Hs} with offsets {0, T}). Rows = T*k; offsets must be non-decreasing with
 * offsets[E] == T*k. y [T*k, d] (dtype). Accumulation in float32; for bfloat16 the hidden
 * activation h is rounded to bfloat16 before the down projection and y is rounded once.
 */
moe_status moe_grouped_ffn(const moe_shape* s, const void* x, const int32_t* perm_src,
                           const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                           const void* w_down, void* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn_gelu -- moe_grouped_ffn with the two-layer GELU expert of the overview
 * article's layer code (section 4.1: Linear(d -> H), GELU, Linear(H -> d), each linear with a bias)
 * in place of SwiGLU:
 *   for each e and each row r in [expert_offsets[e], expert_offsets[e+1]):
 *     src = perm_src ? perm_src[r] / k : r
 *     h = GELU(w1[e] . x[src] + b1[e]),  GELU(z) = z * Phi(z) = z * erfc(-z / sqrt 2) / 2
 *     y[r] = w2[e] . h + b2[e]
 * bfloat16 layers only and weight_layout MOE_LAYOUT_ROWMAJOR or MOE_LAYOUT_FRAG16 (otherwise
 * MOE_ERR_UNSUPPORTED). w1 [E, H, d] and w2 [E, d, H] are stored like w_gate and w_down; b1 [E, H]
 * and b2 [E, d] are float32, or NULL for a zero bias. d_shared_hidden is ignored (routed experts
 * only). The hidden activations live in the workspace (moe_workspace_bytes() of the same shape). A
 * layer with these experts is moe_route, moe_permute, moe_grouped_ffn_gelu and moe_combine with
 * shared_out NULL. Accumulation in float32; h is rounded to bfloat16 before the second linear and
 * y once. Like moe_grouped_ffn, the experts run as weight-streaming kernels when the buckets are
 * small (fewer than 32 rows per expert on average: decode) and as the tiled grouped GEMM otherwise
 * (prefill), with the biases and the GELU applied in the GEMM's epilogues.
 */
moe_status moe_grouped_ffn_gelu(const moe_shape* s, const void* x, const int32_t* perm_src,
                                const int32_t* expert_offsets, const void* w1, const float* b1, const void* w2,
                                const float* b2, void* y, void* workspace, size_t ws_bytes, void* stream);

/* Kernel of one layer of moe_grouped_ffn_gelu for this shape (layer 0: the first linear and GELU,
 * 1: the second linear), as the profiler names it; "" for an invalid shape or layer. On the grouped
 * GEMM path a third, small launch (gemm_schedule_kernel) precedes them. */
const char* moe_gelu_kernel_name(const moe_shape* s, int layer);

/*
 * moe_combine -- back to token order and weighted merge (overview article section 2.2 step 4;
 * MoE-kernels page section 1.1: the shared expert's output is added for every token):
 *   out[t] = shared_out[t] + sum_{j<k} topk_w[t, j] * y_perm[inv_perm[t*k + j]]
 * y_perm [T*k, d], shared_out [T, d] or NULL, out [T, d] (all dtype). float32 accumulation in
 * fixed j order, one rounding to dtype.
 */
moe_status moe_combine(const moe_shape* s, const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                       const void* shared_out, void* out, void* stream);

/*
 * moe_layer_forward -- the whole layer: moe_route, moe_permute, the grouped FFN of the routed
 * experts together with the shared expert (w_shared_* may be NULL when d_shared_hidden == 0),
 * and moe_combine. out [T, d] is required. topk_idx_out [T, k], topk_w_out [T, k],
 * counts_out [E] and logits_out [T, E] are optional copies of the intermediates (NULL = keep
 * them in the workspace).
 */
moe_status moe_layer_forward(const moe_shape* s, const void* x, const void* w_router, const float* logit_bias,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* w_shared_gate, const void* w_shared_up, const void* w_shared_down,
                             void* out, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                             float* logits_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_layer_forward_noalloc -- moe_layer_forward with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. The intermediates live in a fixed device array of MOE_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends; the call itself allocates and
 * frees nothing. Shapes whose moe_workspace_bytes() exceed that size return MOE_ERR_TOO_LARGE
 * (64 MiB holds the DeepSeek-V3-shaped decode layer up to T = 401 tokens). The current device must
 * be the device of `stream` (else MOE_ERR_INVALID_ARG); the first call on a device looks up that
 * device's address of the array, so make it outside stream capture. Every call on one GPU uses the
 * same array and leaves its contents behind: calls that overlap on one GPU (other streams, other
 * threads) race, so serialize them. Arguments and results otherwise as moe_layer_forward.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_shape* s, const void* x, const void* w_router,
                                     const float* logit_bias, const void* w_gate, const void* w_up,
                                     const void* w_down, const void* w_shared_gate, const void* w_shared_up,
                                     const void* w_shared_down, void* out, int32_t* topk_idx_out,
                                     float* topk_w_out, int32_t* counts_out, float* logits_out, void* stream);

/*
 * Kernel stages of moe_layer_forward, for per-kernel timing. moe_layer_forward_timed() is
 * moe_layer_forward with hipEvent_t `events[2*i]` recorded on `stream` just before stage i's
 * kernel launch and `events[2*i+1]` just after it (NULL entries are skipped; a stage that
 * launches nothing records both events back to back). `events` may be NULL.
 */
enum {
  MOE_STAGE_ROUTE_LOGITS = 0,
  MOE_STAGE_ROUTE_TOPK = 1,   /* with T <= 16 and T*k <= 4096: top-k, softmax and the whole
                                 dispatch in one launch, and the three permute stages launch nothing */
  MOE_STAGE_PERMUTE_COUNT = 2,
  MOE_STAGE_PERMUTE_SCAN = 3,
  MOE_STAGE_PERMUTE_SCATTER = 4,
  MOE_STAGE_FFN_SCHEDULE = 5, /* tile schedule of the grouped GEMM (launches nothing on the GEMV path) */
  MOE_STAGE_FFN_GATE_UP = 6,
  MOE_STAGE_FFN_DOWN = 7,
  MOE_STAGE_COMBINE = 8,
  MOE_NUM_STAGES = 9
};

moe_status moe_layer_forward_timed(const moe_shape* s, const void* x, const void* w_router,
                                   const float* logit_bias, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* w_shared_gate, const void* w_shared_up,
                                   const void* w_shared_down, void* out, int32_t* topk_idx_out,
                                   float* topk_w_out, int32_t* counts_out, float* logits_out, void* workspace,
                                   size_t ws_bytes, void* stream, void* const* events);

/* Name of the kernel (as a profiler lists it) that stage `stage` launches for shape `s`, or ""
 * if it launches none. */
const char* moe_stage_kernel_name(const moe_shape* s, int stage);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */

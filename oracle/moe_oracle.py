"""CPU oracle for one sparse Mixture-of-Experts FFN layer forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module;
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it. It shares no code
with the HIP library.

Everything is computed in float64 (NumPy; BLAS dgemm is plain fp64 accumulation). Inputs arrive
as bfloat16 bit patterns (uint16) or float32 and are widened to float64 exactly. The result is the
plain definition of the layer; experts run in a per-expert loop, which is fine on the CPU.

Sources (the pages this follows):
  [MoE overview]  Sparse-MoE overview article, adg.csdn.net (6a31135810ee7a33f27dd6b8), §2.2 "router
                  mechanism": Top-K routing = scoring, selection, weighting, combination; §4.1 MoE
                  layer code (flatten, score, top-k, softmax over the k, per-expert loop).
  [MoE kernels]   "MoE inference kernels: expert parallelism, dynamic routing gates and all-to-all
                  overlap", blog.llmgo.top, §1.1 (always-on shared expert + fine-grained routed
                  experts), §1.2 (W_gate, W_up, W_down per expert), §4.2 (grouped GEMM over an
                  offsets array), §4.3 (token permutation: flatten ids, sort, bincount, offsets).
  [Data movement] "Computation and Data Movement for Inference", §4 and §15 (sort routes by expert,
                  run each expert once over its bucket, convert back to token order, weight, merge).
  [Inference ch.6] "大模型推理优化基础" (LLM-from-scratch ch. 6), roofline section: a gated MLP is
                  up, gate and down matmuls.
  [Inference ch.6 quant] the same chapter, model-compression part, second route ("make every byte
                  cheaper"): for memory-bound decode, 1-byte weights halve the bytes read; affine
                  quantization x_q = round(x / s) + z, x_hat = (x_q - z) * s, with a per-tensor,
                  per-channel or per-group scale. [MoE overview] §4.3 quantizes expert weights to
                  INT8 for the same reason.
  [MoE kernels §2.2] the same page, §2.2 (DeepSeek-V3 routing without an auxiliary loss): experts
                  are picked on sigmoid affinities plus a per-expert bias; the weights use the
                  selected experts' sigmoid affinities without the bias, normalised to sum to one;
                  and the router listing of §4.3 (sigmoid of the raw logits plus the bias, top-k on
                  that, weights from the unbiased sigmoid of the selected).

Readings where the pages are silent or garbled:
  * combine: out = Shared(x) + sum_j w_j * Expert_{e_j}(x); the shared expert has weight 1, no
    residual and no norm inside the layer (the [MoE kernels] §1.1 formula is lost in extraction).
  * no learned router bias; an optional per-expert logit bias is an explicit input, added to the
    logits before both selection and softmax (softmax routing).
  * sigmoid routing ([MoE kernels §2.2]): S_e = sigmoid(l_e) + b_e decides the selection;
    w_e = sigmoid(l_e) / sum over the selected of sigmoid(l_j). The listing adds 1e-6 to that
    denominator; the formula of §2.2 does not, and the oracle follows the formula (a sum of k
    positive sigmoids needs no guard in float64).
  * gate = softmax over the K selected raw logits, temperature 1 ([MoE overview] §2.2 step 3).
  * expert = SwiGLU: h = SiLU(x W_gate^T) * (x W_up^T), y = h W_down^T, SiLU(z) = z * sigmoid(z)
    (standard definition; the pages name the three matrices but never define the activation).
  * GELU expert ([MoE overview] §4.1 layer code, the optional two-layer variant): y = GELU(x W1^T
    + b1) W2^T + b2, both linears with a bias, GELU(z) = z * Phi(z) with Phi the standard normal
    CDF (the exact form, the default of the linear-GELU-linear block the listing builds; the
    page does not define GELU itself), no shared expert.
  * top-K order: value descending, ties to the lower expert index.
  * permutation: rows sorted by (expert, token), i.e. flat position t*k+j ascending inside each
    expert; offsets are exclusive with E+1 entries.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "widen", "router_logits", "select_topk", "softmax_selected", "route", "permute", "silu",
    "swiglu", "grouped_ffn", "combine", "layer_forward", "layer_forward_tokens", "layer_forward_tokens_many",
    "topk_gap",
    "logistic", "selection_scores", "sigmoid_weights_selected", "ROUTINGS",
    "quantize", "dequantize", "quantize_rows_int8", "dequantize_rows_int8", "load_stats",
    "E4M3_MAX", "fp8_e4m3_decode", "fp8_e4m3_encode", "quantize_rows_fp8", "dequantize_rows_fp8",
    "gelu", "gelu_mlp", "grouped_ffn_gelu", "layer_forward_gelu",
]

ROUTINGS = ("softmax", "sigmoid")


# ----------------------------------------------------------------------------- input decoding

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> float64, exactly."""
    a = np.asarray(a)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return a.astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- routing

def router_logits(x: np.ndarray, w_router: np.ndarray, logit_bias: np.ndarray | None = None) -> np.ndarray:
    """Scoring: s[t, e] = x_t . W_g[e] (+ b_e).

    [MoE overview] §2.2 step 1: a small linear layer scores each token against every expert;
    W_g is stored [E, d] like a linear layer's [out, in] weight ([MoE kernels] §4.3 gate).
    """
    L = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if logit_bias is not None:
        L = L + np.asarray(logit_bias, np.float64)[None, :]
    return L


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """Selection: per token, the k experts with the highest scores.

    [MoE overview] §2.2 step 2 (sort all E scores, keep the K best). Order: value descending, ties
    to the lower expert index. A stable sort of the negated scores gives exactly that order.
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def softmax_selected(L: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Weighting: softmax over the k selected scores, so the k weights sum to 1.

    [MoE overview] §2.2 step 3 and the §4.1 code (softmax over the top-k scores).
    The largest selected score is subtracted first; that does not change the value.
    """
    v = np.take_along_axis(np.asarray(L, np.float64), idx, axis=1)
    if v.shape[1] == 0:
        return v
    m = v.max(axis=1, keepdims=True)
    e = np.exp(v - m)
    return e / e.sum(axis=1, keepdims=True)


def logistic(z: np.ndarray) -> np.ndarray:
    """sigmoid(z) = 1 / (1 + e^-z), written so that neither branch overflows."""
    z = np.asarray(z, np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def selection_scores(L: np.ndarray, routing: str = "softmax", bias: np.ndarray | None = None) -> np.ndarray:
    """What the top-K selection ranks.

    softmax routing: the logits themselves (a logit bias is already inside L).
    sigmoid routing, [MoE kernels §2.2]: the sigmoid affinity plus the per-expert bias,
    S_e = sigmoid(l_e) + b_e.
    """
    if routing == "softmax":
        return np.asarray(L, np.float64)
    if routing == "sigmoid":
        S = logistic(L)
        if bias is not None:
            S = S + np.asarray(bias, np.float64)[None, :]
        return S
    raise ValueError(routing)


def sigmoid_weights_selected(L: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Weighting of sigmoid routing, [MoE kernels §2.2]: the selected experts' sigmoid affinities of
    the raw logits (no bias), divided by their sum over the selected set."""
    s = np.take_along_axis(logistic(L), idx, axis=1)
    if s.shape[1] == 0:
        return s
    return s / s.sum(axis=1, keepdims=True)


def route(x, w_router, k, bias=None, routing="softmax"):
    """Scoring, selection and weighting for every token: (logits [T,E], idx [T,k], w [T,k]).

    softmax routing: ``bias`` (optional) is added to the logits, which then decide the selection
    and are softmax-normalised over the k selected. sigmoid routing: the logits are x . W_g^T
    without bias; ``bias`` (optional) only shifts the sigmoid scores used for the selection.
    """
    if routing == "softmax":
        L = router_logits(x, w_router, bias)
        idx = select_topk(L, k)
        return L, idx, softmax_selected(L, idx)
    if routing == "sigmoid":
        L = router_logits(x, w_router, None)
        idx = select_topk(selection_scores(L, "sigmoid", bias), k)
        return L, idx, sigmoid_weights_selected(L, idx)
    raise ValueError(routing)


def topk_gap(L: np.ndarray, k: int) -> np.ndarray:
    """Per-token margin between the k-th and (k+1)-th largest score (inf when k == E)."""
    T, E = L.shape
    if k >= E:
        return np.full(T, np.inf)
    s = -np.sort(-np.asarray(L, np.float64), axis=1)
    return s[:, k - 1] - s[:, k]


# ----------------------------------------------------------------------------- weight quantization

def quantize(x, s, z=0):
    """[Inference ch.6 quant]: x_q = round(x / s) + z (round half to even)."""
    return np.rint(np.asarray(x, np.float64) / s) + z


def dequantize(q, s, z=0):
    """[Inference ch.6 quant]: x_hat = (x_q - z) * s."""
    return (np.asarray(q, np.float64) - z) * s


def quantize_rows_int8(w: np.ndarray):
    """Per-output-channel symmetric INT8 of a [..., rows, cols] weight: z = 0 and one scale per
    row (output channel), s = max|w_row| / 127, codes round(w / s) in [-127, 127]; an all-zero row
    gets s = 0 and zero codes. The codes are integers decided by floating point, and the pages fix
    no precision for that decision; the weights are stored in bf16 and the GPU kernel quantizes in
    float32, so the oracle takes the same decision in float32 (fl32 = rounding to float32):
    s = fl32(max / 127), q = rint(fl32(w / s)). The dequantized weight q * s that the layer uses
    is then exact in float64. Returns (q int8, s float32 [..., rows])."""
    w32 = np.asarray(w, np.float64).astype(np.float32)
    m = np.abs(w32).max(axis=-1)
    s = (m / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((w32 / safe[..., None]).astype(np.float32))
    q = np.where(s[..., None] > 0, np.clip(q, -127, 127), 0)
    return q.astype(np.int8), s


def dequantize_rows_int8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The float64 weight an INT8 row-scaled matrix stands for: q * s per row."""
    return dequantize(q, np.asarray(s, np.float64)[..., None])


# FP8 weights ([Inference ch.6 quant]: any 1-byte code halves the bytes decode reads; the pages name
# no FP8 format, so the reading is the OCP 8-bit floating-point format E4M3 in its "fn" variant:
# 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities, and the
# pattern S.1111.111 reserved for NaN, so the largest finite magnitude is 1.75 * 2^8 = 448).

E4M3_MAX = 448.0


def fp8_e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64: (-1)^s (1 + m/8) 2^(e-7) for e > 0, (-1)^s m 2^-9
    for e = 0 (subnormals); NaN for the reserved pattern."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Code (uint8) of the E4M3 value nearest to each float32 input, ties to the even code;
    magnitudes of 464 and above (past the midpoint between 448 and the 480 the format does not
    have) saturate to 448. The sign bit is the input's (-0.0 gives 0x80). Every step below is exact
    in float64 for float32 inputs, so the rounding is decided on the exact value."""
    x = np.asarray(x, np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    sub = np.rint(np.minimum(a, 1.0) * 512.0)        # subnormal grid 2^-9; 8 is 2^-6, the first normal
    frac, ex = np.frexp(np.where(a > 0, a, 1.0))     # a = frac 2^ex, frac in [0.5, 1)
    e = ex - 1 + 7                                   # biased exponent of a = (1 + m/8) 2^(ex-1)
    m = np.rint((2.0 * frac - 1.0) * 8.0)            # 0 .. 8
    carry = m == 8.0
    e = e + carry
    m = np.where(carry, 0.0, m)
    normal = (e.astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(a >= 464.0, 0x7E, np.where(a < 2.0 ** -6, sub.astype(np.int64), normal))
    return (code | sign).astype(np.uint8)


def quantize_rows_fp8(w: np.ndarray):
    """Per-output-channel FP8 (E4M3) of a [..., rows, cols] weight: one scale per row,
    s = max|w_row| / 448, codes E4M3(w / s), so each row's largest magnitude maps to 448; an
    all-zero row gets s = 0 and zero codes. The pages fix no precision for the division; as for the
    INT8 codes the decision is taken in float32, the precision the GPU kernel quantizes in:
    s = fl32(max / 448), code = E4M3(fl32(w / s)). Returns (codes uint8, s float32 [..., rows])."""
    w32 = np.asarray(w, np.float64).astype(np.float32)
    mx = np.abs(w32).max(axis=-1)
    s = (mx / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = fp8_e4m3_encode((w32 / safe[..., None]).astype(np.float32))
    codes = np.where(s[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, s


def dequantize_rows_fp8(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The float64 weight an FP8 row-scaled matrix stands for: E4M3 value * s per row."""
    return fp8_e4m3_decode(codes) * np.asarray(s, np.float64)[..., None]


# ----------------------------------------------------------------------------- dispatch

def permute(idx: np.ndarray, E: int):
    """Dispatch bookkeeping: (counts [E], offsets [E+1], perm_src [T*k], inv_perm [T*k]).

    [MoE kernels] §4.3: flatten the selected expert ids, bring equal ids together, count tokens per
    expert (bincount) and turn the counts into offsets for the grouped GEMM (§4.2).
    [Data movement] §4: route records sorted by expert id so that one weight load serves a bucket.

    perm_src[r] is the flat position t*k + j of the r-th row in expert order; rows of one expert are
    in increasing flat position (hence increasing token). inv_perm is its inverse.
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(E, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm_src = np.empty(T * k, np.int64)
    fill = offsets[:E].copy()
    for p in range(T * k):           # flat positions in increasing order
        e = flat[p]
        perm_src[fill[e]] = p
        fill[e] += 1
    inv_perm = np.empty(T * k, np.int64)
    inv_perm[perm_src] = np.arange(T * k)
    return counts, offsets, perm_src, inv_perm


def load_stats(counts: np.ndarray, T: int, k: int, coef: float = 0.01):
    """Per-expert load and the balance penalty of the [MoE overview] §4.1 layer code: each expert's
    share of the T*k assignments, load_e = counts_e / (T k), and
    aux = coef * sum_e (load_e - 1/E)^2 (coef 0.01 there). Returns (load [E], aux); T = 0 gives
    zero loads and the penalty of an empty batch, coef * sum_e (1/E)^2 = coef / E."""
    counts = np.asarray(counts, np.float64)
    E = counts.shape[0]
    load = counts / (T * k) if T * k > 0 else np.zeros(E)
    aux = coef * float(((load - 1.0 / E) ** 2).sum())
    return load, aux


# ----------------------------------------------------------------------------- experts

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU (Swish with beta = 1): z * sigmoid(z)."""
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One gated expert MLP: y = (SiLU(X W_gate^T) * (X W_up^T)) W_down^T.

    [MoE kernels] §1.2: each routed expert holds W_gate, W_up, W_down; [Inference ch.6] roofline
    section: a gated MLP is the up, gate and down matmuls. Weights are [out, in].
    """
    X = np.asarray(X, np.float64)
    G = X @ np.asarray(w_gate, np.float64).T
    U = X @ np.asarray(w_up, np.float64).T
    return (silu(G) * U) @ np.asarray(w_down, np.float64).T


_erfc = np.frompyfunc(math.erfc, 1, 1)


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU, exact form: z * Phi(z), with Phi(z) = erfc(-z / sqrt 2) / 2 (the C library's erfc;
    the same as (1 + erf(z / sqrt 2)) / 2 without its cancellation for negative z)."""
    z = np.asarray(z, np.float64)
    return z * _erfc(-z / math.sqrt(2.0)).astype(np.float64) / 2.0


def gelu_mlp(X: np.ndarray, w1: np.ndarray, b1, w2: np.ndarray, b2) -> np.ndarray:
    """The two-layer expert of the [MoE overview] §4.1 layer code: Linear(d -> H), GELU,
    Linear(H -> d), each linear with a bias (None = zero). Weights are [out, in]."""
    X = np.asarray(X, np.float64)
    Z = X @ np.asarray(w1, np.float64).T
    if b1 is not None:
        Z = Z + np.asarray(b1, np.float64)[None, :]
    Y = gelu(Z) @ np.asarray(w2, np.float64).T
    if b2 is not None:
        Y = Y + np.asarray(b2, np.float64)[None, :]
    return Y


def grouped_ffn_gelu(x_rows: np.ndarray, offsets: np.ndarray, expert_fn) -> np.ndarray:
    """``grouped_ffn`` with the GELU expert: ``expert_fn(e)`` returns float64 (W1 [H,d], b1 [H] or
    None, W2 [d,H], b2 [d] or None)."""
    x_rows = np.asarray(x_rows, np.float64)
    y = np.zeros_like(x_rows)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = gelu_mlp(x_rows[a:b], *expert_fn(e))
    return y


def grouped_ffn(x_rows: np.ndarray, offsets: np.ndarray, expert_fn) -> np.ndarray:
    """Every expert over its own contiguous bucket of rows; empty buckets do no work.

    [MoE kernels] §4.2: one grouped GEMM over ragged groups given by an offsets array.
    ``x_rows`` are the dispatched rows (expert order); ``expert_fn(e)`` returns float64
    (W_gate [H,d], W_up [H,d], W_down [d,H]).
    """
    x_rows = np.asarray(x_rows, np.float64)
    y = np.zeros_like(x_rows)
    E = len(offsets) - 1
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            g, u, dn = expert_fn(e)
            y[a:b] = swiglu(x_rows[a:b], g, u, dn)
    return y


def combine(y_perm: np.ndarray, inv_perm: np.ndarray, w: np.ndarray, shared_out: np.ndarray | None = None):
    """Combination: out_t = Shared(x_t) + sum_j w[t, j] * y[row of (t, j)].

    [MoE overview] §2.2 step 4 (weighted sum of the selected experts); [MoE kernels] §1.1 (the
    shared expert's output is added for every token); [Data movement] §4 (expert outputs go back
    to token order, are weighted and merged).
    """
    w = np.asarray(w, np.float64)
    T, k = w.shape
    y_perm = np.asarray(y_perm, np.float64)
    d = y_perm.shape[1] if y_perm.ndim == 2 else (shared_out.shape[1] if shared_out is not None else 0)
    out = np.zeros((T, d)) if shared_out is None else np.array(shared_out, np.float64, copy=True)
    for j in range(k):
        rows = np.asarray(inv_perm, np.int64).reshape(T, k)[:, j]
        out += w[:, j:j + 1] * y_perm[rows]
    return out


# ----------------------------------------------------------------------------- whole layer

def layer_forward(x, w_router, k, expert_fn, shared_fn=None, bias=None, routing="softmax"):
    """The full layer on float64 inputs. Returns a dict of every intermediate.

    ``expert_fn(e)`` / ``shared_fn()`` return float64 (W_gate, W_up, W_down); ``bias`` and
    ``routing`` as in ``route``.
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    L, idx, w = route(x, w_router, k, bias, routing)
    counts, offsets, perm_src, inv_perm = permute(idx, E)
    x_rows = x[perm_src // k] if T else np.zeros((0, x.shape[1]))
    y_perm = grouped_ffn(x_rows, offsets, expert_fn)
    shared = swiglu(x, *shared_fn()) if shared_fn is not None else None
    out = combine(y_perm, inv_perm, w, shared)
    return dict(logits=L, idx=idx, w=w, counts=counts, offsets=offsets, perm_src=perm_src,
                inv_perm=inv_perm, y_perm=y_perm, shared=shared, out=out)


def layer_forward_tokens(x_rows, w_router, k, expert_fn, shared_fn=None, bias=None, routing="softmax"):
    """Output rows for a sample of tokens. Each token's result depends only on its own row (routing
    is per token and the experts act row by row), so a sample of rows can be checked on its own at
    any batch size. Experts are visited once each, in increasing id, and their weighted outputs
    added to the tokens that selected them: the same sum over the k selected experts as
    ``combine``, in another order of addition."""
    x_rows = np.asarray(x_rows, np.float64)
    L, idx, w = route(x_rows, w_router, k, bias, routing)
    out = np.zeros_like(x_rows)
    if shared_fn is not None:
        out += swiglu(x_rows, *shared_fn())
    for e in np.unique(idx):
        t_sel, j_sel = np.nonzero(idx == e)
        g, u, dn = expert_fn(int(e))
        out[t_sel] += w[t_sel, j_sel][:, None] * swiglu(x_rows[t_sel], g, u, dn)
    return dict(logits=L, idx=idx, w=w, out=out)


def layer_forward_tokens_many(cases, expert_fn, shared_fn=None):
    """``layer_forward_tokens`` for several token samples that share the expert weights (each with
    its own router weight, k, bias and routing rule), visiting every expert once for all of them:
    on the CPU the expert weights, not the rows, are the cost. ``cases`` is a list of
    (x_rows, w_router, k, bias, routing); returns one dict (logits, idx, w, out) per case, each
    equal to what ``layer_forward_tokens`` gives for that case on its own."""
    res = []
    for x_rows, w_router, k, bias, routing in cases:
        x_rows = np.asarray(x_rows, np.float64)
        L, idx, w = route(x_rows, w_router, k, bias, routing)
        res.append(dict(logits=L, idx=idx, w=w, out=np.zeros_like(x_rows), x=x_rows))
    if shared_fn is not None and any(r["x"].shape[0] for r in res):
        sw = shared_fn()
        for r in res:
            r["out"] += swiglu(r["x"], *sw)
    experts = sorted(set().union(*(set(np.unique(r["idx"]).tolist()) for r in res))) if res else []
    for e in experts:
        g, u, dn = expert_fn(int(e))
        for r in res:
            t_sel, j_sel = np.nonzero(r["idx"] == e)
            if t_sel.size:
                r["out"][t_sel] += r["w"][t_sel, j_sel][:, None] * swiglu(r["x"][t_sel], g, u, dn)
    for r in res:
        del r["x"]
    return res


def layer_forward_gelu(x, w_router, k, expert_fn, bias=None, routing="softmax"):
    """The layer of the [MoE overview] §4.1 code with its two-layer GELU experts: routing, dispatch,
    ``grouped_ffn_gelu`` and the weighted combine, no shared expert. ``expert_fn(e)`` as in
    ``grouped_ffn_gelu``; ``bias`` and ``routing`` as in ``route`` (the listing's biased router
    linear is the logit bias of softmax routing)."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    L, idx, w = route(x, w_router, k, bias, routing)
    counts, offsets, perm_src, inv_perm = permute(idx, E)
    x_rows = x[perm_src // k] if T else np.zeros((0, x.shape[1]))
    y_perm = grouped_ffn_gelu(x_rows, offsets, expert_fn)
    out = combine(y_perm, inv_perm, w, None)
    return dict(logits=L, idx=idx, w=w, counts=counts, offsets=offsets, perm_src=perm_src,
                inv_perm=inv_perm, y_perm=y_perm, out=out)

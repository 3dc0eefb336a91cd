"""Python binding of libmoe.so, the MI355X sparse-MoE layer forward (C ABI in include/moe.h).

Argument marshalling only: every function here passes device pointers and sizes to the
C entry point of the same name, on the current (or given) HIP stream. PyTorch provides device
memory and streams. There is no fallback: if the HIP library is missing, importing this package
fails with an error that says how to build it.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime first, so libmoe.so binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_moe_layer_router_amd/build.py` "
                      "(hipcc, gfx950). There is no CPU fallback.")
_lib = ctypes.CDLL(LIB_PATH)

(MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
 MOE_ERR_TOO_LARGE) = range(7)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # fixed device scratch of moe_layer_forward_noalloc
MOE_CALIB_READ_BLOCKS, MOE_CALIB_MFMA_BLOCKS = 512, 256   # workgroups (sink entries) of the probes
MOE_F32, MOE_BF16 = 0, 1
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_FRAG16, MOE_LAYOUT_INT8_FRAG, MOE_LAYOUT_FP8_FRAG = 0, 1, 2, 3
MOE_ROUTING_SOFTMAX, MOE_ROUTING_SIGMOID = 0, 1
STAGES = ["route_logits", "route_topk", "permute_count", "permute_scan", "permute_scatter", "ffn_schedule",
          "ffn_gate_up", "ffn_down", "combine"]
MOE_NUM_STAGES = len(STAGES)


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_hidden", ctypes.c_int32), ("d_shared_hidden", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("weight_layout", ctypes.c_int32), ("routing", ctypes.c_int32)]


def make_shape(T, d_model, n_experts, top_k, d_hidden, d_shared_hidden=0, dtype=MOE_BF16,
               weight_layout=MOE_LAYOUT_ROWMAJOR, routing=MOE_ROUTING_SOFTMAX) -> moe_shape:
    if isinstance(dtype, str):
        dtype = {"bf16": MOE_BF16, "f32": MOE_F32}[dtype]
    elif isinstance(dtype, torch.dtype):
        dtype = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[dtype]
    if isinstance(routing, str):
        routing = {"softmax": MOE_ROUTING_SOFTMAX, "sigmoid": MOE_ROUTING_SIGMOID}[routing]
    return moe_shape(T, d_model, n_experts, top_k, d_hidden, d_shared_hidden, dtype, weight_layout, routing)


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {moe_status_string(status)} (status {status})")


_P = ctypes.c_void_p
_S = ctypes.POINTER(moe_shape)
_sigs = {
    "moe_workspace_bytes": (ctypes.c_size_t, [_S]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_permute": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_grouped_ffn": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_ffn_gelu": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_gelu_kernel_name": (ctypes.c_char_p, [_S, ctypes.c_int]),
    "moe_layer_forward": (ctypes.c_int, [_S] + [_P] * 15 + [ctypes.c_size_t, _P]),
    "moe_layer_forward_timed": (ctypes.c_int, [_S] + [_P] * 15 + [ctypes.c_size_t, _P, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_S] + [_P] * 15),   # 14 tensors + the stream
    "moe_stage_kernel_name": (ctypes.c_char_p, [_S, ctypes.c_int]),
    "moe_pack_weights": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P]),
    "moe_quantize_weights": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P]),
    "moe_quantize_weights_fp8": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P]),
    "moe_dequantize_weights": (ctypes.c_int, [_P, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              _P]),
    "moe_load_stats": (ctypes.c_int, [_S, _P, ctypes.c_float, _P, _P, _P]),
    "moe_quantized_weight_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    # measurement probes (include/moe_calib.h)
    "moe_calib_read_stream": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_int, _P]),
    "moe_calib_mfma": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype, _f.argtypes = _res, _args

EXPORTED = tuple(_sigs)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(workspace):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_workspace_bytes(shape: moe_shape) -> int:
    return int(_lib.moe_workspace_bytes(ctypes.byref(shape)))


def allocate_workspace(shape: moe_shape, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_workspace_bytes(shape), 1), dtype=torch.uint8, device=device)


def moe_route(shape, x, w_router, logit_bias, logits_out, topk_idx, topk_w, workspace=None, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_route", _lib.moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                       _ptr(logits_out), _ptr(topk_idx), _ptr(topk_w), ws, nb, _stream(stream)))


def moe_permute(shape, topk_idx, expert_counts, expert_offsets, perm_src, inv_perm, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_permute", _lib.moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(expert_counts),
                                           _ptr(expert_offsets), _ptr(perm_src), _ptr(inv_perm), ws, nb,
                                           _stream(stream)))


def moe_grouped_ffn(shape, x, perm_src, expert_offsets, w_gate, w_up, w_down, y, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_grouped_ffn", _lib.moe_grouped_ffn(ctypes.byref(shape), _ptr(x), _ptr(perm_src),
                                                   _ptr(expert_offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                                   _ptr(y), ws, nb, _stream(stream)))


def moe_grouped_ffn_gelu(shape, x, perm_src, expert_offsets, w1, b1, w2, b2, y, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check("moe_grouped_ffn_gelu", _lib.moe_grouped_ffn_gelu(ctypes.byref(shape), _ptr(x), _ptr(perm_src),
                                                             _ptr(expert_offsets), _ptr(w1), _ptr(b1), _ptr(w2),
                                                             _ptr(b2), _ptr(y), ws, nb, _stream(stream)))


def gelu_layer_buffers(shape, device="cuda"):
    """Intermediates of a layer with GELU experts: routing, dispatch and expert outputs, and the
    workspace (hidden activations, logits, permutation scratch)."""
    T, k, E, d = shape.T, shape.top_k, shape.n_experts, shape.d_model
    i32 = dict(dtype=torch.int32, device=device)
    return dict(idx=torch.empty(T, k, **i32), w=torch.empty(T, k, dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32), perm_src=torch.empty(T * k, **i32),
                inv_perm=torch.empty(T * k, **i32), y=torch.empty(T * k, d, dtype=torch.bfloat16, device=device),
                workspace=allocate_workspace(shape, device))


def moe_layer_forward_gelu(shape, x, w_router, logit_bias, w1, b1, w2, b2, out, buffers, stream=None):
    """A layer with the two-layer GELU experts: moe_route, moe_permute, moe_grouped_ffn_gelu and
    moe_combine (no shared expert) on `buffers` from gelu_layer_buffers."""
    b = buffers
    moe_route(shape, x, w_router, logit_bias, None, b["idx"], b["w"], b["workspace"], stream)
    moe_permute(shape, b["idx"], b["counts"], b["offsets"], b["perm_src"], b["inv_perm"], b["workspace"], stream)
    moe_grouped_ffn_gelu(shape, x, b["perm_src"], b["offsets"], w1, b1, w2, b2, b["y"], b["workspace"], stream)
    moe_combine(shape, b["y"], b["inv_perm"], b["w"], None, out, stream)


def moe_gelu_kernel_name(shape, layer: int) -> str:
    return _lib.moe_gelu_kernel_name(ctypes.byref(shape), layer).decode()


def moe_combine(shape, y_perm, inv_perm, topk_w, shared_out, out, stream=None):
    _check("moe_combine", _lib.moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w),
                                           _ptr(shared_out), _ptr(out), _stream(stream)))


def _layer_args(shape, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                w_shared_down, out, topk_idx_out, topk_w_out, counts_out, logits_out, workspace, stream):
    ws, nb = _ws(workspace)
    return [ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w_gate), _ptr(w_up),
            _ptr(w_down), _ptr(w_shared_gate), _ptr(w_shared_up), _ptr(w_shared_down), _ptr(out),
            _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(counts_out), _ptr(logits_out), ws, nb, _stream(stream)]


def moe_layer_forward(shape, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                      w_shared_down, out, topk_idx_out=None, topk_w_out=None, counts_out=None, logits_out=None,
                      workspace=None, stream=None):
    _check("moe_layer_forward", _lib.moe_layer_forward(*_layer_args(
        shape, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up, w_shared_down, out,
        topk_idx_out, topk_w_out, counts_out, logits_out, workspace, stream)))


def moe_layer_forward_noalloc(shape, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                              w_shared_down, out, topk_idx_out=None, topk_w_out=None, counts_out=None,
                              logits_out=None, stream=None):
    """moe_layer_forward on the library's fixed per-GPU scratch: no workspace argument."""
    _check("moe_layer_forward_noalloc", _lib.moe_layer_forward_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(w_shared_gate), _ptr(w_shared_up), _ptr(w_shared_down), _ptr(out), _ptr(topk_idx_out),
        _ptr(topk_w_out), _ptr(counts_out), _ptr(logits_out), _stream(stream)))


def moe_layer_forward_timed(shape, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                            w_shared_down, out, topk_idx_out=None, topk_w_out=None, counts_out=None,
                            logits_out=None, workspace=None, stream=None, events=None):
    """`events` is a ctypes array of 2 * MOE_NUM_STAGES hipEvent_t handles (or None)."""
    _check("moe_layer_forward_timed", _lib.moe_layer_forward_timed(*_layer_args(
        shape, x, w_router, logit_bias, w_gate, w_up, w_down, w_shared_gate, w_shared_up, w_shared_down, out,
        topk_idx_out, topk_w_out, counts_out, logits_out, workspace, stream), events))


def moe_pack_weights(src, dst, n_mats, rows, cols, stream=None):
    """Fragment-tiled copy of n_mats row-major bf16 [rows, cols] matrices (MOE_LAYOUT_FRAG16)."""
    _check("moe_pack_weights", _lib.moe_pack_weights(_ptr(src), _ptr(dst), n_mats, rows, cols, _stream(stream)))


def pack_expert_weights(w_gate, w_up, w_down, shared=None, stream=None):
    """Packed copies of [E,H,d], [E,H,d], [E,d,H] (and an optional shared triple) bf16 weights."""
    out = []
    for w in (w_gate, w_up, w_down) + (tuple(shared) if shared is not None else ()):
        p = torch.empty_like(w)
        n = 1 if w.dim() == 2 else w.shape[0]
        moe_pack_weights(w, p, n, w.shape[-2], w.shape[-1], stream)
        out.append(p)
    return out


def moe_load_stats(shape, expert_counts, coef=0.01, load_out=None, aux_loss_out=None, stream=None):
    """Per-expert load counts/(T*k) and the balance penalty coef * sum (load - 1/E)^2."""
    _check("moe_load_stats", _lib.moe_load_stats(ctypes.byref(shape), _ptr(expert_counts), coef, _ptr(load_out),
                                                 _ptr(aux_loss_out), _stream(stream)))


def moe_quantize_weights(src, dst, n_mats, rows, cols, stream=None):
    """INT8 codes (fragment order) + per-row float32 scales of n_mats bf16 [rows, cols] matrices
    (MOE_LAYOUT_INT8_FRAG)."""
    _check("moe_quantize_weights", _lib.moe_quantize_weights(_ptr(src), _ptr(dst), n_mats, rows, cols,
                                                             _stream(stream)))


def moe_quantized_weight_bytes(n_mats, rows, cols) -> int:
    return int(_lib.moe_quantized_weight_bytes(n_mats, rows, cols))


def moe_quantize_weights_fp8(src, dst, n_mats, rows, cols, stream=None):
    """FP8 E4M3 codes (fragment order) + per-row float32 scales of n_mats bf16 [rows, cols] matrices
    (MOE_LAYOUT_FP8_FRAG)."""
    _check("moe_quantize_weights_fp8", _lib.moe_quantize_weights_fp8(_ptr(src), _ptr(dst), n_mats, rows, cols,
                                                                     _stream(stream)))


def moe_dequantize_weights(src, weight_layout, dst, n_mats, rows, cols, stream=None):
    """The float32 [n_mats, rows, cols] weights value(q) * s an INT8 or FP8 buffer stands for."""
    _check("moe_dequantize_weights", _lib.moe_dequantize_weights(_ptr(src), weight_layout, _ptr(dst), n_mats, rows,
                                                                 cols, _stream(stream)))


def quantize_expert_weights(w_gate, w_up, w_down, shared=None, stream=None, fp8=False):
    """INT8 (or, with fp8=True, FP8 E4M3) buffers (uint8 tensors) of [E,H,d], [E,H,d], [E,d,H] (and an
    optional shared triple)."""
    fn = moe_quantize_weights_fp8 if fp8 else moe_quantize_weights
    out = []
    for w in (w_gate, w_up, w_down) + (tuple(shared) if shared is not None else ()):
        n = 1 if w.dim() == 2 else w.shape[0]
        q = torch.empty(moe_quantized_weight_bytes(n, w.shape[-2], w.shape[-1]), dtype=torch.uint8, device=w.device)
        fn(w, q, n, w.shape[-2], w.shape[-1], stream)
        out.append(q)
    return out


def moe_stage_kernel_name(shape, stage: int) -> str:
    return _lib.moe_stage_kernel_name(ctypes.byref(shape), stage).decode()


def moe_calib_read_stream(buf, sink, nontemporal=True, stream=None):
    """Read all of ``buf`` once (16-byte loads); sink: MOE_CALIB_READ_BLOCKS uint32 (int32 tensor)."""
    _check("moe_calib_read_stream", _lib.moe_calib_read_stream(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(bool(nontemporal)), _stream(stream)))


def moe_calib_mfma(operands, iters, sink, clocks=None, stream=None):
    """bf16 MFMA loop on ``operands`` (MOE_CALIB_MFMA_BLOCKS * 512 * 16 bf16); sink: float32
    [MOE_CALIB_MFMA_BLOCKS]; clocks: int64 [MOE_CALIB_MFMA_BLOCKS * 8 * 4] or None."""
    _check("moe_calib_mfma", _lib.moe_calib_mfma(_ptr(operands), int(iters), _ptr(sink), _ptr(clocks),
                                                 _stream(stream)))

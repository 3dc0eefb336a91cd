"""Seeded synthetic inputs for the sparse-MoE layer (shared by the oracle tests and the GPU path).

This module holds none of the MoE layer's arithmetic. It draws normal numbers from a counter-based
stream (Philox4x32-10 + Box-Muller, see ``csrc/synth.hip``), rounds them to the storage type and
lays them out in the shapes the layer takes. Every tensor has its own stream id, so any slice (one
expert, one token row) can be regenerated on the host bit-for-bit, and the big weight sets can be
filled directly in device memory.

Shapes follow the configurations the layer is measured on: a tiny fp32 layer, a DeepSeek-V3-shaped
layer (d_model 7168, 256 routed SwiGLU experts of hidden 2048 plus one shared expert, top-8) at
T = 8, 256 and 8192 tokens, and a Mixtral-shaped skewed layer (d_model 4096, 8 experts of hidden
14336, top-2, router logits biased by 2 ln of a Zipf(1.2) law); the decode layer also comes with
sigmoid routing and a selection-only expert bias N(0, 0.05^2). Weights are N(0, std = 1/sqrt(fan_in)),
activations N(0, 1).
"""

from __future__ import annotations

import ctypes
import math
import os
import dataclasses
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

# stream kinds: stream id = kind * 2**40 + index
K_X, K_WG, K_GATE, K_UP, K_DOWN, K_SGATE, K_SUP, K_SDOWN, K_REDRAW, K_SBIAS = range(1, 11)
K_GELU = 16   # GELU expert variant: index 0 W1 [E, H, d], 1 W2 [E, d, H], 2 b1 [E, H], 3 b2 [E, d]
_KSHIFT = 1 << 40


def stream_id(kind: int, index: int = 0) -> int:
    return kind * _KSHIFT + index


def redraw_stream(token: int, attempt: int) -> int:
    """Stream of the `attempt`-th replacement draw of activation row `token`."""
    return stream_id(K_REDRAW, token * 4096 + attempt)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(LIB_PATH)
        u64, i32 = ctypes.c_uint64, ctypes.c_int
        lib.syn_fill_host.argtypes = [ctypes.c_void_p, i32, u64, u64, u64, u64, u64, u64, ctypes.c_double, i32]
        lib.syn_fill_host.restype = i32
        lib.syn_fill_device.argtypes = [ctypes.c_void_p, i32, u64, u64, u64, u64, u64, u64, ctypes.c_double,
                                        ctypes.c_void_p]
        lib.syn_fill_device.restype = i32
        _lib = lib
    return _lib


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def normal_host(shape, seed: int, stream: int, std: float, dtype: str, *, nblk: int = 1,
                stream_step: int = 1, first: int = 0) -> np.ndarray:
    """Host draw. ``dtype`` "bf16" returns raw uint16 bf16 bits, "f32" float32.

    The result has ``nblk`` blocks (leading axis when nblk > 1); block j uses stream
    ``stream + j * stream_step`` and elements ``first .. first + blk - 1`` of it.
    """
    shape = tuple(int(s) for s in shape)
    blk = int(np.prod(shape[1:] if nblk > 1 else shape, dtype=np.int64))
    is_bf16 = dtype == "bf16"
    out = np.empty(shape, dtype=np.uint16 if is_bf16 else np.float32)
    if out.size:
        _load().syn_fill_host(out.ctypes.data, int(is_bf16), nblk, blk, first, seed, stream, stream_step,
                              float(std), host_threads())
    return out


def normal_device(tensor, seed: int, stream: int, std: float, *, nblk: int = 1, stream_step: int = 1,
                  first: int = 0, hip_stream=None) -> None:
    """Fill a contiguous CUDA(HIP) torch tensor (bfloat16 or float32) in place."""
    import torch

    assert tensor.is_contiguous() and tensor.is_cuda
    is_bf16 = tensor.dtype == torch.bfloat16
    assert is_bf16 or tensor.dtype == torch.float32
    n = tensor.numel()
    if n == 0:
        return
    assert n % nblk == 0
    if hip_stream is None:
        hip_stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _load().syn_fill_device(ctypes.c_void_p(tensor.data_ptr()), int(is_bf16), nblk, n // nblk, first, seed,
                                 stream, stream_step, float(std), ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError(f"syn_fill_device failed with hipError {rc}")


# --------------------------------------------------------------------------- configurations

@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    H: int
    Hs: int          # shared-expert hidden size, 0 = none
    dtype: str       # "f32" or "bf16"
    zipf_s: float | None = None          # softmax routing: logit bias 2 ln Zipf(s)
    routing: str = "softmax"             # "softmax" (top-k of logits, softmax over the k) or "sigmoid"
    score_bias_std: float | None = None  # sigmoid routing: selection bias b_e ~ N(0, std^2), fp32
    note: str = field(default="", compare=False)


CONFIGS = [
    LayerConfig("tiny_fp32", 16, 64, 8, 2, 128, 0, "f32",
                note="T=16, d=64, E=8, k=2, SwiGLU hidden 128, no shared expert, fp32"),
    LayerConfig("dsv3_decode_t8", 8, 7168, 256, 8, 2048, 2048, "bf16",
                note="DeepSeek-V3-shaped layer at decode, 0.25 tokens per expert"),
    LayerConfig("dsv3_decode_t256", 256, 7168, 256, 8, 2048, 2048, "bf16",
                note="DeepSeek-V3-shaped layer, decode batch of 256, ~8 tokens per expert"),
    LayerConfig("dsv3_prefill_t8192", 8192, 7168, 256, 8, 2048, 2048, "bf16",
                note="DeepSeek-V3-shaped layer, prefill chunk of 8192, ~256 tokens per expert"),
    LayerConfig("skewed_mixtral_t4096", 4096, 4096, 8, 2, 14336, 0, "bf16", zipf_s=1.2,
                note="8 experts of hidden 14336, top-2, Zipf(1.2) router bias"),
    LayerConfig("dsv3_sigmoid_decode_t8", 8, 7168, 256, 8, 2048, 2048, "bf16", routing="sigmoid",
                score_bias_std=0.05,
                note="the decode layer with sigmoid routing and a selection-only expert bias"),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def with_tokens(cfg: LayerConfig, T: int) -> LayerConfig:
    return dataclasses.replace(cfg, T=T)


def zipf_logit_bias(E: int, s: float) -> np.ndarray:
    """b_e = 2 ln p_e with p_e = (e+1)^-s / sum_r r^-s (expert 0 is the most popular), as float32."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p = p / p.sum()
    return (2.0 * np.log(p)).astype(np.float32)


def weight_std(fan_in: int) -> float:
    return 1.0 / math.sqrt(fan_in)


@dataclass
class HostInputs:
    """Host copies of the small inputs (x, router, bias). bf16 tensors are uint16 bit arrays."""
    cfg: LayerConfig
    seed: int
    x: np.ndarray
    w_router: np.ndarray
    logit_bias: np.ndarray | None               # softmax routing: added to the logits
    redraws: dict = field(default_factory=dict)   # token -> attempts used
    score_bias: np.ndarray | None = None        # sigmoid routing: added to the scores for selection

    @property
    def router_bias(self) -> np.ndarray | None:
        """The one per-expert bias vector the layer takes, whichever routing it belongs to."""
        return self.score_bias if self.cfg.routing == "sigmoid" else self.logit_bias


def host_small_inputs(cfg: LayerConfig, seed: int = 0) -> HostInputs:
    x = normal_host((cfg.T, cfg.d), seed, stream_id(K_X), 1.0, cfg.dtype)
    wg = normal_host((cfg.E, cfg.d), seed, stream_id(K_WG), weight_std(cfg.d), cfg.dtype)
    bias = zipf_logit_bias(cfg.E, cfg.zipf_s) if cfg.zipf_s is not None else None
    sbias = None
    if cfg.score_bias_std is not None:
        sbias = normal_host((cfg.E,), seed, stream_id(K_SBIAS), cfg.score_bias_std, "f32")
    return HostInputs(cfg, seed, x, wg, bias, score_bias=sbias)


def redraw_rows(inp: HostInputs, rows) -> None:
    """Replace activation rows by fresh draws from their redraw streams (one more attempt each)."""
    for t in rows:
        t = int(t)
        a = inp.redraws.get(t, 0) + 1
        inp.redraws[t] = a
        inp.x[t] = normal_host((inp.cfg.d,), inp.seed, redraw_stream(t, a), 1.0, inp.cfg.dtype)


def expert_weights_host(cfg: LayerConfig, seed: int, e: int, shared: bool = False):
    """(W_gate [H,d], W_up [H,d], W_down [d,H]) of routed expert e, or of the shared expert."""
    if shared:
        H, kg, ku, kd, idx = cfg.Hs, K_SGATE, K_SUP, K_SDOWN, 0
    else:
        H, kg, ku, kd, idx = cfg.H, K_GATE, K_UP, K_DOWN, e
    g = normal_host((H, cfg.d), seed, stream_id(kg, idx), weight_std(cfg.d), cfg.dtype)
    u = normal_host((H, cfg.d), seed, stream_id(ku, idx), weight_std(cfg.d), cfg.dtype)
    dn = normal_host((cfg.d, H), seed, stream_id(kd, idx), weight_std(H), cfg.dtype)
    return g, u, dn


def all_expert_weights_host(cfg: LayerConfig, seed: int):
    """Stacked [E,H,d], [E,H,d], [E,d,H] host weights (only sensible for small layers)."""
    E, H, d = cfg.E, cfg.H, cfg.d
    g = normal_host((E, H, d), seed, stream_id(K_GATE), weight_std(d), cfg.dtype, nblk=E)
    u = normal_host((E, H, d), seed, stream_id(K_UP), weight_std(d), cfg.dtype, nblk=E)
    dn = normal_host((E, d, H), seed, stream_id(K_DOWN), weight_std(H), cfg.dtype, nblk=E)
    return g, u, dn


def fill_expert_weights_device(cfg: LayerConfig, seed: int, w_gate, w_up, w_down, shared=None) -> None:
    """Fill device tensors [E,H,d], [E,H,d], [E,d,H] (and optionally the shared triple) in place."""
    E, H, d = cfg.E, cfg.H, cfg.d
    normal_device(w_gate, seed, stream_id(K_GATE), weight_std(d), nblk=E)
    normal_device(w_up, seed, stream_id(K_UP), weight_std(d), nblk=E)
    normal_device(w_down, seed, stream_id(K_DOWN), weight_std(H), nblk=E)
    if shared is not None:
        sg, su, sd = shared
        normal_device(sg, seed, stream_id(K_SGATE), weight_std(d))
        normal_device(su, seed, stream_id(K_SUP), weight_std(d))
        normal_device(sd, seed, stream_id(K_SDOWN), weight_std(cfg.Hs))

"""GPU-side test plumbing: seeded inputs on the device and the oracle's view of the same tensors."""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle
import synth
from tests import helpers

import sparse_moe_layer_router_amd as moe

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Host array (bf16 bit patterns or float32) -> device tensor of the storage type."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@dataclass
class DeviceLayer:
    cfg: synth.LayerConfig
    seed: int
    host: synth.HostInputs
    x: torch.Tensor
    w_router: torch.Tensor
    bias: torch.Tensor | None
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    ws_gate: torch.Tensor | None
    ws_up: torch.Tensor | None
    ws_down: torch.Tensor | None
    stacked_host: tuple | None   # host copies of all expert weights (small layers only)
    layout: int = moe.MOE_LAYOUT_ROWMAJOR

    @property
    def shape(self):
        c = self.cfg
        return moe.make_shape(c.T, c.d, c.E, c.k, c.H, c.Hs, c.dtype, self.layout, c.routing)

    @property
    def quant(self):
        """One-byte weight format of the layout ("int8", "fp8"), or None for bf16 / fp32 weights."""
        return {moe.MOE_LAYOUT_INT8_FRAG: "int8", moe.MOE_LAYOUT_FP8_FRAG: "fp8"}.get(self.layout)

    def expert_fn(self, cache=True):
        return helpers.expert_fn_host(self.cfg, self.seed, self.stacked_host, cache=cache, quant=self.quant)

    def shared_fn(self):
        return helpers.shared_fn_host(self.cfg, self.seed, quant=self.quant)


def make_weights(cfg: synth.LayerConfig, seed: int, host_copy: bool):
    """Expert weights on the device; small layers are drawn on the host and uploaded, big ones are
    drawn directly in device memory from the same generator streams (bit-identical)."""
    dt = TORCH_DT[cfg.dtype]
    E, H, d = cfg.E, cfg.H, cfg.d
    if host_copy:
        g, u, dn = synth.all_expert_weights_host(cfg, seed)
        dev = tuple(to_dev(a, cfg.dtype) for a in (g, u, dn))
        stacked = (g, u, dn)
    else:
        dev = (torch.empty(E, H, d, dtype=dt, device="cuda"), torch.empty(E, H, d, dtype=dt, device="cuda"),
               torch.empty(E, d, H, dtype=dt, device="cuda"))
        synth.fill_expert_weights_device(cfg, seed, *dev)
        stacked = None
    shared = (None, None, None)
    if cfg.Hs:
        sg, su, sd = synth.expert_weights_host(cfg, seed, 0, shared=True)
        shared = tuple(to_dev(a, cfg.dtype) for a in (sg, su, sd))
    torch.cuda.synchronize()
    return dev, shared, stacked


def packed_weights(weights):
    """The same weights in the fragment-tiled layout (device copies)."""
    (g, u, dn), shared, stacked = weights
    sh = tuple(shared) if shared[0] is not None else None
    out = moe.pack_expert_weights(g, u, dn, sh)
    torch.cuda.synchronize()
    return (tuple(out[:3]), tuple(out[3:]) if sh else (None, None, None), stacked)


def int8_weights(weights, fp8=False):
    """Per-row INT8 (or FP8 E4M3) copies of the same bf16 weights (MOE_LAYOUT_INT8_FRAG or
    MOE_LAYOUT_FP8_FRAG buffers)."""
    (g, u, dn), shared, stacked = weights
    sh = tuple(shared) if shared[0] is not None else None
    out = moe.quantize_expert_weights(g, u, dn, sh, fp8=fp8)
    torch.cuda.synchronize()
    return (tuple(out[:3]), tuple(out[3:]) if sh else (None, None, None), stacked)


def make_layer(cfg: synth.LayerConfig, seed: int = 0, screen: bool = True, weights=None,
               layout: int = moe.MOE_LAYOUT_ROWMAJOR) -> DeviceLayer:
    host = synth.host_small_inputs(cfg, seed)
    if screen:
        helpers.screen_gaps(host)
    small = cfg.E * cfg.H * cfg.d <= 64 * 1024 * 1024
    if weights is None:
        weights = make_weights(cfg, seed, host_copy=small)
        if layout == moe.MOE_LAYOUT_FRAG16:
            weights = packed_weights(weights)
        elif layout == moe.MOE_LAYOUT_INT8_FRAG:
            weights = int8_weights(weights)
        elif layout == moe.MOE_LAYOUT_FP8_FRAG:
            weights = int8_weights(weights, fp8=True)
    (g, u, dn), (sg, su, sd), stacked = weights
    bias = torch.from_numpy(host.router_bias).cuda() if host.router_bias is not None else None
    return DeviceLayer(cfg, seed, host, to_dev(host.x, cfg.dtype), to_dev(host.w_router, cfg.dtype), bias,
                       g, u, dn, sg, su, sd, stacked, layout)


@dataclass
class LayerRun:
    out: torch.Tensor
    idx: torch.Tensor
    w: torch.Tensor
    counts: torch.Tensor
    logits: torch.Tensor


def run_layer(L: DeviceLayer, workspace=None) -> LayerRun:
    c = L.cfg
    s = L.shape
    dt = TORCH_DT[c.dtype]
    out = torch.empty(c.T, c.d, dtype=dt, device="cuda")
    idx = torch.empty(c.T, c.k, dtype=torch.int32, device="cuda")
    w = torch.empty(c.T, c.k, dtype=torch.float32, device="cuda")
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    logits = torch.empty(c.T, c.E, dtype=torch.float32, device="cuda")
    ws = workspace if workspace is not None else moe.allocate_workspace(s)
    moe.moe_layer_forward(s, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up, L.ws_down,
                          out, idx, w, counts, logits, ws)
    torch.cuda.synchronize()
    return LayerRun(out, idx, w, counts, logits)


def tolerance_ok(gpu: np.ndarray, ref: np.ndarray):
    """max|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3 over the whole tensor."""
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    bound = 1e-2 * (float(np.max(np.abs(ref))) if ref.size else 0.0) + 1e-3
    return err <= bound, err, bound


def oracle_inputs(L: DeviceLayer):
    """(x, W_g, bias) in float64/float32 as the oracle takes them; the bias is the one the routing
    rule uses (logit bias for softmax routing, selection bias for sigmoid routing)."""
    c = L.cfg
    x = oracle.widen(L.host.x, c.dtype)
    wg = oracle.widen(L.host.w_router, c.dtype)
    return x, wg, L.host.router_bias

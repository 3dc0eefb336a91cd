#!/usr/bin/env python3
"""Throughput of the sparse-MoE layer forward on one MI355X.

One step = one moe_layer_forward (router, top-k + softmax, permutation, routed + shared SwiGLU
experts, combine) over one batch of synthetic tokens already resident in HBM. W untimed warm-up
steps, then exactly K timed steps between two device synchronizations; the step cycles through a
few distinct token batches so consecutive steps route differently.

Prints one JSON line: tokens/s for the whole step, the dominant kernel's roofline fraction (its
average duration taken from the two HIP events recorded on the launch stream around that kernel in
each timed step, and its algorithmic bytes or flops per launch), the per-stage breakdown (from an
untimed pass with events around every stage), and the CPU oracle timed on a bounded sample of the
same workload on the host cores.

The default workload is the DeepSeek-V3-shaped prefill chunk (T = 8192, the compute-bound half of
the metric, against the bf16 MFMA peak). The same run then measures the same layer and weights at
the decode sizes T = 8 and T = 256 (the HBM-bound half) and carries them under "decode".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-decode]
                       [--no-cpu-baseline] [--layout frag16|rowmajor|int8|fp8] [--expert swiglu|gelu]
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; achieved HBM TB/s (decode) and MFMA util (prefill)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
N_BATCHES = 4                   # distinct token batches cycled through the steps
FLUSH_BYTES = 1 << 30          # cache-evicting copy between the steps of the distribution pass


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="dsv3_prefill_t8192")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode sub-records (the same layer at T = 8 and 256) of a prefill run")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceilings", action="store_true", help="skip the measured read and MFMA ceilings")
    p.add_argument("--ceilings", action="store_true",
                   help="only measure the read-stream, copy and MFMA ceilings of this GPU (one JSON line)")
    p.add_argument("--cpu-sample-tokens", type=int, default=None)
    p.add_argument("--expert", choices=["swiglu", "gelu"], default="swiglu",
                   help="expert form: SwiGLU (with the shared expert), or the two-layer GELU expert with "
                        "biased linears (moe_grouped_ffn_gelu; no shared expert)")
    p.add_argument("--layout", choices=["frag16", "rowmajor", "int8", "fp8"], default="frag16",
                   help="expert weight layout (frag16: packed once at load time, before timing; int8, fp8: "
                        "per-row INT8 or E4M3 codes made once from the bf16 weights, before timing)")
    p.add_argument("--ep-share", type=int, default=0, metavar="G",
                   help="instead of the layer, time the expert stage of one GPU of G in expert parallel: "
                        "its E/G experts over the rows routed to them from G batches of T tokens, and the "
                        "shared expert over its own T tokens (bf16 weights)")
    return p.parse_args()


# ------------------------------------------------------------------------------------ HIP events
class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (events on the library's stream)."""

    def __init__(self, n):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev[i] = h

    def record(self, i, stream):
        rc = self.lib.hipEventRecord(self.ev[i], ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def array(self, start, count):
        return ctypes.cast(ctypes.byref(self.ev, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for h in self.ev:
            self.lib.hipEventDestroy(h)


# ------------------------------------------------------------------------------- work accounting
def alg_bytes_and_flops(cfg, counts_list, es, one_byte=False):
    """Per-stage algorithmic bytes and flops of one step, averaged over the cycled batches.

    Bytes are what the method must move once: each active expert's weights (one byte per weight
    plus a float32 scale per row for INT8 or FP8 weights), the shared expert's, the router, x in, out out
    (plus, per kernel, its own inputs and outputs). Flops are 2*T*d*E (router) + 6*rows*d*H (gated
    MLP) + 6*T*d*Hs."""
    T, d, E, k, H, Hs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.H, cfg.Hs
    rows = T * k
    wb = 1 if one_byte else es
    res = []
    for counts in counts_list:
        n_act = int((counts > 0).sum())
        sc_gu = 4 * (n_act * 2 * H + 2 * Hs) if one_byte else 0
        sc_dn = 4 * (n_act * d + (d if Hs else 0)) if one_byte else 0
        gate_up_w = wb * (n_act * 2 * H * d + 2 * Hs * d) + sc_gu
        down_w = wb * (n_act * d * H + d * Hs) + sc_dn
        gate_up = gate_up_w + es * T * d + es * (rows * H + T * Hs)              # weights + x + hidden out
        down = down_w + es * (rows * H + T * Hs) + es * (rows + (T if Hs else 0)) * d
        layer = gate_up_w + down_w + es * E * d + es * T * d + es * T * d
        flops_gate_up = 4 * rows * d * H + 4 * T * d * Hs
        flops_down = 2 * rows * d * H + 2 * T * d * Hs
        res.append(dict(n_act=n_act, gate_up=gate_up, down=down, layer=layer,
                        flops_gate_up=flops_gate_up, flops_down=flops_down,
                        flops_layer=2 * T * d * E + 6 * rows * d * H + 6 * T * d * Hs,
                        unit_gate_up=wb * 2 * H * d, unit_down=wb * d * H))
    avg = {key: sum(r[key] for r in res) / len(res) for key in res[0]}
    return avg


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload, kernel):
    """profiles/traffic_<kernel with template arguments>_<workload>.json"""
    name = "_".join(filter(None, "".join(c if c.isalnum() else " " for c in kernel).split()))
    return os.path.join(ROOT, "profiles", f"traffic_{name}_{workload}.json")


def traffic_for(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they match this source."""
    path = traffic_path(workload, kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel") != kernel or t.get("source_sha") != source_sha(t.get("sources", [])):
        return None
    return t.get("bytes_per_launch")


# ----------------------------------------------------------------------------------- CPU oracle
def cpu_baseline(cfg, host, n_tokens, min_seconds=10.0, max_repeats=8, quant=None):
    """The fp64 oracle on a bounded sample of the same workload (input generation excluded).

    The sample's oracle pass (routing, conversion of the selected experts' stored weights to fp64, SwiGLU,
    combine) is repeated until about ``min_seconds`` of CPU work has been timed."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = None
    rng = np.random.default_rng(1)
    tokens = np.sort(rng.choice(cfg.T, size=min(n_tokens, cfg.T), replace=False))
    x_bits = host.x[tokens]
    wg_bits = host.w_router
    _, idx, _ = oracle.route(oracle.widen(x_bits, cfg.dtype), oracle.widen(wg_bits, cfg.dtype), cfg.k,
                             host.router_bias, cfg.routing)
    raw = {int(e): synth.expert_weights_host(cfg, 0, int(e)) for e in np.unique(idx)}   # untimed
    shared_raw = synth.expert_weights_host(cfg, 0, 0, shared=True) if cfg.Hs else None
    # stored form of each weight (untimed): the bf16 bits, or per-row INT8 / FP8 codes and scales
    qz, dq = {"int8": (oracle.quantize_rows_int8, oracle.dequantize_rows_int8),
              "fp8": (oracle.quantize_rows_fp8, oracle.dequantize_rows_fp8)}.get(quant, (None, None))
    store = (lambda a: qz(oracle.widen(a, cfg.dtype))) if quant else (lambda a: a)
    stored = {e: tuple(store(a) for a in m) for e, m in raw.items()}
    shared_stored = tuple(store(a) for a in shared_raw) if shared_raw else None

    def weight(a):   # stored form -> the float64 weight the layer uses (timed, like the GPU's loads)
        return dq(*a) if quant else oracle.widen(a, cfg.dtype)
    expert_fn = lambda e: tuple(weight(a) for a in stored[e])  # noqa: E731
    shared_fn = (lambda: tuple(weight(a) for a in shared_stored)) if shared_stored else None
    reps, total = 0, 0.0
    while reps < max_repeats and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        ref = oracle.layer_forward_tokens(oracle.widen(x_bits, cfg.dtype), oracle.widen(wg_bits, cfg.dtype),
                                          cfg.k, expert_fn, shared_fn, host.router_bias, cfg.routing)
        total += time.perf_counter() - t0
        reps += 1
    assert ref["out"].shape == (len(tokens), cfg.d)
    return {"value": round(len(tokens) * reps / total, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sampled": True, "sample_tokens": int(len(tokens)), "workload_tokens": cfg.T,
            "sample": f"{len(tokens)} of {cfg.T} tokens of {cfg.name}, {reps} passes in {total:.1f} s (routing, "
                      f"{quant.upper() if quant else cfg.dtype}->fp64 conversion of the {len(raw)} selected experts"
                      f"{' + shared' if shared_raw else ''}, SwiGLU, combine; expert weight generation"
                      f"{' and quantization' if quant else ''} excluded)"}


# ------------------------------------------------------------------------ GELU expert variant
def gelu_alg_bytes(cfg, counts_list):
    """Algorithmic bytes of moe_grouped_ffn_gelu per call, averaged over the cycled batches: the
    active experts' W1 and W2 (bf16) and biases (fp32), x read, hidden rows written and read, expert
    rows written."""
    T, d, H, k = cfg.T, cfg.d, cfg.H, cfg.k
    rows = T * k
    tot = 0
    for counts in counts_list:
        n_act = int((counts > 0).sum())
        tot += n_act * (2 * 2 * H * d + 4 * (H + d)) + 2 * T * d + 2 * 2 * rows * H + 2 * rows * d
    return tot / len(counts_list)


def cpu_baseline_gelu(cfg, host, n_tokens, min_seconds=10.0, max_repeats=8):
    """The fp64 oracle of the GELU-expert layer on a bounded sample of tokens (weight generation
    excluded; the bf16 -> fp64 conversion of the selected experts is timed)."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = None
    E, H, d = cfg.E, cfg.H, cfg.d
    rng = np.random.default_rng(1)
    tokens = np.sort(rng.choice(cfg.T, size=min(n_tokens, cfg.T), replace=False))
    x = oracle.widen(host.x[tokens], cfg.dtype)
    wg = oracle.widen(host.w_router, cfg.dtype)
    _, idx, _ = oracle.route(x, wg, cfg.k, host.router_bias, cfg.routing)
    sid = lambda i: synth.stream_id(synth.K_GELU, i)  # noqa: E731
    raw = {int(e): (synth.normal_host((H, d), 0, sid(0), 1.0 / np.sqrt(d), "bf16", first=int(e) * H * d),
                    synth.normal_host((H,), 0, sid(2), 0.1, "f32", first=int(e) * H),
                    synth.normal_host((d, H), 0, sid(1), 1.0 / np.sqrt(H), "bf16", first=int(e) * d * H),
                    synth.normal_host((d,), 0, sid(3), 0.1, "f32", first=int(e) * d))
           for e in np.unique(idx)}   # untimed
    expert_fn = lambda e: (oracle.widen(raw[e][0], "bf16"), raw[e][1].astype(np.float64),  # noqa: E731
                           oracle.widen(raw[e][2], "bf16"), raw[e][3].astype(np.float64))
    reps, total = 0, 0.0
    while reps < max_repeats and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        ref = oracle.layer_forward_gelu(x, wg, cfg.k, expert_fn, host.router_bias, cfg.routing)
        total += time.perf_counter() - t0
        reps += 1
    assert ref["out"].shape == (len(tokens), d)
    return {"value": round(len(tokens) * reps / total, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sampled": True, "sample_tokens": int(len(tokens)), "workload_tokens": cfg.T,
            "sample": f"{len(tokens)} of {cfg.T} tokens of {cfg.name} with GELU experts, {reps} passes in "
                      f"{total:.1f} s (routing, bf16->fp64 conversion of the {len(raw)} selected experts, "
                      f"GELU experts, combine; expert weight generation excluded)"}


def main_gelu(args, cfg, K, W):
    """The layer with two-layer GELU experts: moe_route, moe_permute, moe_grouped_ffn_gelu and
    moe_combine per step; the timed steps carry hipEvents around the expert stage (its two kernels)."""
    import numpy as np
    import torch

    import synth
    import sparse_moe_layer_router_amd as moe

    if cfg.dtype != "bf16" or args.layout in ("int8", "fp8"):
        print("--expert gelu runs bf16 layers with row-major or fragment-tiled weights", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    E, H, d = cfg.E, cfg.H, cfg.d
    t_setup = time.perf_counter()
    w1 = torch.empty(E, H, d, dtype=torch.bfloat16, device=dev)
    w2 = torch.empty(E, d, H, dtype=torch.bfloat16, device=dev)
    b1 = torch.empty(E, H, dtype=torch.float32, device=dev)
    b2 = torch.empty(E, d, dtype=torch.float32, device=dev)
    for i, (t, std) in enumerate(((w1, 1.0 / np.sqrt(d)), (w2, 1.0 / np.sqrt(H)), (b1, 0.1), (b2, 0.1))):
        synth.normal_device(t, 0, synth.stream_id(synth.K_GELU, i), std)
    layout = moe.MOE_LAYOUT_ROWMAJOR
    if args.layout == "frag16" and d % 32 == 0 and H % 32 == 0:
        p1, p2 = torch.empty_like(w1), torch.empty_like(w2)
        moe.moe_pack_weights(w1, p1, E, H, d)
        moe.moe_pack_weights(w2, p2, E, d, H)
        torch.cuda.synchronize()
        w1, w2, layout = p1, p2, moe.MOE_LAYOUT_FRAG16
        torch.cuda.empty_cache()
    host = synth.host_small_inputs(cfg, 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    w_router = up(host.w_router)
    bias = torch.from_numpy(host.router_bias).to(dev) if host.router_bias is not None else None
    xs = [up(host.x)] + [up(synth.normal_host((cfg.T, d), 100 + b, synth.stream_id(synth.K_X), 1.0, "bf16"))
                         for b in range(1, N_BATCHES)]
    shape = moe.make_shape(cfg.T, d, E, cfg.k, H, 0, "bf16", layout, cfg.routing)
    bufs = [moe.gelu_layer_buffers(shape, dev) for _ in range(N_BATCHES)]
    outs = [torch.empty(cfg.T, d, dtype=torch.bfloat16, device=dev) for _ in range(N_BATCHES)]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    def step(i, ev=None, e0=0):
        bf, x = bufs[i % N_BATCHES], xs[i % N_BATCHES]
        moe.moe_route(shape, x, w_router, bias, None, bf["idx"], bf["w"], bf["workspace"], stream)
        moe.moe_permute(shape, bf["idx"], bf["counts"], bf["offsets"], bf["perm_src"], bf["inv_perm"],
                        bf["workspace"], stream)
        if ev is not None:
            ev.record(e0, stream.cuda_stream)
        moe.moe_grouped_ffn_gelu(shape, x, bf["perm_src"], bf["offsets"], w1, b1, w2, b2, bf["y"],
                                 bf["workspace"], stream)
        if ev is not None:
            ev.record(e0 + 1, stream.cuda_stream)
        moe.moe_combine(shape, bf["y"], bf["inv_perm"], bf["w"], None, outs[i % N_BATCHES], stream)

    for i in range(max(W, N_BATCHES)):
        step(i)
    torch.cuda.synchronize()
    # per-step distribution (cold caches: a 1 GiB evicting copy between steps, outside the events)
    n_dist = 30
    flush_src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_dst = torch.empty_like(flush_src)
    ev_d = HipEvents(2 * n_dist)
    for i in range(n_dist):
        flush_dst.copy_(flush_src)
        ev_d.record(2 * i, stream.cuda_stream)
        step(i)
        ev_d.record(2 * i + 1, stream.cuda_stream)
    torch.cuda.synchronize()
    step_ms = [ev_d.elapsed_ms(2 * i, 2 * i + 1) for i in range(n_dist)]
    ev_d.close()
    del flush_src, flush_dst
    # timed steps: events around the expert stage only
    ev = HipEvents(2 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, ev, 2 * i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ffn_ms = sum(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)) / K
    ev.close()
    counts_np = [bf["counts"].cpu().numpy() for bf in bufs]
    byt = gelu_alg_bytes(cfg, counts_np)
    flops = 4 * cfg.T * cfg.k * d * H          # two linears of 2 rows d H flops each
    achieved = byt / (ffn_ms * 1e-3) / 1e9
    kname = moe.moe_gelu_kernel_name(shape, 0) + " + " + moe.moe_gelu_kernel_name(shape, 1)
    prefill = cfg.T * cfg.k / cfg.E > 32        # the grouped-GEMM regime: against the bf16 MFMA peak
    if prefill:
        tf = flops / (ffn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    roof.update({"kernel": kname, "kernel_ms": round(ffn_ms, 4), "traffic": traffic_for(cfg.name + "_gelu", kname)})
    ms_per_step = elapsed * 1e3 / K
    line = {
        "metric": METRIC, "value": round(cfg.T * K / elapsed, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Philox normal draws; random-init weights of the named layer shape)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": d, "n_experts": E, "top_k": cfg.k, "d_hidden": H,
                   "d_shared_hidden": 0, "expert": "gelu (two linears with bias)", "routing": cfg.routing,
                   "weight_layout": "frag16" if layout == moe.MOE_LAYOUT_FRAG16 else "rowmajor",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"ffn_alg_bytes": int(byt), "ffn_alg_flops": int(flops),
                  "ffn_hbm_GBps": round(achieved, 1), "ffn_tflops": round(flops / (ffn_ms * 1e-3) / 1e12, 2),
                  "active_experts_mean": float(np.mean([(c > 0).sum() for c in counts_np]))},
        "step_ms_events": {"mean": round(statistics.mean(step_ms), 4), "std": round(statistics.pstdev(step_ms), 4),
                           "median": round(statistics.median(step_ms), 4), "steps": n_dist,
                           "between_steps": "1 GiB device copy (L2 and Infinity Cache evicted)"},
        "setup_s": round(t_setup, 1),
    }
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_gelu(
        cfg, host, args.cpu_sample_tokens or (8 if cfg.E > 8 else 16))
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------------------------- measured roofs
def measure_ceilings(dev, read_gib=4, mfma_iters=40000, reps=7, expert_cfg=None):
    """What this GPU sustains, from the library's probes (include/moe_calib.h), timed with HIP
    events on the launch stream (medians over ``reps``): a streaming read of a ``read_gib`` GiB
    buffer with and without the non-temporal hint, a device copy (read + write), and a register-only
    bf16 MFMA loop, two waves per SIMD, on random and on constant operands, with the shader clock
    each ran at (from the counters each wave reads at its start and end). With ``expert_cfg`` (a
    layer of many rows per expert) also the vendor GEMM on that layer's expert work: see
    ``library_expert_gemm``."""
    import torch
    import sparse_moe_layer_router_amd as moe

    stream = torch.cuda.current_stream(dev)
    nbytes = read_gib << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
    sink_r = torch.empty(moe.MOE_CALIB_READ_BLOCKS, dtype=torch.int32, device=dev)
    ev = HipEvents(2 * reps)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        for i in range(reps):
            ev.record(2 * i, stream.cuda_stream)
            fn()
            ev.record(2 * i + 1, stream.cuda_stream)
        torch.cuda.synchronize()
        return statistics.median(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps))

    out = {}
    for nt in (True, False):
        ms = timed(lambda: moe.moe_calib_read_stream(buf, sink_r, nt, stream))
        out["read_nontemporal_GBps" if nt else "read_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    half = buf[: buf.numel() // 2]
    dst = torch.empty_like(half)
    ms = timed(lambda: dst.copy_(half))
    out["copy_GBps"] = round(2 * half.numel() * 4 / (ms * 1e-3) / 1e9, 1)   # read + write
    del buf, half, dst
    n_ops = moe.MOE_CALIB_MFMA_BLOCKS * 512 * 16
    sink_m = torch.empty(moe.MOE_CALIB_MFMA_BLOCKS, dtype=torch.float32, device=dev)
    clocks = torch.zeros(moe.MOE_CALIB_MFMA_BLOCKS * 8 * 4, dtype=torch.int64, device=dev)
    flops = moe.MOE_CALIB_MFMA_BLOCKS * 8 * mfma_iters * 8 * 32768
    gen = torch.Generator(device=dev).manual_seed(0)
    for name, ops in (("random", torch.randn(n_ops, generator=gen, device=dev).to(torch.bfloat16)),
                      ("constant", torch.ones(n_ops, dtype=torch.bfloat16, device=dev))):
        ms = timed(lambda: moe.moe_calib_mfma(ops, mfma_iters, sink_m, clocks, stream))
        c = clocks.view(-1, 4).cpu().double()
        ghz = ((c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * 0.1).median().item()   # real-time counter: 100 MHz
        out[f"mfma_bf16_{name}_TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 1)
        out[f"mfma_bf16_{name}_clock_GHz"] = round(ghz, 3)
    ev.close()
    out["note"] = (f"read/copy: {read_gib} GiB; MFMA: {moe.MOE_CALIB_MFMA_BLOCKS} workgroups x 8 waves, "
                   f"{mfma_iters} x 8 32x32x16 bf16 MFMAs per wave; medians of {reps} event-timed runs")
    torch.cuda.empty_cache()
    if expert_cfg is not None:
        out["library_expert_gemm"] = library_expert_gemm(expert_cfg, dev, 10)
    return out


def library_expert_gemm(cfg, dev, reps=7):
    """The vendor GEMM (torch.bmm, which dispatches to hipBLASLt) on the expert work of ``cfg`` made
    as easy as it gets: every routed expert holding exactly T*k/E rows, already gathered into
    contiguous [E, M, d] blocks, no shared expert, no activation epilogue. Two batched products per
    layer, each expert with its own weights streamed from HBM: gate and up as one [M, d] x [d, 2H]
    product per expert, and down as [M, H] x [H, d]. Right operands are contiguous (never a
    transposed view). Timed like the probes, with more warm-up (the library's first calls run
    slower, 4.1 -> 3.6 ms over the first eight gate/up calls in a trace): three untimed calls, then
    ``reps`` calls between HIP events on the current stream, median."""
    import torch

    E, d, H = cfg.E, cfg.d, cfg.H
    M = round(cfg.T * cfg.k / E)
    stream = torch.cuda.current_stream(dev)
    ev = HipEvents(2 * reps)
    gen = torch.Generator(device=dev).manual_seed(1)
    res = {"shape": f"{E} experts x {M} rows, d={d}, H={H} (uniform buckets, contiguous rows)"}
    for name, (m, kk, n) in (("gate_up", (M, d, 2 * H)), ("down", (M, H, d))):
        a = torch.randn(E, m, kk, generator=gen, device=dev, dtype=torch.bfloat16)
        b = torch.randn(E, kk, n, generator=gen, device=dev, dtype=torch.bfloat16)
        c = torch.empty(E, m, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.bmm(a, b, out=c)
        torch.cuda.synchronize()
        for i in range(reps):
            ev.record(2 * i, stream.cuda_stream)
            torch.bmm(a, b, out=c)
            ev.record(2 * i + 1, stream.cuda_stream)
        torch.cuda.synchronize()
        ms = statistics.median(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps))
        tflops = 2.0 * E * m * kk * n / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "TFLOPs": round(tflops, 1), "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
        del a, b, c
        torch.cuda.empty_cache()
    ev.close()
    return res


# ----------------------------------------------------------------------------------------- main
DECODE_SUBRECORDS = ("dsv3_decode_t8", "dsv3_decode_t256")   # same layer and weights as the prefill chunk


def make_weights(args, cfg, dev):
    """Expert weights of ``cfg`` drawn in device memory and, before any timing, put in the layout the
    bench runs (fragment-tiled, or per-row INT8 or FP8): one-time preparation, like a model load."""
    import torch
    import synth
    import sparse_moe_layer_router_amd as moe
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[cfg.dtype]
    E, H, d = cfg.E, cfg.H, cfg.d
    wgt = torch.empty(E, H, d, dtype=dt, device=dev)
    wup = torch.empty(E, H, d, dtype=dt, device=dev)
    wdn = torch.empty(E, d, H, dtype=dt, device=dev)
    shared = None
    if cfg.Hs:
        shared = (torch.empty(cfg.Hs, d, dtype=dt, device=dev), torch.empty(cfg.Hs, d, dtype=dt, device=dev),
                  torch.empty(d, cfg.Hs, dtype=dt, device=dev))
    synth.fill_expert_weights_device(cfg, 0, wgt, wup, wdn, shared)
    layout = moe.MOE_LAYOUT_ROWMAJOR
    if args.layout in ("int8", "fp8"):
        if cfg.dtype != "bf16" or cfg.d % 64 or cfg.H % 64 or cfg.Hs % 64:
            print(f"--layout {args.layout} needs a bf16 layer with d, H, Hs multiples of 64 ({cfg.name} is not)",
                  file=sys.stderr)
            sys.exit(2)
        quant = moe.quantize_expert_weights(wgt, wup, wdn, shared, fp8=args.layout == "fp8")
        torch.cuda.synchronize()
        wgt, wup, wdn = quant[:3]
        shared = tuple(quant[3:]) if shared else None
        layout = moe.MOE_LAYOUT_FP8_FRAG if args.layout == "fp8" else moe.MOE_LAYOUT_INT8_FRAG
        del quant
        torch.cuda.empty_cache()
    elif args.layout == "frag16" and cfg.dtype == "bf16" and cfg.d % 32 == 0 and cfg.H % 32 == 0 and cfg.Hs % 32 == 0:
        packed = moe.pack_expert_weights(wgt, wup, wdn, shared)
        torch.cuda.synchronize()
        wgt, wup, wdn = packed[:3]
        shared = tuple(packed[3:]) if shared else None
        layout = moe.MOE_LAYOUT_FRAG16
        del packed
        torch.cuda.empty_cache()
    return (wgt, wup, wdn, shared), layout


def run_layer_bench(cfg, K, W, weights, layout, dev):
    """One workload on resident weights: warm-up, a per-stage event pass, a cold-cache distribution
    pass, then K timed steps with events around the dominant kernel only. Returns the measurement
    (without the CPU baseline) and the host inputs."""
    import numpy as np
    import torch

    import synth
    import sparse_moe_layer_router_amd as moe

    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[cfg.dtype]
    es = 2 if cfg.dtype == "bf16" else 4
    prefill = cfg.T * cfg.k / cfg.E > 32
    wgt, wup, wdn, shared = weights
    d, E = cfg.d, cfg.E
    host = synth.host_small_inputs(cfg, 0)

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    w_router = up(host.w_router)
    bias = torch.from_numpy(host.router_bias).to(dev) if host.router_bias is not None else None
    xs = [up(host.x)] + [up(synth.normal_host((cfg.T, d), 100 + b, synth.stream_id(synth.K_X), 1.0, cfg.dtype))
                         for b in range(1, N_BATCHES)]
    shape = moe.make_shape(cfg.T, d, E, cfg.k, cfg.H, cfg.Hs, cfg.dtype, layout, cfg.routing)
    ws = moe.allocate_workspace(shape)
    outs = [torch.empty(cfg.T, d, dtype=dt, device=dev) for _ in range(N_BATCHES)]
    counts = [torch.zeros(E, dtype=torch.int32, device=dev) for _ in range(N_BATCHES)]
    sg, su, sd = shared if shared else (None, None, None)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step(i, events=None):
        b = i % N_BATCHES
        if events is None:
            moe.moe_layer_forward(shape, xs[b], w_router, bias, wgt, wup, wdn, sg, su, sd, outs[b],
                                  counts_out=counts[b], workspace=ws, stream=stream)
        else:
            moe.moe_layer_forward_timed(shape, xs[b], w_router, bias, wgt, wup, wdn, sg, su, sd, outs[b],
                                        counts_out=counts[b], workspace=ws, stream=stream, events=events)

    for i in range(max(W, N_BATCHES)):
        step(i)
    torch.cuda.synchronize()

    # Per-stage breakdown: an untimed pass with events around every stage (each event record costs
    # GPU time, so the timed steps below carry only the two around the dominant kernel).
    n_st = moe.MOE_NUM_STAGES
    n_prof = min(K, 10)
    ev_all = HipEvents(2 * n_st * n_prof)
    for i in range(n_prof):
        step(i, ev_all.array(2 * n_st * i, 2 * n_st))
    torch.cuda.synchronize()
    stage_ms = {}
    for s in range(n_st):
        durs = [ev_all.elapsed_ms(2 * n_st * i + 2 * s, 2 * n_st * i + 2 * s + 1) for i in range(n_prof)]
        stage_ms[moe.STAGES[s]] = sum(durs) / n_prof
    ev_all.close()
    # Per-step distribution of the whole layer: an untimed pass of 30 steps with one event pair per
    # step (at the first stage's start and the last stage's end), for mean, standard deviation and
    # median. Between steps, outside the event pairs, a 1 GiB device-to-device copy evicts L2 and
    # the 256 MB Infinity Cache, so every step starts cold; the copies, timed with their own events,
    # also give a measured large-copy HBM bandwidth.
    n_dist = 30
    flush_src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_dst = torch.empty_like(flush_src)
    ev_d = HipEvents(4 * n_dist)
    slots_d = [(ctypes.c_void_p * (2 * n_st))() for _ in range(n_dist)]
    for i in range(n_dist):
        slots_d[i][0] = ev_d.ev[2 * i]
        slots_d[i][2 * n_st - 1] = ev_d.ev[2 * i + 1]
    torch.cuda.synchronize()
    for i in range(n_dist):
        ev_d.record(2 * n_dist + 2 * i, stream.cuda_stream)
        flush_dst.copy_(flush_src)
        ev_d.record(2 * n_dist + 2 * i + 1, stream.cuda_stream)
        step(i, ctypes.cast(slots_d[i], ctypes.POINTER(ctypes.c_void_p)))
    torch.cuda.synchronize()
    step_ms = [ev_d.elapsed_ms(2 * i, 2 * i + 1) for i in range(n_dist)]
    copy_ms = statistics.median(ev_d.elapsed_ms(2 * n_dist + 2 * i, 2 * n_dist + 2 * i + 1) for i in range(n_dist))
    ev_d.close()
    del flush_src, flush_dst
    copy_GBps = 2 * FLUSH_BYTES / (copy_ms * 1e-3) / 1e9   # read + write
    step_dist = {"mean": round(statistics.mean(step_ms), 4), "std": round(statistics.pstdev(step_ms), 4),
                 "median": round(statistics.median(step_ms), 4), "steps": n_dist,
                 "between_steps": "1 GiB device copy (L2 and Infinity Cache evicted)"}

    dominant = max(("ffn_gate_up", "ffn_down"), key=lambda s_: stage_ms[s_])
    dom = moe.STAGES.index(dominant)

    # Timed steps: hipEvents on the launch stream just around the dominant kernel, nothing else.
    ev = HipEvents(2 * K)
    slots = [(ctypes.c_void_p * (2 * n_st))() for _ in range(K)]
    for i in range(K):
        slots[i][2 * dom] = ev.ev[2 * i]
        slots[i][2 * dom + 1] = ev.ev[2 * i + 1]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, ctypes.cast(slots[i], ctypes.POINTER(ctypes.c_void_p)))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kms = sum(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)) / K
    ev.close()

    counts_np = [c.cpu().numpy() for c in counts]
    work = alg_bytes_and_flops(cfg, counts_np, es, one_byte=layout in (moe.MOE_LAYOUT_INT8_FRAG, moe.MOE_LAYOUT_FP8_FRAG))
    ms_per_step = elapsed * 1e3 / K
    kname = moe.moe_stage_kernel_name(shape, dom)
    if prefill:
        flops = work["flops_gate_up" if dominant == "ffn_gate_up" else "flops_down"]
        achieved = flops / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        byt = work["gate_up" if dominant == "ffn_gate_up" else "down"]
        achieved = byt / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    roof["kernel"] = kname
    roof["kernel_ms"] = round(kms, 4)
    roof["traffic"] = traffic_for(cfg.name, kname)
    if roof["bound"] == "hbm":   # the same kernel against the large-copy bandwidth measured above
        roof["measured_copy_GBps"] = round(copy_GBps, 1)
        roof["frac_of_measured_copy"] = round(achieved / copy_GBps, 4)
    # both expert kernels from the per-stage pass, against the roofline of the regime
    kernels = {}
    for st_, wkey, fkey in (("ffn_gate_up", "gate_up", "flops_gate_up"), ("ffn_down", "down", "flops_down")):
        ms_ = stage_ms[st_]
        kernels[st_] = {"kernel": moe.moe_stage_kernel_name(shape, moe.STAGES.index(st_)), "ms": round(ms_, 4),
                        "TFLOPs": round(work[fkey] / (ms_ * 1e-3) / 1e12, 2),
                        "GBps": round(work[wkey] / (ms_ * 1e-3) / 1e9, 1)}
        kernels[st_]["frac"] = round(kernels[st_]["TFLOPs"] / BF16_PEAK_TFLOPS if prefill
                                     else kernels[st_]["GBps"] / HBM_PEAK_GBPS, 4)

    rec = {
        "value": round(cfg.T * K / elapsed, 2),
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E, "top_k": cfg.k,
                   "d_hidden": cfg.H, "d_shared_hidden": cfg.Hs, "zipf_bias": cfg.zipf_s, "routing": cfg.routing,
                   "weight_layout": {moe.MOE_LAYOUT_FRAG16: "frag16", moe.MOE_LAYOUT_INT8_FRAG: "int8 per-row",
                                     moe.MOE_LAYOUT_FP8_FRAG: "fp8 e4m3 per-row",
                                     moe.MOE_LAYOUT_ROWMAJOR: "rowmajor"}[layout],
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"alg_bytes": int(work["layer"]), "alg_flops": int(work["flops_layer"]),
                  "hbm_GBps": round(work["layer"] / (ms_per_step * 1e-3) / 1e9, 1),
                  "tflops": round(work["flops_layer"] / (ms_per_step * 1e-3) / 1e12, 2),
                  "active_experts_mean": work["n_act"], "expert_kernels": kernels},
        "stage_ms": {k_: round(v, 4) for k_, v in stage_ms.items()},   # untimed pass, events on every stage
        "step_ms_events": step_dist,   # untimed pass, cold caches, events around each whole layer call
    }
    del ws, outs, xs
    torch.cuda.empty_cache()
    return rec, host


def ep_share_rows(cfg, G, weights_dtype, dev):
    """The rows one GPU of G receives in an expert-parallel layer: G batches of T tokens (one per GPU)
    are routed and permuted by the layer's own kernels; GPU 0 holds experts [0, E/G) and receives
    every row routed to them, which the dispatch places in local-expert order (each source's rows of
    an expert contiguous, the sources in rank order). Returns the received rows [R, d], the local
    bucket offsets [E/G + 1] and the per-expert counts (host)."""
    import numpy as np
    import torch

    import synth
    import sparse_moe_layer_router_amd as moe

    El = cfg.E // G
    host = synth.host_small_inputs(cfg, 0)
    dt = weights_dtype
    w_router = torch.from_numpy(np.ascontiguousarray(host.w_router).view(np.int16)).view(torch.bfloat16).to(dev)
    bias = torch.from_numpy(host.router_bias).to(dev) if host.router_bias is not None else None
    shape = moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.H, cfg.Hs, cfg.dtype, moe.MOE_LAYOUT_ROWMAJOR, cfg.routing)
    ws = moe.allocate_workspace(shape)
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev)
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    tw = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device=dev)
    cnt = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    offs = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(cfg.T * cfg.k, dtype=torch.int32, device=dev)
    inv = torch.empty(cfg.T * cfg.k, dtype=torch.int32, device=dev)
    chunks = [[] for _ in range(El)]
    for g in range(G):
        x = torch.empty(cfg.T, cfg.d, dtype=dt, device=dev)
        synth.normal_device(x, 300 + g, synth.stream_id(synth.K_X), 1.0)
        moe.moe_route(shape, x, w_router, bias, logits, idx, tw, ws)
        moe.moe_permute(shape, idx, cnt, offs, perm, inv, ws)
        o = offs.cpu().numpy()
        for e in range(El):
            src = (perm[int(o[e]):int(o[e + 1])] // cfg.k).long()
            chunks[e].append(x.index_select(0, src))
        del x
    rows = [torch.cat(c) for c in chunks]
    counts = np.array([r.shape[0] for r in rows], dtype=np.int64)
    xr = torch.cat(rows).contiguous()
    del rows, chunks, ws
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return xr, offsets, counts


def main_ep_share(args, cfg, K, W):
    """Expert stage of one GPU of ``args.ep_share`` in expert parallel, at the prefill size per GPU:
    moe_grouped_ffn over the GPU's E/G experts and the rows routed to them from all G batches, then
    the shared expert over the GPU's own T tokens (a second moe_grouped_ffn; in a full layer it can
    run while the dispatch exchange is in flight). The exchange itself is not part of this build.
    One JSON line: the expert stage's tokens/s (the GPU's own T tokens per stage time) and the routed
    call (schedule, gate/up and down launches) against the bf16 MFMA peak."""
    import torch

    import synth
    import sparse_moe_layer_router_amd as moe

    G = args.ep_share
    if cfg.dtype != "bf16" or args.layout not in ("frag16", "rowmajor") or cfg.E % G or args.expert != "swiglu":
        print("--ep-share needs a bf16 SwiGLU layer, --layout frag16 or rowmajor, and G dividing E", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    El = cfg.E // G
    (wgt, wup, wdn, shared), layout = make_weights(args, cfg, dev)
    wgt, wup, wdn = wgt[:El], wup[:El], wdn[:El]   # experts [0, E/G): contiguous prefixes
    xr, offs, counts = ep_share_rows(cfg, G, wgt.dtype, dev)
    R = int(counts.sum())
    s_r = moe.make_shape(R, cfg.d, El, 1, cfg.H, 0, cfg.dtype, layout, cfg.routing)
    ws_r = moe.allocate_workspace(s_r)
    y_r = torch.empty(R, cfg.d, dtype=wgt.dtype, device=dev)
    x_own = torch.empty(cfg.T, cfg.d, dtype=wgt.dtype, device=dev)
    synth.normal_device(x_own, 300, synth.stream_id(synth.K_X), 1.0)
    s_s = moe.make_shape(cfg.T, cfg.d, 1, 1, cfg.Hs, 0, cfg.dtype, layout, cfg.routing)
    ws_s = moe.allocate_workspace(s_s)
    offs_s = torch.tensor([0, cfg.T], dtype=torch.int32, device=dev)
    y_s = torch.empty(cfg.T, cfg.d, dtype=wgt.dtype, device=dev)
    sg, su, sd = shared
    stream = torch.cuda.current_stream(dev)

    def routed():
        moe.moe_grouped_ffn(s_r, xr, None, offs, wgt, wup, wdn, y_r, ws_r, stream)

    def shared_ffn():
        moe.moe_grouped_ffn(s_s, x_own, None, offs_s, sg, su, sd, y_s, ws_s, stream)

    for _ in range(W):
        routed()
        shared_ffn()
    torch.cuda.synchronize()
    ev = HipEvents(4 * K)
    t0 = time.perf_counter()
    for i in range(K):
        ev.record(4 * i, stream.cuda_stream)
        routed()
        ev.record(4 * i + 1, stream.cuda_stream)
        ev.record(4 * i + 2, stream.cuda_stream)
        shared_ffn()
        ev.record(4 * i + 3, stream.cuda_stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    r_ms = statistics.median(ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(K))
    s_ms = statistics.median(ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(K))
    ev.close()
    flops_r = 6.0 * R * cfg.d * cfg.H
    flops_s = 6.0 * cfg.T * cfg.d * cfg.Hs
    ach = flops_r / (r_ms * 1e-3) / 1e12
    kname = " + ".join(moe.moe_stage_kernel_name(s_r, moe.STAGES.index(st)) for st in ("ffn_gate_up", "ffn_down"))
    line = {"metric": "expert-stage tokens/s of one GPU's expert-parallel share", "value": round(cfg.T * K / elapsed, 2),
            "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(elapsed * 1e3 / K, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
            "data": "synthetic (seeded Philox normal draws; random-init weights of the named layer shape)",
            "config": {"workload": f"{cfg.name}_ep{G}_share", "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E,
                       "top_k": cfg.k, "d_hidden": cfg.H, "d_shared_hidden": cfg.Hs, "ep_degree": G,
                       "local_experts": El, "received_rows": R,
                       "rows_per_expert": {"min": int(counts.min()), "mean": round(float(counts.mean()), 1),
                                           "max": int(counts.max())},
                       "weight_layout": "frag16" if layout == moe.MOE_LAYOUT_FRAG16 else "rowmajor",
                       "parallelism": f"one GPU's share of ep{G} (the exchange not included)"},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / BF16_PEAK_TFLOPS, 4), "kernel": kname, "kernel_ms": round(r_ms, 4),
                         "kernel_scope": "the routed moe_grouped_ffn call (schedule, gate/up and down launches)",
                         "traffic": None},
            "shared_expert": {"ms": round(s_ms, 4), "TFLOPs": round(flops_s / (s_ms * 1e-3) / 1e12, 2)},
            "cpu_baseline": None}
    print(json.dumps(line), flush=True)


def sub_record(rec):
    """The decode figures carried next to the headline: step time, tokens/s and the dominant
    kernel against the HBM roofline (with its counter traffic when the summary is current)."""
    r = rec["roofline"]
    return {"workload": rec["config"]["workload"], "T": rec["config"]["T"], "steps": rec["steps"],
            "ms_per_step": rec["ms_per_step"], "tokens_per_s": rec["value"], "kernel": r["kernel"],
            "kernel_ms": r["kernel_ms"], "bound": r["bound"], "achieved": r["achieved"], "unit": r["unit"],
            "frac": r["frac"], "traffic": r["traffic"], "layer_hbm_GBps": rec["layer"]["hbm_GBps"],
            "stage_ms": rec["stage_ms"], "step_ms_events": rec["step_ms_events"]}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (expert-parallel "
              "all-to-all is out of scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if args.ceilings:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        c = synth.CONFIG_BY_NAME[args.workload]
        many_rows = c.dtype == "bf16" and c.T * c.k / c.E > 32
        print(json.dumps({"ceilings": measure_ceilings(dev, expert_cfg=c if many_rows else None)}), flush=True)
        return
    cfg = synth.CONFIG_BY_NAME[args.workload]
    prefill = cfg.T * cfg.k / cfg.E > 32
    K = args.steps if args.steps is not None else (30 if prefill else 50)
    W = args.warmup if args.warmup is not None else 5
    if args.ep_share:
        return main_ep_share(args, cfg, K, W)
    if args.expert == "gelu":
        return main_gelu(args, cfg, K, W)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_setup = time.perf_counter()
    weights, layout = make_weights(args, cfg, dev)
    t_setup = time.perf_counter() - t_setup
    rec, host = run_layer_bench(cfg, K, W, weights, layout, dev)
    line = {"metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": cfg.dtype,
            "data": "synthetic (seeded Philox normal draws; random-init weights of the named layer shape)"}
    line.update({k_: rec[k_] for k_ in ("config", "roofline", "layer", "stage_ms", "step_ms_events")})
    line["setup_s"] = round(t_setup, 1)
    # The decode half of the metric, on the same weights: the DeepSeek-V3-shaped layer at T = 8 and 256.
    same_layer = lambda c: (c.d, c.E, c.k, c.H, c.Hs, c.dtype, c.routing) == (  # noqa: E731
        cfg.d, cfg.E, cfg.k, cfg.H, cfg.Hs, cfg.dtype, cfg.routing)
    if not args.no_decode:
        subs = {}
        for name in DECODE_SUBRECORDS:
            c = synth.CONFIG_BY_NAME[name]
            if name != cfg.name and same_layer(c):
                subs[name] = sub_record(run_layer_bench(c, 50, 5, weights, layout, dev)[0])
        if subs:
            line["decode"] = subs
    if not args.no_ceilings:   # measured after the layer runs, so they do not disturb them
        ceil = measure_ceilings(dev, expert_cfg=cfg if prefill and cfg.dtype == "bf16" else None)
        line["ceilings"] = ceil
        rf = line["roofline"]
        if rf["bound"] == "mfma":
            rf["measured_mfma_random_TFLOPs"] = ceil["mfma_bf16_random_TFLOPs"]
            rf["frac_of_measured_mfma"] = round(rf["achieved"] / ceil["mfma_bf16_random_TFLOPs"], 4)
            lib = ceil.get("library_expert_gemm")
            if lib and args.expert == "swiglu":   # the dominant kernel is the gate/up pass
                rf["library_gate_up_TFLOPs"] = lib["gate_up"]["TFLOPs"]
                rf["frac_of_library"] = round(rf["achieved"] / lib["gate_up"]["TFLOPs"], 4)
        else:
            rf["measured_read_GBps"] = ceil["read_nontemporal_GBps"]
            rf["frac_of_measured_read"] = round(rf["achieved"] / ceil["read_nontemporal_GBps"], 4)
        for sub in line.get("decode", {}).values():
            sub["frac_of_measured_read"] = round(sub["achieved"] / ceil["read_nontemporal_GBps"], 4)
    if not args.no_cpu_baseline:
        n_tok = args.cpu_sample_tokens or (8 if cfg.E > 8 else 16)
        line["cpu_baseline"] = cpu_baseline(cfg, host, n_tok, quant=args.layout if args.layout in ("int8", "fp8") else None)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

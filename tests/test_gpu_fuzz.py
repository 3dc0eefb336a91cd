"""Small-shape fuzz of the whole layer against the oracle (needs an MI355X).

Sixty layers drawn from a fixed seed over the shape space the C ABI accepts: token counts on every
path (the single-block decode tail up to 16 tokens, one wave per token above, the router GEMM from
2048), 1 to 300 experts, top-k up to 12, model and hidden sizes that are multiples of 8 (and of 32
or 64 where the weight layout needs it), with or without a shared expert, bf16 or float32, softmax
or sigmoid routing, and every weight layout the sizes allow. Each layer: routing and permutation
bit-exact on the GPU's own logits, logits and outputs within the layer tolerance of the oracle.
"""

import numpy as np
import pytest

import oracle
from synth import LayerConfig
from tests import gpu_util as G
from tests.test_gpu_parity import check_logits_close, check_routing_on_gpu_logits

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu

LAYOUTS = {"rowmajor": moe.MOE_LAYOUT_ROWMAJOR, "frag16": moe.MOE_LAYOUT_FRAG16,
           "int8": moe.MOE_LAYOUT_INT8_FRAG, "fp8": moe.MOE_LAYOUT_FP8_FRAG}


def draw_cases(n=60, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        path = rng.choice(["tail", "wave", "gemm", "router_gemm"])
        E = int(rng.choice([1, 2, 3, 8, 16, 37, 64, 129, 300]))
        k = int(rng.integers(1, min(E, 12) + 1))
        if path == "tail":
            T = int(rng.integers(1, 17))
        elif path == "wave":
            T = int(rng.integers(17, 400))
        elif path == "gemm":       # at least 32 rows per expert on average: the grouped GEMM
            T = int(max(17, min(1500, -(-32 * E // k) + rng.integers(0, 300))))
        else:
            T = int(rng.integers(2048, 2300))
        dtype = "bf16" if rng.random() < 0.8 else "f32"
        align = int(rng.choice([8, 32, 64])) if dtype == "bf16" else 8
        d = align * int(rng.integers(1, 256 // align + 1))
        H = align * int(rng.integers(1, 192 // align + 1))
        Hs = 0 if rng.random() < 0.4 else align * int(rng.integers(1, 128 // align + 1))
        routing = "sigmoid" if rng.random() < 0.3 else "softmax"
        layouts = ["rowmajor"]
        if dtype == "bf16" and d % 32 == 0 and H % 32 == 0 and Hs % 32 == 0:
            layouts.append("frag16")
        if dtype == "bf16" and d % 64 == 0 and H % 64 == 0 and Hs % 64 == 0:
            layouts += ["int8", "fp8"]
        layout = str(rng.choice(layouts))
        # keep the float64 oracle within a second or two per layer
        if T * k * d * H > 6e8 or T * d * Hs > 3e8:
            continue
        name = f"fz{len(cases):02d}_{path}_T{T}_d{d}_E{E}_k{k}_H{H}_Hs{Hs}_{dtype}_{routing}_{layout}"
        cfg = LayerConfig(name, T, d, E, k, H, Hs, dtype, routing=routing,
                          score_bias_std=0.05 if routing == "sigmoid" else None)
        cases.append((cfg, layout))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("cfg,layout", CASES, ids=[c.name for c, _ in CASES])
def test_layer_fuzz(cfg, layout):
    print(f"[{cfg.name}] moe_layer_forward", flush=True)
    L = G.make_layer(cfg, layout=LAYOUTS[layout])
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward(x, wg, cfg.k, L.expert_fn(), L.shared_fn(), b, cfg.routing)
    np.testing.assert_array_equal(np.sort(r.idx.cpu().numpy(), 1), np.sort(ref["idx"], 1))
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out), ref["out"])
    assert ok, (err, bound)

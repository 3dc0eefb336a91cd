"""INT8 expert weights (MOE_LAYOUT_INT8_FRAG) on the GPU vs the oracle (needs an MI355X).

Quantization codes and scales are integers and floats decided by float32 arithmetic, so the GPU's
are compared bit for bit with the oracle's (the packed byte order is rebuilt here from the
documented layout formula). Layers with INT8 experts are compared with the oracle run on the
dequantized weights q * s, to the same tolerance as the bf16 layers.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import LayerConfig
from tests import gpu_util as G
from tests.test_gpu_parity import check_logits_close, check_routing_on_gpu_logits

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu


def packed_reference(q: np.ndarray) -> np.ndarray:
    """Codes [n, rows, cols] in the MOE_LAYOUT_INT8_FRAG byte order (moe.h, moe_quantize_weights)."""
    n, rows, cols = q.shape
    m, r, c = np.indices(q.shape)
    lane = (r % 16) + 16 * ((c % 32) // 8)
    pos = (m * rows * cols + ((r // 16) * (cols // 64) + c // 64) * 1024 + lane * 16 + ((c % 64) // 32) * 8
           + c % 8)
    out = np.empty(n * rows * cols, np.int8)
    out[pos.reshape(-1)] = q.reshape(-1)
    return out


@pytest.mark.parametrize("n,rows,cols", [(1, 16, 64), (3, 48, 192), (1, 2048, 7168)])
def test_quantize_weights_bit_exact(n, rows, cols):
    rng = np.random.default_rng(rows + cols)
    w = (rng.standard_normal((n, rows, cols)) * rng.uniform(1e-3, 3.0, (n, rows, 1))).astype(np.float32)
    w[0, 5 % rows] = 0.0                              # an all-zero row: scale 0, codes 0
    if rows > 20:
        w[-1, 17, :7] = [0.5, -0.5, 1.5, 2.5, -2.5, 127.0, -127.0]   # halves and the extremes
    wb = torch.from_numpy(w).to(torch.bfloat16)
    dev = wb.cuda()
    buf = torch.empty(moe.moe_quantized_weight_bytes(n, rows, cols), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_weights(dev, buf, n, rows, cols)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    q_o, s_o = oracle.quantize_rows_int8(wb.float().numpy().astype(np.float64))
    ncode = n * rows * cols
    np.testing.assert_array_equal(got[:ncode].view(np.int8), packed_reference(q_o))
    np.testing.assert_array_equal(got[ncode:].view(np.float32).reshape(n, rows).view(np.uint32),
                                  s_o.view(np.uint32))


INT8 = [
    LayerConfig("int8_mid_shared", 40, 256, 16, 4, 128, 64, "bf16"),
    LayerConfig("int8_zipf", 64, 512, 64, 6, 256, 0, "bf16", zipf_s=1.2),
    LayerConfig("int8_sigmoid_fused", 12, 128, 64, 6, 64, 64, "bf16", routing="sigmoid", score_bias_std=0.05),
    # grouped GEMM (>= 32 rows per expert): 150 rows per expert, a partial N-tile (H = 192 = 128 + 64)
    # and a down pass over three K pairs (K = 192)
    LayerConfig("int8_many_rows", 600, 256, 8, 2, 192, 128, "bf16"),
    # grouped GEMM: ~600 rows per expert (two M-tiles), one K pair in gate/up (d = 64), skew
    LayerConfig("int8_gemm_two_mtiles", 1200, 64, 4, 2, 256, 0, "bf16", zipf_s=0.8),
    # grouped GEMM: shared expert of four M-tiles over 1000 tokens, two K pairs (d = 128)
    LayerConfig("int8_gemm_shared", 1000, 128, 16, 2, 128, 192, "bf16"),
    # grouped GEMM: d = 320, a partial 256-wide N-tile in the down pass (bands and scales past d
    # never used) and five K pairs in gate/up (the pair ring wraps)
    LayerConfig("int8_gemm_ragged_d", 600, 320, 8, 2, 128, 64, "bf16"),
]


def expected_stage_names(cfg, code):
    """The expert kernels the layer runs: the grouped GEMM from 32 rows per expert, else streaming."""
    if cfg.T * cfg.k / cfg.E >= 32:
        return f"grouped_gemm_kernel<0, {code}>", f"grouped_gemm_kernel<1, {code}>"
    if cfg.T <= 16:   # gate and up in separate waves
        return f"ffn_gate_up_stream_pair<1, {code}>", f"ffn_down_stream<1, {code}>"
    return f"ffn_gate_up_stream_wide<{code}>", f"ffn_down_stream_wide<{code}>"   # 32 weight rows per wave


@pytest.mark.parametrize("cfg", INT8, ids=lambda c: c.name)
def test_layer_int8_weights_match_oracle(cfg):
    L = G.make_layer(cfg, layout=moe.MOE_LAYOUT_INT8_FRAG)
    gu, dn = expected_stage_names(cfg, 2)
    assert moe.moe_stage_kernel_name(L.shape, moe.STAGES.index("ffn_gate_up")) == gu
    assert moe.moe_stage_kernel_name(L.shape, moe.STAGES.index("ffn_down")) == dn
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward(x, wg, cfg.k, L.expert_fn(), L.shared_fn(), b, cfg.routing)
    np.testing.assert_array_equal(np.sort(r.idx.cpu().numpy(), 1), np.sort(ref["idx"], 1))
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out), ref["out"])
    assert ok, (err, bound)


def test_int8_layer_stays_close_to_bf16_layer():
    """Per-row INT8 weights move the output by about the rounding of the codes, far less than the
    output itself (a sanity check of the scale direction; the oracle comparison is the parity test)."""
    cfg = INT8[0]
    Lb = G.make_layer(cfg)
    Lq = G.make_layer(cfg, layout=moe.MOE_LAYOUT_INT8_FRAG)
    ob, oq = G.to_f64(G.run_layer(Lb).out), G.to_f64(G.run_layer(Lq).out)
    rel = np.abs(oq - ob).max() / np.abs(ob).max()
    assert 1e-4 < rel < 0.05, rel

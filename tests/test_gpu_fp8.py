"""FP8 (E4M3) expert weights (MOE_LAYOUT_FP8_FRAG) on the GPU vs the oracle (needs an MI355X).

The codes are decided by float32 arithmetic (the row scale max|w| / 448, the division, then the
nearest E4M3 value), so the GPU's codes and scales are compared bit for bit with the oracle's (the
byte order is the INT8 layout's, rebuilt from its documented formula). Layers with FP8 experts
are compared with the oracle run on the decoded weights value(q) * s, to the layer tolerance, at
mid sizes here and at the DeepSeek-V3 decode sizes in the full-size module.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import LayerConfig
from tests import gpu_util as G
from tests.test_gpu_int8 import expected_stage_names, packed_reference
from tests.test_gpu_parity import check_logits_close, check_routing_on_gpu_logits

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,rows,cols", [(1, 16, 64), (3, 48, 192), (1, 2048, 7168)])
def test_quantize_weights_fp8_bit_exact(n, rows, cols):
    rng = np.random.default_rng(rows + cols + 1)
    w = (rng.standard_normal((n, rows, cols)) * rng.uniform(1e-3, 3.0, (n, rows, 1))).astype(np.float32)
    w[0, 5 % rows] = 0.0                                   # an all-zero row: scale 0, codes 0
    w[-1, 2 % rows, :3] = [-0.0, 1e-30, -1e-30]            # signed zero and values far below the grid
    if rows > 20:
        # the row maximum 448 s, a tie between codes, a subnormal tie, a value at the subnormal edge
        w[-1, 17, :5] = [448.0, 1.0625, 1.5 * 2.0 ** -9, 7.5 * 2.0 ** -9, -3.5]
    wb = torch.from_numpy(w).to(torch.bfloat16)
    buf = torch.empty(moe.moe_quantized_weight_bytes(n, rows, cols), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_weights_fp8(wb.cuda(), buf, n, rows, cols)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    q_o, s_o = oracle.quantize_rows_fp8(wb.float().numpy().astype(np.float64))
    ncode = n * rows * cols
    np.testing.assert_array_equal(got[:ncode].view(np.int8), packed_reference(q_o.view(np.int8)))
    np.testing.assert_array_equal(got[ncode:].view(np.float32).reshape(n, rows).view(np.uint32),
                                  s_o.view(np.uint32))


@pytest.mark.parametrize("layout", ["int8", "fp8"])
def test_dequantize_every_code_bit_exact(layout):
    """Every byte value at many positions and under row scales of many sizes (0 among them): the
    decode the weight-streaming kernels run, times the scale in float32, against the oracle's
    value(q) * s (exact in float64, so one rounding to float32 is the float32 product). The two NaN
    codes of E4M3 must give NaN."""
    n, rows, cols = 2, 32, 256
    rng = np.random.default_rng(7)
    codes = rng.permutation(np.tile(np.arange(256, dtype=np.uint8), n * rows * cols // 256)).reshape(n, rows, cols)
    s = (2.0 ** rng.integers(-20, 12, (n, rows)) * rng.uniform(1.0, 2.0, (n, rows))).astype(np.float32)
    s[0, 3] = 0.0
    s[1, 0] = 1.0
    buf = np.empty(n * rows * cols + 4 * n * rows, np.uint8)
    buf[:n * rows * cols] = packed_reference(codes.view(np.int8)).view(np.uint8)
    buf[n * rows * cols:] = s.reshape(-1).view(np.uint8)
    dst = torch.empty(n, rows, cols, dtype=torch.float32, device="cuda")
    code = {"int8": moe.MOE_LAYOUT_INT8_FRAG, "fp8": moe.MOE_LAYOUT_FP8_FRAG}[layout]
    moe.moe_dequantize_weights(torch.from_numpy(buf).cuda(), code, dst, n, rows, cols)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    if layout == "int8":
        want = oracle.dequantize_rows_int8(codes.view(np.int8), s)
    else:
        want = oracle.dequantize_rows_fp8(codes, s)
    want = want.astype(np.float32)
    nan = np.isnan(want)
    assert nan.sum() == (2 * n * rows * cols // 256 if layout == "fp8" else 0)   # codes 0x7F and 0xFF
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


FP8 = [
    LayerConfig("fp8_mid_shared", 40, 256, 16, 4, 128, 64, "bf16"),
    LayerConfig("fp8_zipf", 64, 512, 64, 6, 256, 0, "bf16", zipf_s=1.2),
    LayerConfig("fp8_sigmoid_fused", 12, 128, 64, 6, 64, 64, "bf16", routing="sigmoid", score_bias_std=0.05),
    # grouped GEMM cases, as for INT8: a partial N-tile and three K pairs; two M-tiles and one K
    # pair; a shared expert of four M-tiles and two K pairs
    LayerConfig("fp8_many_rows", 600, 256, 8, 2, 192, 128, "bf16"),
    LayerConfig("fp8_gemm_two_mtiles", 1200, 64, 4, 2, 256, 0, "bf16", zipf_s=0.8),
    LayerConfig("fp8_gemm_shared", 1000, 128, 16, 2, 128, 192, "bf16"),
    # grouped GEMM: d = 320, a partial 256-wide N-tile in the down pass (bands and scales past d
    # never used) and five K pairs in gate/up (the pair ring wraps)
    LayerConfig("fp8_gemm_ragged_d", 600, 320, 8, 2, 128, 64, "bf16"),
]


@pytest.mark.parametrize("cfg", FP8, ids=lambda c: c.name)
def test_layer_fp8_weights_match_oracle(cfg):
    L = G.make_layer(cfg, layout=moe.MOE_LAYOUT_FP8_FRAG)
    gu, dn = expected_stage_names(cfg, 3)
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


def test_fp8_layer_stays_close_to_bf16_layer():
    """E4M3 codes keep 3 mantissa bits: the output moves by about their rounding, far less than the
    output itself (a sanity check of the scale and decoding; the oracle comparison is the parity test)."""
    cfg = FP8[0]
    Lb = G.make_layer(cfg)
    Lq = G.make_layer(cfg, layout=moe.MOE_LAYOUT_FP8_FRAG)
    ob, oq = G.to_f64(G.run_layer(Lb).out), G.to_f64(G.run_layer(Lq).out)
    rel = np.abs(oq - ob).max() / np.abs(ob).max()
    assert 1e-3 < rel < 0.15, rel

"""The two-layer GELU expert variant on the GPU (moe_grouped_ffn_gelu and the layer composed of
moe_route, moe_permute, moe_grouped_ffn_gelu and moe_combine) against the oracle (needs an MI355X).

Inputs: the seeded activations and router of a LayerConfig (near-ties in the top-k redrawn, as for
the SwiGLU layer), expert weights W1 [E, H, d] ~ N(0, 1/d) and W2 [E, d, H] ~ N(0, 1/H) in bf16 and
biases b1, b2 ~ N(0, 0.1^2) in float32, each from a seeded stream of its own. Comparison: routing
bit-exact, outputs within max|gpu - oracle| <= 1e-2 max|oracle| + 1e-3 (the layer tolerance).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as G
from tests import helpers

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu

CONFIGS = [
    synth.LayerConfig("gelu_decode", 8, 256, 16, 4, 128, 0, "bf16"),
    synth.LayerConfig("gelu_ragged", 300, 264, 16, 2, 200, 0, "bf16"),          # d % 32 and H % 16 != 0
    synth.LayerConfig("gelu_many_rows", 2048, 512, 8, 2, 384, 0, "bf16", zipf_s=1.2),
    synth.LayerConfig("gelu_sigmoid", 40, 128, 32, 6, 64, 0, "bf16", routing="sigmoid", score_bias_std=0.05),
    # grouped-GEMM path with many groups: ~256 rows per expert (one M-tile, some spilling into a
    # second), partial N-tiles of both passes (H = 192 < 256)
    synth.LayerConfig("gelu_gemm_groups", 4096, 256, 64, 4, 192, 0, "bf16"),
    # the shapes of the overview article's layer example (section 4.1): model width 768, 8 experts
    # of width 3072, top-2, a batch of 2 sequences of 10 tokens (20 rows)
    synth.LayerConfig("gelu_overview_example", 20, 768, 8, 2, 3072, 0, "bf16"),
]
CASES = [(c, moe.MOE_LAYOUT_ROWMAJOR) for c in CONFIGS] + \
        [(c, moe.MOE_LAYOUT_FRAG16) for c in CONFIGS if c.d % 32 == 0 and c.H % 32 == 0]


def gelu_weights(cfg, seed, with_bias=True):
    """Host copies (bf16 bits / float32) of W1, b1, W2, b2."""
    E, H, d = cfg.E, cfg.H, cfg.d
    w1 = synth.normal_host((E, H, d), seed, synth.stream_id(synth.K_GELU, 0), 1.0 / np.sqrt(d), "bf16")
    w2 = synth.normal_host((E, d, H), seed, synth.stream_id(synth.K_GELU, 1), 1.0 / np.sqrt(H), "bf16")
    b1 = synth.normal_host((E, H), seed, synth.stream_id(synth.K_GELU, 2), 0.1, "f32") if with_bias else None
    b2 = synth.normal_host((E, d), seed, synth.stream_id(synth.K_GELU, 3), 0.1, "f32") if with_bias else None
    return w1, b1, w2, b2


def device_weights(cfg, host_w, layout):
    w1, b1, w2, b2 = host_w
    dw1, dw2 = G.to_dev(w1, "bf16"), G.to_dev(w2, "bf16")
    if layout == moe.MOE_LAYOUT_FRAG16:
        p1, p2 = torch.empty_like(dw1), torch.empty_like(dw2)
        moe.moe_pack_weights(dw1, p1, cfg.E, cfg.H, cfg.d)
        moe.moe_pack_weights(dw2, p2, cfg.E, cfg.d, cfg.H)
        dw1, dw2 = p1, p2
    db1 = torch.from_numpy(b1).cuda() if b1 is not None else None
    db2 = torch.from_numpy(b2).cuda() if b2 is not None else None
    return dw1, db1, dw2, db2


def oracle_experts(host_w):
    w1, b1, w2, b2 = host_w
    W1, W2 = oracle.widen(w1, "bf16"), oracle.widen(w2, "bf16")
    return lambda e: (W1[e], None if b1 is None else b1[e].astype(np.float64), W2[e],
                      None if b2 is None else b2[e].astype(np.float64))


def shape_of(cfg, layout):
    return moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.H, 0, "bf16", layout, cfg.routing)


@pytest.mark.parametrize("cfg,layout", CASES, ids=lambda v: v.name if hasattr(v, "name") else
                         {moe.MOE_LAYOUT_ROWMAJOR: "rowmajor", moe.MOE_LAYOUT_FRAG16: "frag16"}[v])
def test_gelu_layer_matches_oracle(cfg, layout):
    host = synth.host_small_inputs(cfg, 0)
    helpers.screen_gaps(host)
    hw = gelu_weights(cfg, 0)
    w1, b1, w2, b2 = device_weights(cfg, hw, layout)
    s = shape_of(cfg, layout)
    x = G.to_dev(host.x, "bf16")
    wr = G.to_dev(host.w_router, "bf16")
    bias = torch.from_numpy(host.router_bias).cuda() if host.router_bias is not None else None
    buf = moe.gelu_layer_buffers(s)
    out = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward_gelu(s, x, wr, bias, w1, b1, w2, b2, out, buf)
    torch.cuda.synchronize()
    ref = oracle.layer_forward_gelu(oracle.widen(host.x, "bf16"), oracle.widen(host.w_router, "bf16"), cfg.k,
                                    oracle_experts(hw), host.router_bias, cfg.routing)
    np.testing.assert_array_equal(buf["idx"].cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(buf["perm_src"].cpu().numpy(), ref["perm_src"])
    ok, err, bound = G.tolerance_ok(G.to_f64(buf["y"]), ref["y_perm"])
    assert ok, ("expert rows", err, bound)
    ok, err, bound = G.tolerance_ok(G.to_f64(out), ref["out"])
    assert ok, ("layer output", err, bound)


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_ROWMAJOR, moe.MOE_LAYOUT_FRAG16], ids=["rowmajor", "frag16"])
def test_gelu_ffn_on_given_rows_without_bias(layout):
    """perm_src NULL (x holds the rows in bucket order), no biases, ragged buckets incl. empty ones."""
    cfg = synth.LayerConfig("gelu_rows", 40, 192, 6, 1, 96, 0, "bf16")
    hw = gelu_weights(cfg, 3, with_bias=False)
    w1, b1, w2, b2 = device_weights(cfg, hw, layout)
    counts = np.array([0, 17, 1, 0, 22, 0])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = synth.normal_host((cfg.T, cfg.d), 7, synth.stream_id(synth.K_GELU, 9), 1.0, "bf16")
    s = shape_of(cfg, layout)
    y = torch.full((cfg.T, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_ffn_gelu(s, G.to_dev(rows, "bf16"), None, torch.from_numpy(offsets).cuda(), w1, b1, w2, b2, y,
                             moe.allocate_workspace(s))
    torch.cuda.synchronize()
    ref = oracle.grouped_ffn_gelu(oracle.widen(rows, "bf16"), offsets, oracle_experts(hw))
    ok, err, bound = G.tolerance_ok(G.to_f64(y), ref)
    assert ok, (err, bound)


def test_gelu_layer_is_deterministic_and_empty_batch_is_a_no_op():
    cfg = CONFIGS[2]
    host = synth.host_small_inputs(cfg, 0)
    w1, b1, w2, b2 = device_weights(cfg, gelu_weights(cfg, 0), moe.MOE_LAYOUT_FRAG16)
    s = shape_of(cfg, moe.MOE_LAYOUT_FRAG16)
    x, wr = G.to_dev(host.x, "bf16"), G.to_dev(host.w_router, "bf16")
    bias = torch.from_numpy(host.router_bias).cuda()
    buf = moe.gelu_layer_buffers(s)
    outs = []
    for _ in range(2):
        out = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")
        moe.moe_layer_forward_gelu(s, x, wr, bias, w1, b1, w2, b2, out, buf)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    s0 = moe.make_shape(0, cfg.d, cfg.E, cfg.k, cfg.H, 0, "bf16", moe.MOE_LAYOUT_FRAG16)
    moe.moe_grouped_ffn_gelu(s0, None, None, None, None, None, None, None, None, None)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_sample", [("dsv3_decode_t8", None), ("dsv3_decode_t256", 6),
                                           ("dsv3_prefill_t8192", "structural")])
def test_gelu_layer_full_size(name, n_sample):
    """The DeepSeek-V3-shaped layer with GELU experts (d 7168, 256 experts of hidden 2048, top-8,
    no shared expert) at the decode sizes (weight streaming) and the prefill chunk (grouped GEMM),
    fragment-tiled weights drawn in device memory as the benchmark does; the oracle regenerates on
    the host only the experts the checked tokens select. At the prefill size the checked tokens hold
    the first and last row of every M-tile of every expert bucket."""
    base = synth.CONFIG_BY_NAME[name]
    cfg = synth.LayerConfig(name + "_gelu", base.T, base.d, base.E, base.k, base.H, 0, "bf16")
    E, H, d = cfg.E, cfg.H, cfg.d
    host = synth.host_small_inputs(cfg, 0)
    helpers.screen_gaps(host)
    w = [torch.empty(E, H, d, dtype=torch.bfloat16, device="cuda"), torch.empty(E, d, H, dtype=torch.bfloat16, device="cuda"),
         torch.empty(E, H, dtype=torch.float32, device="cuda"), torch.empty(E, d, dtype=torch.float32, device="cuda")]
    for i, (t, std) in enumerate(zip(w, (1.0 / np.sqrt(d), 1.0 / np.sqrt(H), 0.1, 0.1))):
        synth.normal_device(t, 0, synth.stream_id(synth.K_GELU, i), std)
    p1, p2 = torch.empty_like(w[0]), torch.empty_like(w[1])
    moe.moe_pack_weights(w[0], p1, E, H, d)
    moe.moe_pack_weights(w[1], p2, E, d, H)
    del w[:2]
    b1, b2 = w
    s = shape_of(cfg, moe.MOE_LAYOUT_FRAG16)
    buf = moe.gelu_layer_buffers(s)
    out = torch.empty(cfg.T, d, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward_gelu(s, G.to_dev(host.x, "bf16"), G.to_dev(host.w_router, "bf16"), None, p1, b1, p2, b2,
                               out, buf)
    torch.cuda.synchronize()
    del p1, p2
    if n_sample is None:
        tokens = np.arange(cfg.T)
    elif n_sample == "structural":
        idx, counts = buf["idx"].cpu().numpy(), buf["counts"].cpu().numpy()
        tokens = helpers.structural_tokens(idx, cfg.T, 0)
        helpers.assert_tile_edges_covered(idx, counts, tokens, cfg.T, 0)
    else:
        tokens = np.unique(np.concatenate([[0, cfg.T - 1], np.random.default_rng(0).choice(cfg.T, n_sample - 2,
                                                                                            replace=False)]))
    print(f"[{cfg.name}] kernels {moe.moe_gelu_kernel_name(s, 0)} + {moe.moe_gelu_kernel_name(s, 1)}; "
          f"{len(tokens)} checked tokens", flush=True)
    sid = lambda i: synth.stream_id(synth.K_GELU, i)  # noqa: E731

    seen = []

    def expert(e):
        seen.append(e)
        if len(seen) % 32 == 0:
            print(f"  oracle: {len(seen)} experts", flush=True)
        return (oracle.widen(synth.normal_host((H, d), 0, sid(0), 1.0 / np.sqrt(d), "bf16", first=e * H * d), "bf16"),
                synth.normal_host((H,), 0, sid(2), 0.1, "f32", first=e * H).astype(np.float64),
                oracle.widen(synth.normal_host((d, H), 0, sid(1), 1.0 / np.sqrt(H), "bf16", first=e * d * H), "bf16"),
                synth.normal_host((d,), 0, sid(3), 0.1, "f32", first=e * d).astype(np.float64))

    ref = oracle.layer_forward_gelu(oracle.widen(host.x[tokens], "bf16"), oracle.widen(host.w_router, "bf16"), cfg.k,
                                    expert, None, cfg.routing)
    np.testing.assert_array_equal(np.sort(buf["idx"].cpu().numpy()[tokens], 1), np.sort(ref["idx"], 1))
    ok, err, bound = G.tolerance_ok(G.to_f64(out)[tokens], ref["out"])
    assert ok, (err, bound)

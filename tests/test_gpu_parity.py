"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Contract: with the oracle's selection run on the GPU's own float32 logits, top-k ids (with order),
counts, offsets, perm_src and inv_perm are bit-exact and the weights agree within 1e-5. End to
end on gap-screened inputs (every token's k-th and (k+1)-th fp64 router scores differ by at
least 1e-4), the selected sets match exactly and the output satisfies
max|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3 over the whole tensor (or over the sampled
tokens at the full DeepSeek-V3 and Mixtral sizes, where each token is checked one by one).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import LayerConfig
from tests import gpu_util as G

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu

# Mid-size layers the oracle finishes in seconds: several blocks of H and d, ragged tails (d and H
# multiples of 8 but not of 32 / 64), more than one permutation tile, a shared expert of another size.
MID = [
    LayerConfig("mid_ragged_shared", 300, 264, 16, 4, 200, 136, "bf16"),
    LayerConfig("mid_zipf_bias", 64, 512, 64, 6, 256, 0, "bf16", zipf_s=1.2),
    LayerConfig("mid_fp32_shared", 50, 96, 8, 3, 40, 24, "f32"),
    LayerConfig("single_expert_k1", 5, 64, 1, 1, 32, 0, "bf16"),
    LayerConfig("k_equals_E", 20, 128, 4, 4, 64, 32, "bf16"),
    LayerConfig("k12_wide_topk", 40, 128, 32, 12, 64, 32, "bf16"),  # combine with more than 8 slots
    LayerConfig("one_token", 1, 256, 32, 8, 128, 64, "bf16"),
    # a decode batch (gate and up in separate waves) whose hidden sizes end inside a 16-row group and
    # whose d ends inside a 32-wide k-step
    LayerConfig("decode_ragged_shared", 12, 264, 16, 4, 200, 136, "bf16"),
    LayerConfig("wide_E1024", 40, 64, 1024, 2, 16, 0, "bf16"),
    # the smallest sizes the ABI takes (d, H, Hs = 8: a single K chunk shorter than a k-step or a
    # GEMM slice) on the decode tail, the grouped GEMM and the router GEMM
    LayerConfig("tiny_dims_decode", 5, 8, 4, 2, 8, 8, "bf16"),
    LayerConfig("tiny_dims_gemm", 600, 8, 2, 1, 8, 8, "bf16"),
    LayerConfig("tiny_dims_router_gemm", 2048, 8, 4, 2, 16, 0, "bf16"),
    synth.CONFIGS[0],
    # many rows per expert: tiled MFMA grouped GEMM (K tails of 8, partial N and M tiles)
    LayerConfig("gemm_ragged_shared", 600, 264, 16, 2, 200, 136, "bf16"),
    # 2048 tokens: router GEMM too (E = 8 < one N tile), skewed buckets
    LayerConfig("gemm_zipf_router", 2048, 512, 8, 2, 384, 0, "bf16", zipf_s=1.2),
    # 1024 routed experts + the shared one: more than 1024 groups (two-round tile schedule) and more
    # than 1024 tiles per pass (XCD ranges balanced by work); the router GEMM over four N tiles
    LayerConfig("gemm_many_groups", 16384, 64, 1024, 2, 32, 32, "bf16"),
    # skewed buckets of several M-tiles each and more than 1024 gate/up tiles (XCD ranges balanced
    # by work, bounds falling between the M-tiles of one N-tile)
    LayerConfig("gemm_balanced_zipf", 4096, 512, 8, 2, 4608, 0, "bf16", zipf_s=1.2),
    # sigmoid routing with a selection-only bias: one-wave-per-token top-k with the grouped GEMM,
    # the single-block decode tail, float32 without a bias, and the router GEMM
    LayerConfig("sigmoid_mid_shared", 300, 264, 16, 4, 200, 136, "bf16", routing="sigmoid", score_bias_std=0.05),
    LayerConfig("sigmoid_small_fused", 12, 128, 64, 6, 64, 32, "bf16", routing="sigmoid", score_bias_std=0.05),
    LayerConfig("sigmoid_fp32_nobias", 50, 96, 8, 3, 40, 24, "f32", routing="sigmoid"),
    LayerConfig("sigmoid_gemm_router", 2048, 512, 8, 2, 384, 0, "bf16", routing="sigmoid", score_bias_std=0.05),
]


MID_BY_NAME = {c.name: c for c in MID}


def pick(*names):
    """Configs of MID by name (a missing name fails at collection)."""
    return [MID_BY_NAME[n] for n in names]


def check_routing_on_gpu_logits(L, r):
    """Oracle selection and permutation applied to the GPU's own logits: bit-exact."""
    c = L.cfg
    lg = r.logits.cpu().numpy().astype(np.float64)
    if c.routing == "sigmoid":
        idx_o = oracle.select_topk(oracle.selection_scores(lg, "sigmoid", L.host.score_bias), c.k)
        w_o = oracle.sigmoid_weights_selected(lg, idx_o)
    else:
        idx_o = oracle.select_topk(lg, c.k)
        w_o = oracle.softmax_selected(lg, idx_o)
    np.testing.assert_array_equal(r.idx.cpu().numpy(), idx_o)
    np.testing.assert_allclose(r.w.cpu().numpy(), w_o, rtol=0, atol=1e-5)
    counts_o, offsets_o, perm_o, inv_o = oracle.permute(idx_o, c.E)
    np.testing.assert_array_equal(r.counts.cpu().numpy(), counts_o)
    # the permutation entry point on the same ids
    s = L.shape
    offs = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    cnt = torch.empty(c.E, dtype=torch.int32, device="cuda")
    perm = torch.empty(c.T * c.k, dtype=torch.int32, device="cuda")
    inv = torch.empty(c.T * c.k, dtype=torch.int32, device="cuda")
    moe.moe_permute(s, r.idx, cnt, offs, perm, inv, moe.allocate_workspace(s))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cnt.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(offs.cpu().numpy(), offsets_o)
    np.testing.assert_array_equal(perm.cpu().numpy(), perm_o)
    np.testing.assert_array_equal(inv.cpu().numpy(), inv_o)
    return offs, perm, inv


def check_logits_close(L, r):
    x, wg, b = G.oracle_inputs(L)
    lg_o = oracle.router_logits(x, wg, b if L.cfg.routing == "softmax" else None)
    err = np.abs(r.logits.cpu().numpy() - lg_o).max()
    assert err < 1e-4 + 1e-5 * np.abs(lg_o).max(), err


@pytest.mark.parametrize("cfg", MID, ids=lambda c: c.name)
def test_layer_matches_oracle_mid_sizes(cfg):
    L = G.make_layer(cfg)
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward(x, wg, cfg.k, L.expert_fn(), L.shared_fn(), b, cfg.routing)
    # gap-screened: the selected sets agree with the oracle's own fp64 routing
    np.testing.assert_array_equal(np.sort(r.idx.cpu().numpy(), 1), np.sort(ref["idx"], 1))
    np.testing.assert_array_equal(r.counts.cpu().numpy(), ref["counts"])
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out), ref["out"])
    assert ok, (err, bound)


@pytest.mark.parametrize("cfg", pick("mid_ragged_shared", "mid_zipf_bias", "mid_fp32_shared", "gemm_ragged_shared",
                                      "gemm_zipf_router", "gemm_many_groups", "sigmoid_mid_shared",
                                      "sigmoid_fp32_nobias", "sigmoid_gemm_router"), ids=lambda c: c.name)
def test_entry_points_separately(cfg):
    """moe_route -> moe_permute -> moe_grouped_ffn (routed, then shared as a one-group call) -> moe_combine."""
    L = G.make_layer(cfg)
    s = L.shape
    c = cfg
    dt = G.TORCH_DT[c.dtype]
    ws = moe.allocate_workspace(s)
    idx = torch.empty(c.T, c.k, dtype=torch.int32, device="cuda")
    w = torch.empty(c.T, c.k, dtype=torch.float32, device="cuda")
    moe.moe_route(s, L.x, L.w_router, L.bias, None, idx, w, ws)
    offs = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(c.T * c.k, dtype=torch.int32, device="cuda")
    inv = torch.empty(c.T * c.k, dtype=torch.int32, device="cuda")
    moe.moe_permute(s, idx, None, offs, perm, inv, ws)
    y = torch.empty(c.T * c.k, c.d, dtype=dt, device="cuda")
    moe.moe_grouped_ffn(s, L.x, perm, offs, L.w_gate, L.w_up, L.w_down, y, ws)
    shared = None
    if c.Hs:
        s1 = moe.make_shape(c.T, c.d, 1, 1, c.Hs, 0, c.dtype)
        offs1 = torch.tensor([0, c.T], dtype=torch.int32, device="cuda")
        shared = torch.empty(c.T, c.d, dtype=dt, device="cuda")
        moe.moe_grouped_ffn(s1, L.x, None, offs1, L.ws_gate, L.ws_up, L.ws_down, shared, moe.allocate_workspace(s1))
    out = torch.empty(c.T, c.d, dtype=dt, device="cuda")
    moe.moe_combine(s, y, inv, w, shared, out)
    torch.cuda.synchronize()

    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward(x, wg, c.k, L.expert_fn(), L.shared_fn(), b, c.routing)
    np.testing.assert_array_equal(np.sort(idx.cpu().numpy(), 1), np.sort(ref["idx"], 1))
    # expert outputs row by row in dispatch order (the dispatch order of the GPU's own routing)
    idx_g = idx.cpu().numpy()
    counts_g, offs_g, perm_g, inv_g = oracle.permute(idx_g, c.E)
    y_ref = oracle.grouped_ffn(x[perm_g // c.k], offs_g, L.expert_fn())
    ok, err, bound = G.tolerance_ok(G.to_f64(y), y_ref)
    assert ok, ("grouped_ffn", err, bound)
    if c.Hs:
        ok, err, bound = G.tolerance_ok(G.to_f64(shared), ref["shared"])
        assert ok, ("shared", err, bound)
    ok, err, bound = G.tolerance_ok(G.to_f64(out), ref["out"])
    assert ok, ("out", err, bound)


# Decode-sized batches (T <= 16, T*k <= 4096) route and dispatch in one single-block kernel inside
# moe_layer_forward; the separate entry points keep the multi-kernel path. Both must agree bit for bit.
FUSED = [
    LayerConfig("fused_zipf", 16, 512, 64, 6, 256, 0, "bf16", zipf_s=1.2),
    LayerConfig("fused_E1024", 13, 64, 1024, 2, 16, 0, "bf16"),
    LayerConfig("fused_boundary_4096_slots", 16, 64, 256, 256, 32, 0, "bf16"),
    LayerConfig("fused_k_equals_E", 9, 128, 4, 4, 64, 0, "bf16"),
    LayerConfig("fused_one_token_f32", 1, 64, 8, 3, 32, 0, "f32"),
    LayerConfig("fused_sigmoid", 16, 256, 256, 8, 64, 0, "bf16", routing="sigmoid", score_bias_std=0.05),
]


@pytest.mark.parametrize("cfg", FUSED, ids=lambda c: c.name)
def test_fused_small_batch_dispatch_matches_entry_points(cfg):
    c = cfg
    s = moe.make_shape(c.T, c.d, c.E, c.k, c.H, c.Hs, c.dtype, routing=c.routing)
    assert moe.moe_stage_kernel_name(s, 1).startswith("route_tail_small_kernel<")
    L = G.make_layer(cfg)
    r = G.run_layer(L)
    dt = G.TORCH_DT[c.dtype]
    ws = moe.allocate_workspace(s)
    idx = torch.empty(c.T, c.k, dtype=torch.int32, device="cuda")
    w = torch.empty(c.T, c.k, dtype=torch.float32, device="cuda")
    moe.moe_route(s, L.x, L.w_router, L.bias, None, idx, w, ws)
    cnt = torch.empty(c.E, dtype=torch.int32, device="cuda")
    offs = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(c.T * c.k, dtype=torch.int32, device="cuda")
    inv = torch.empty(c.T * c.k, dtype=torch.int32, device="cuda")
    moe.moe_permute(s, idx, cnt, offs, perm, inv, ws)
    y = torch.empty(c.T * c.k, c.d, dtype=dt, device="cuda")
    moe.moe_grouped_ffn(s, L.x, perm, offs, L.w_gate, L.w_up, L.w_down, y, ws)
    out = torch.empty(c.T, c.d, dtype=dt, device="cuda")
    moe.moe_combine(s, y, inv, w, None, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r.idx.cpu().numpy(), idx.cpu().numpy())
    np.testing.assert_array_equal(r.w.cpu().numpy().view(np.uint32), w.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(r.counts.cpu().numpy(), cnt.cpu().numpy())
    # the layer's internal permutation fed the same experts in the same order: identical output bits
    np.testing.assert_array_equal(r.out.view(torch.int16 if c.dtype == "bf16" else torch.int32).cpu().numpy(),
                                  out.view(torch.int16 if c.dtype == "bf16" else torch.int32).cpu().numpy())
    check_routing_on_gpu_logits(L, r)


def test_permute_stress_patterns():
    """Skewed, duplicate and single-expert id patterns across many tiles: bit-exact."""
    rng = np.random.default_rng(0)
    cases = [
        (4096, 2, 8, np.full((4096, 2), 3)),                             # everything on one expert
        (20000, 3, 256, rng.integers(0, 256, (20000, 3))),                 # random, with duplicates
        (9000, 4, 1024, np.minimum(rng.zipf(1.5, (9000, 4)) - 1, 1023)),   # heavy head, long tail
        (1, 1, 1, np.zeros((1, 1))),
    ]
    for T, k, E, ids in cases:
        s = moe.make_shape(T, 64, E, k, 64, 0, "bf16")
        ids_t = torch.from_numpy(ids.astype(np.int32)).cuda()
        offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        cnt = torch.empty(E, dtype=torch.int32, device="cuda")
        perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
        inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
        moe.moe_permute(s, ids_t, cnt, offs, perm, inv, moe.allocate_workspace(s))
        torch.cuda.synchronize()
        c_o, o_o, p_o, i_o = oracle.permute(ids.astype(np.int64), E)
        np.testing.assert_array_equal(cnt.cpu().numpy(), c_o)
        np.testing.assert_array_equal(offs.cpu().numpy(), o_o)
        np.testing.assert_array_equal(perm.cpu().numpy(), p_o)
        np.testing.assert_array_equal(inv.cpu().numpy(), i_o)


def test_route_ties_go_to_lower_index():
    """Exactly tied logits (identical router rows) select the lower expert id first."""
    T, d, E, k = 8, 64, 16, 4
    x = torch.randn(T, d, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16).cuda()
    row = torch.randn(1, d, generator=torch.Generator().manual_seed(1))
    wr = row.repeat(E, 1).to(torch.bfloat16).cuda()          # all experts score the same
    bias = torch.zeros(E, dtype=torch.float32)
    bias[5] = bias[9] = 1.0                                  # two tied winners above the rest
    bias = bias.cuda()
    s = moe.make_shape(T, d, E, k, 64, 0, "bf16")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
    moe.moe_route(s, x, wr, bias, lg, idx, w, moe.allocate_workspace(s))
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == [[5, 9, 0, 1]] * T
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.select_topk(lg.cpu().numpy().astype(np.float64), k))


@pytest.mark.parametrize("T", [8, 40])   # the fused decode tail (T <= 16) and the one-wave-per-token kernel
def test_route_nan_and_inf_scores(T):
    """Logit biases holding NaN and -inf, through the whole layer: a NaN score orders like -inf
    (ties to the lower id), every token still gets k distinct ids, the selected -inf / NaN scores
    get weight 0 and the output stays finite. The ids equal the oracle's selection on the GPU's
    logits with NaN read as -inf."""
    d, E, k = 64, 16, 12
    x = torch.randn(T, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).cuda()
    wr = (torch.randn(E, d, generator=torch.Generator().manual_seed(3)) / 8).to(torch.bfloat16).cuda()
    bias = torch.zeros(E, dtype=torch.float32)
    bias[[0, 7, 12]] = -float("inf")
    bias[[3, 9, 14]] = float("nan")        # 10 finite scores: 2 of the 6 others are selected
    bias = bias.cuda()
    H = 64
    s = moe.make_shape(T, d, E, k, H, 0, "bf16")
    gen = torch.Generator().manual_seed(4)
    wgt, wup = ((torch.randn(E, H, d, generator=gen) / 8).to(torch.bfloat16).cuda() for _ in range(2))
    wdn = (torch.randn(E, d, H, generator=gen) / 8).to(torch.bfloat16).cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
    out = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward(s, x, wr, bias, wgt, wup, wdn, None, None, None, out, idx, w, None, lg,
                          moe.allocate_workspace(s))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ids, wt, L = idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy().astype(np.float64)
    assert np.isnan(L[:, [3, 9, 14]]).all() and np.isneginf(L[:, [0, 7, 12]]).all()
    assert all(len(set(r)) == k for r in ids.tolist()) and ids.min() >= 0 and ids.max() < E
    assert (ids[:, 10:] == [0, 3]).all()    # the two lowest ids of the -inf / NaN group
    Ln = np.where(np.isnan(L), -np.inf, L)
    np.testing.assert_array_equal(ids, oracle.select_topk(Ln, k))
    np.testing.assert_allclose(wt, oracle.softmax_selected(Ln, ids), rtol=0, atol=1e-5)
    assert (wt[:, 10:] == 0).all()


@pytest.mark.parametrize("routing", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E", [1, 3, 64, 65, 128, 200, 256, 300, 512, 777, 1024])
def test_topk_tie_heavy_every_lane_width(E, routing):
    """Router rows drawn from a handful of distinct vectors and biases from a few values, so most
    logits tie exactly; every candidates-per-lane width (E up to 64, 128, 256, 512, 1024), through
    both the one-wave-per-token kernel (T=40) and the single-block decode tail (T=9, via the layer)."""
    g = torch.Generator().manual_seed(E)
    d = 64
    protos = torch.randn(5, d, generator=g)
    wr = protos[torch.randint(0, 5, (E,), generator=g)].to(torch.bfloat16).cuda()
    bias = torch.tensor([0.0, 0.5, -0.25])[torch.randint(0, 3, (E,), generator=g)].float().cuda()
    for T in (40, 9):
        k = min(E, 9)
        x = torch.randn(T, d, generator=g).to(torch.bfloat16).cuda()
        s = moe.make_shape(T, d, E, k, 32, 0, "bf16", routing=routing)
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k, dtype=torch.float32, device="cuda")
        lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
        moe.moe_route(s, x, wr, bias, lg, idx, w, moe.allocate_workspace(s))
        torch.cuda.synchronize()
        lg64 = lg.cpu().numpy().astype(np.float64)
        if routing == "sigmoid":
            # the selection scores in the kernel's own precision (float32 sigmoid + bias), so that
            # the exact ties between experts sharing a router row and a bias stay exact
            a32 = (1.0 / (1.0 + np.exp(-lg.cpu().numpy().astype(np.float32)))).astype(np.float32)
            S = (a32 + bias.cpu().numpy()).astype(np.float32).astype(np.float64)
            idx_o = oracle.select_topk(S, k)
            w_o = oracle.sigmoid_weights_selected(lg64, idx_o)
        else:
            idx_o = oracle.select_topk(lg64, k)
            w_o = oracle.softmax_selected(lg64, idx_o)
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=0, atol=1e-6)
        if T <= 16:   # the layer's fused tail must select the same ids from the same logits
            wg = torch.zeros(E, 32, d, dtype=torch.bfloat16, device="cuda")
            wd = torch.zeros(E, d, 32, dtype=torch.bfloat16, device="cuda")
            out = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
            idx2 = torch.empty_like(idx)
            w2 = torch.empty_like(w)
            moe.moe_layer_forward(s, x, wr, bias, wg, wg, wd, None, None, None, out, idx2, w2,
                                  workspace=moe.allocate_workspace(s))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(idx2.cpu().numpy(), idx_o)
            np.testing.assert_array_equal(w2.cpu().numpy().view(np.uint32), w.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("cfg", pick("mid_ragged_shared", "mid_zipf_bias", "wide_E1024") + [synth.CONFIGS[0]],
                         ids=lambda c: c.name)
def test_load_stats_match_oracle(cfg):
    """Per-expert load and balance penalty of the GPU's own routing, against the oracle's."""
    L = G.make_layer(cfg)
    r = G.run_layer(L)
    load = torch.empty(cfg.E, dtype=torch.float32, device="cuda")
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    moe.moe_load_stats(L.shape, r.counts, 0.01, load, aux)
    aux2 = torch.empty(1, dtype=torch.float32, device="cuda")
    moe.moe_load_stats(L.shape, r.counts, 0.01, None, aux2)        # the load output is optional
    torch.cuda.synchronize()
    load_o, aux_o = oracle.load_stats(r.counts.cpu().numpy(), cfg.T, cfg.k, 0.01)
    np.testing.assert_allclose(load.cpu().numpy(), load_o, rtol=1e-6, atol=0)
    assert abs(aux.item() - aux_o) <= 1e-5 * aux_o + 1e-12, (aux.item(), aux_o)
    assert aux2.item() == aux.item()


def test_deterministic_bitwise():
    L = G.make_layer(MID[0])
    a = G.run_layer(L)
    b = G.run_layer(L)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.idx, b.idx) and torch.equal(a.w, b.w)


def test_empty_batch_is_a_no_op():
    cfg = synth.with_tokens(MID[0], 0)
    L = G.make_layer(cfg, screen=False)
    out = torch.full((0, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward(L.shape, L.x, L.w_router, None, L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up,
                          L.ws_down, out, workspace=moe.allocate_workspace(L.shape))
    torch.cuda.synchronize()


def test_device_generator_matches_host_bits():
    cfg = synth.CONFIG_BY_NAME["dsv3_decode_t8"]
    n = 3 * 100_003
    dev = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    synth.normal_device(dev, 0, synth.stream_id(synth.K_GATE, 17), synth.weight_std(cfg.d), nblk=3)
    host = synth.normal_host((3, 100_003), 0, synth.stream_id(synth.K_GATE, 17), synth.weight_std(cfg.d), "bf16",
                             nblk=3)
    assert np.array_equal(dev.view(torch.int16).cpu().numpy().view(np.uint16), host.reshape(-1))


# ------------------------------------------------------------------ fragment-tiled weights

def frag16_reference(w: np.ndarray) -> np.ndarray:
    """The packed layout built by array reshaping: [R, C] -> bands of 16 rows, blocks of 32
    columns, inside a block (chunk of 8 columns, row in band, 8 columns) -- lane = row + 16 chunk."""
    R, C = w.shape
    return w.reshape(R // 16, 16, C // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("n,rows,cols", [(1, 16, 32), (3, 48, 96), (2, 2048, 7168 // 4)])
def test_pack_weights_bit_exact(n, rows, cols):
    rng = np.random.default_rng(rows + cols)
    w = rng.integers(0, 1 << 16, size=(n, rows, cols), dtype=np.uint16)
    src = torch.from_numpy(w.view(np.int16)).cuda()
    dst = torch.empty_like(src)
    moe.moe_pack_weights(src, dst, n, rows, cols)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16).reshape(n, -1)
    for m in range(n):
        np.testing.assert_array_equal(got[m], frag16_reference(w[m]))


PACKABLE = [c for c in MID if c.dtype == "bf16" and c.d % 32 == 0 and c.H % 32 == 0 and c.Hs % 32 == 0]


@pytest.mark.parametrize("cfg", PACKABLE, ids=lambda c: c.name)
def test_layer_matches_oracle_packed_weights(cfg):
    L = G.make_layer(cfg, layout=moe.MOE_LAYOUT_FRAG16)
    r = G.run_layer(L)
    check_routing_on_gpu_logits(L, r)
    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward(x, wg, cfg.k, L.expert_fn(), L.shared_fn(), b, cfg.routing)
    np.testing.assert_array_equal(np.sort(r.idx.cpu().numpy(), 1), np.sort(ref["idx"], 1))
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out), ref["out"])
    assert ok, (err, bound)
    # same bits as the row-major path (same kernels' arithmetic, only the operand addressing differs)
    Lr = G.make_layer(cfg)
    rr = G.run_layer(Lr)
    assert torch.equal(r.out.view(torch.int16), rr.out.view(torch.int16))


@pytest.mark.parametrize("T", [12, 200, 3000])   # decode tail, one wave per token, grouped GEMM
@pytest.mark.parametrize("layout", ["rowmajor", "frag16"])
def test_every_token_on_the_same_experts(T, layout):
    """A logit bias that sends every token to experts 5 and 9 (k = 2): one or two buckets hold all the
    rows, the other 14 are empty (at T = 3000 the GEMM runs 10 M-tiles of one group while the tile
    schedule hands out nothing for the rest). Routing bit-exact, output within the layer tolerance."""
    cfg = LayerConfig(f"all_on_two_T{T}", T, 256, 16, 2, 192, 64, "bf16")
    L = G.make_layer(cfg, screen=False, layout={"rowmajor": moe.MOE_LAYOUT_ROWMAJOR,
                                                "frag16": moe.MOE_LAYOUT_FRAG16}[layout])
    bias = np.zeros(cfg.E, dtype=np.float32)
    bias[5], bias[9] = 100.0, 50.0
    L.host.logit_bias = bias
    L.bias = torch.from_numpy(bias).cuda()
    r = G.run_layer(L)
    counts = r.counts.cpu().numpy()
    assert counts[5] == T and counts[9] == T and counts.sum() == 2 * T
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward(x, wg, cfg.k, L.expert_fn(), L.shared_fn(), b, cfg.routing)
    np.testing.assert_array_equal(r.idx.cpu().numpy(), ref["idx"])
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out), ref["out"])
    assert ok, (err, bound)


@pytest.mark.parametrize("name", ["decode_ragged_shared", "gemm_ragged_shared"])
def test_timed_layer_matches_the_layer_and_times_every_stage(name):
    """moe_layer_forward_timed (the entry point the benchmark times stages with) gives the same bits
    as moe_layer_forward, and every event pair it records closes: a positive duration for each stage
    that launches a kernel (moe_stage_kernel_name non-empty), the events of a stage that launches
    nothing recorded back to back."""
    import ctypes
    import bench

    cfg = MID_BY_NAME[name]
    L = G.make_layer(cfg)
    ref = G.run_layer(L)
    n_st = moe.MOE_NUM_STAGES
    ev = bench.HipEvents(2 * n_st)
    try:
        out = torch.empty_like(ref.out)
        stream = torch.cuda.current_stream()
        moe.moe_layer_forward_timed(L.shape, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, L.ws_gate,
                                    L.ws_up, L.ws_down, out, workspace=moe.allocate_workspace(L.shape),
                                    stream=stream, events=ev.array(0, 2 * n_st))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.out.view(torch.int16))
        for st in range(n_st):
            ms = ev.elapsed_ms(2 * st, 2 * st + 1)
            launches = moe.moe_stage_kernel_name(L.shape, st) != ""
            assert (ms > 0) if launches else (0 <= ms < 0.05), (moe.STAGES[st], ms)
    finally:
        ev.close()

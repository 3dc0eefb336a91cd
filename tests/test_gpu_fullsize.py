"""HIP path vs the oracle at the full layer sizes the throughput is measured on (needs an MI355X).

DeepSeek-V3-shaped layer (d 7168, 256 routed experts of hidden 2048 + one shared, top-8) at
T = 8, 256 and 8192 (and with sigmoid routing at T = 8 and 4096), and the Mixtral-shaped skewed layer (d 4096, 8 experts of hidden 14336,
top-2, Zipf router bias) at T = 4096. The 22.5 GB DeepSeek weight set is drawn once in device
memory; the oracle regenerates on the host exactly the experts it needs. Routing and permutation
are checked bit-exactly on the GPU logits for every token; outputs are checked for every token at
T = 8 and for a seeded sample of tokens otherwise (a token's output depends on its row only); where
the grouped GEMM runs, the sample also holds the tokens at the edges of the largest expert buckets.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as G
from tests.test_gpu_parity import check_logits_close, check_routing_on_gpu_logits

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsv3_weights():
    cfg = synth.CONFIG_BY_NAME["dsv3_decode_t8"]
    w = G.make_weights(cfg, 0, host_copy=False)
    yield {moe.MOE_LAYOUT_ROWMAJOR: w, moe.MOE_LAYOUT_FRAG16: G.packed_weights(w),
           moe.MOE_LAYOUT_INT8_FRAG: G.int8_weights(w)}
    del w
    torch.cuda.empty_cache()


def sampled_check(L, r, tokens):
    x, wg, b = G.oracle_inputs(L)
    ref = oracle.layer_forward_tokens(x[tokens], wg, L.cfg.k, L.expert_fn(cache=False), L.shared_fn(), b,
                                      L.cfg.routing)
    np.testing.assert_array_equal(np.sort(r.idx.cpu().numpy()[tokens], 1), np.sort(ref["idx"], 1))
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out)[tokens], ref["out"])
    assert ok, (err, bound)


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=n - 2, replace=False)]))


def bucket_edge_tokens(idx, n_buckets=3, tile_rows=320):
    """Tokens whose rows sit at the ragged edges of the largest expert buckets of the grouped GEMM
    (its M-tiles hold 320 rows): each bucket's last row and, where the bucket is longer than one
    M-tile, the first and last rows of its second M-tile. A bucket lists its tokens in increasing
    order, so a token's row in it is the number of smaller tokens that chose the same expert."""
    idx = np.asarray(idx)
    counts = np.bincount(idx.ravel(), minlength=int(idx.max()) + 1)
    toks = []
    for e in np.argsort(-counts, kind="stable")[:n_buckets]:
        t_e = np.nonzero((idx == e).any(axis=1))[0]
        toks.append(t_e[-1])
        if len(t_e) > tile_rows:
            toks += [t_e[tile_rows], t_e[min(2 * tile_rows, len(t_e)) - 1]]
    return np.unique(np.asarray(toks, dtype=np.int64))


def gemm_sample(T, n, idx):
    """A seeded sample of tokens plus the bucket-edge tokens of the GPU's routing."""
    return np.union1d(sample_tokens(T, n), bucket_edge_tokens(idx.cpu().numpy()))


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_FRAG16, moe.MOE_LAYOUT_ROWMAJOR], ids=["frag16", "rowmajor"])
@pytest.mark.parametrize("name,n_sample", [("dsv3_decode_t8", None), ("dsv3_decode_t256", 12),
                                           ("dsv3_prefill_t8192", 8), ("dsv3_sigmoid_decode_t8", None)])
def test_dsv3_layer(name, n_sample, layout, dsv3_weights):
    cfg = synth.CONFIG_BY_NAME[name]
    L = G.make_layer(cfg, weights=dsv3_weights[layout], layout=layout)
    print(f"[{name}] gap-screen redraws: {sum(L.host.redraws.values())}", flush=True)
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    if n_sample is None:
        tokens = np.arange(cfg.T)
    elif cfg.T >= 2048:   # grouped GEMM experts: also the rows at the bucket edges
        tokens = gemm_sample(cfg.T, n_sample, r.idx)
    else:
        tokens = sample_tokens(cfg.T, n_sample)
    sampled_check(L, r, tokens)


@pytest.mark.parametrize("name,n_sample", [("dsv3_decode_t8", None), ("dsv3_decode_t256", 12)])
def test_dsv3_layer_int8_weights(name, n_sample, dsv3_weights):
    """Per-row INT8 expert weights at the decode sizes, against the oracle on the dequantized weights."""
    cfg = synth.CONFIG_BY_NAME[name]
    L = G.make_layer(cfg, weights=dsv3_weights[moe.MOE_LAYOUT_INT8_FRAG], layout=moe.MOE_LAYOUT_INT8_FRAG)
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    tokens = np.arange(cfg.T) if n_sample is None else sample_tokens(cfg.T, n_sample)
    sampled_check(L, r, tokens)


def test_dsv3_sigmoid_layer_router_gemm_size(dsv3_weights):
    """Sigmoid routing at 4096 tokens: the router GEMM (no bias in its epilogue), the one-wave-per-
    token top-k and the grouped GEMM experts, on the packed weights."""
    cfg = dataclasses.replace(synth.CONFIG_BY_NAME["dsv3_sigmoid_decode_t8"], name="dsv3_sigmoid_t4096", T=4096)
    L = G.make_layer(cfg, weights=dsv3_weights[moe.MOE_LAYOUT_FRAG16], layout=moe.MOE_LAYOUT_FRAG16)
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    sampled_check(L, r, gemm_sample(cfg.T, 8, r.idx))


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_FRAG16, moe.MOE_LAYOUT_ROWMAJOR], ids=["frag16", "rowmajor"])
def test_skewed_mixtral_layer(layout):
    cfg = synth.CONFIG_BY_NAME["skewed_mixtral_t4096"]
    L = G.make_layer(cfg, layout=layout)
    r = G.run_layer(L)
    counts = r.counts.cpu().numpy()
    print(f"[skewed] expert counts {counts.tolist()}", flush=True)
    assert counts[0] > 0.4 * cfg.T * cfg.k       # the Zipf head expert is the straggler
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    sampled_check(L, r, gemm_sample(cfg.T, 8, r.idx))

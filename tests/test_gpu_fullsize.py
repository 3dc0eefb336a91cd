"""HIP path vs the oracle at the full layer sizes the throughput is measured on (needs an MI355X).

DeepSeek-V3-shaped layer (d 7168, 256 routed experts of hidden 2048 + one shared, top-8) at
T = 8, 256 and 8192 (and with sigmoid routing at T = 8 and 4096), and the Mixtral-shaped skewed
layer (d 4096, 8 experts of hidden 14336, top-2, Zipf router bias) at T = 4096. The 22.5 GB
DeepSeek weight set is drawn once in device memory; the oracle regenerates on the host exactly the
experts it needs, once for all cases that share them.

Routing and permutation are checked bit-exactly on the GPU logits for every token. Outputs are
checked for every token at T = 8 and 256. Where the grouped GEMM runs (T >= 2048), the checked
tokens are chosen by the GEMM's structure: the first and the last row of every M-tile (320 rows) of
every expert bucket and of the shared expert's rows, plus a seeded random sample. Every tile of the
grouped GEMM (each (group, N-tile, M-tile), whichever XCD range holds it) then produces at least
two checked rows, at its ragged edges; the test asserts that coverage from the GPU's own counts.
A token's output depends on its own row only, so the oracle computes just those rows.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as G
from tests import helpers
from tests.helpers import M_TILE_ROWS, assert_tile_edges_covered, prefetching_expert_fn, structural_tokens
from tests.test_gpu_parity import check_logits_close, check_routing_on_gpu_logits

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu

GEMM_MIN_TOKENS = 2048  # DeepSeek-shaped layers above this many tokens run the grouped GEMM
LAYOUTS = {"frag16": moe.MOE_LAYOUT_FRAG16, "rowmajor": moe.MOE_LAYOUT_ROWMAJOR}


def tokens_for(cfg, idx):
    if cfg.T < GEMM_MIN_TOKENS:
        return np.arange(cfg.T)
    return structural_tokens(idx, cfg.T, cfg.Hs)


def run_cases(cases, weights_for):
    """Run every (config, layout) case on the GPU and keep what the checks need."""
    runs = {}
    for cfg, lname in cases:
        key = f"{cfg.name}-{lname}"
        print(f"[{key}] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} H={cfg.H} Hs={cfg.Hs} routing={cfg.routing} "
              f"moe_layer_forward", flush=True)
        L = G.make_layer(cfg, weights=weights_for(lname), layout=LAYOUTS[lname])
        r = G.run_layer(L)
        idx = r.idx.cpu().numpy()
        tokens = tokens_for(cfg, idx)
        rows = G.to_f64(r.out[torch.from_numpy(tokens).to(r.out.device)])
        runs[key] = dict(cfg=cfg, L=L, r=r, idx=idx, counts=r.counts.cpu().numpy(), tokens=tokens,
                         out=rows, redraws=sum(L.host.redraws.values()))
        r.out = None   # the checked rows are kept on the host
    return runs


def attach_oracle(runs, expert_fn, shared_fn):
    """One oracle pass over the experts for all runs: runs of the same workload share their inputs,
    so the union of their checked tokens is computed once."""
    by_name = {}
    for key, run in runs.items():
        by_name.setdefault(run["cfg"].name, []).append(key)
    names = sorted(by_name)
    toks = {n: np.unique(np.concatenate([runs[k]["tokens"] for k in by_name[n]])) for n in names}
    cases = []
    for n in names:
        L = runs[by_name[n][0]]["L"]
        x, wg, b = G.oracle_inputs(L)
        cases.append((x[toks[n]], wg, L.cfg.k, b, L.cfg.routing))
    # the weights are regenerated on the host, several experts ahead, with a line every 32 experts
    refs = oracle.layer_forward_tokens_many(cases, prefetching_expert_fn(expert_fn, cases), shared_fn)
    for n, ref in zip(names, refs):
        for key in by_name[n]:
            pos = np.searchsorted(toks[n], runs[key]["tokens"])
            runs[key]["ref_idx"] = ref["idx"][pos]
            runs[key]["ref_out"] = ref["out"][pos]


DSV3 = synth.CONFIG_BY_NAME["dsv3_decode_t8"]
DSV3_CASES = [(synth.CONFIG_BY_NAME[n], lay)
              for n in ("dsv3_decode_t8", "dsv3_decode_t256", "dsv3_prefill_t8192", "dsv3_sigmoid_decode_t8")
              for lay in ("frag16", "rowmajor")]
DSV3_CASES.append((dataclasses.replace(synth.CONFIG_BY_NAME["dsv3_sigmoid_decode_t8"], name="dsv3_sigmoid_t4096",
                                       T=4096), "frag16"))
DSV3_IDS = [f"{c.name}-{lay}" for c, lay in DSV3_CASES]


@pytest.fixture(scope="module")
def dsv3_weights():
    w = G.make_weights(DSV3, 0, host_copy=False)
    yield {"rowmajor": w, "frag16": G.packed_weights(w), "int8": G.int8_weights(w), "fp8": G.int8_weights(w, fp8=True)}
    del w
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def dsv3_runs(dsv3_weights):
    runs = run_cases(DSV3_CASES, lambda lname: dsv3_weights[lname])
    print("[dsv3] oracle pass over the selected experts of every case", flush=True)
    L0 = next(iter(runs.values()))["L"]
    attach_oracle(runs, L0.expert_fn(cache=False), L0.shared_fn())
    yield runs
    runs.clear()
    torch.cuda.empty_cache()


def check_run(run):
    cfg, L, r = run["cfg"], run["L"], run["r"]
    print(f"[{cfg.name}] gap-screen redraws: {run['redraws']}", flush=True)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    if cfg.T >= GEMM_MIN_TOKENS:
        assert_tile_edges_covered(run["idx"], run["counts"], run["tokens"], cfg.T, cfg.Hs)
    np.testing.assert_array_equal(np.sort(run["idx"][run["tokens"]], 1), np.sort(run["ref_idx"], 1))
    ok, err, bound = G.tolerance_ok(run["out"], run["ref_out"])
    assert ok, (err, bound)


@pytest.mark.timeout(1200)   # the first test also runs the shared fixture: every case + one oracle pass
@pytest.mark.parametrize("case", DSV3_IDS)
def test_dsv3_layer(case, dsv3_runs):
    check_run(dsv3_runs[case])


ONE_BYTE_CASES = [(n, k, q) for n, k in (("dsv3_decode_t8", None), ("dsv3_decode_t256", 12)) for q in ("int8", "fp8")]
# the prefill size for INT8 only: the two code formats share every line of the grouped GEMM but the
# code -> bf16 step (checked for all 256 codes of both), and the oracle's host-side E4M3 encoding
# of all 256 experts would double the module's time
ONE_BYTE_CASES.append(("dsv3_prefill_t8192", "structural", "int8"))


@pytest.mark.parametrize("name,n_sample,quant", ONE_BYTE_CASES, ids=lambda v: str(v))
def test_dsv3_layer_one_byte_weights(name, n_sample, quant, dsv3_weights):
    """Per-row INT8 or FP8 expert weights at the decode sizes (weight streaming) and at the prefill
    size (grouped GEMM, every M-tile's first and last row checked), against the oracle on the
    dequantized weights."""
    cfg = synth.CONFIG_BY_NAME[name]
    print(f"[{name}-{quant}] moe_layer_forward", flush=True)
    layout = {"int8": moe.MOE_LAYOUT_INT8_FRAG, "fp8": moe.MOE_LAYOUT_FP8_FRAG}[quant]
    L = G.make_layer(cfg, weights=dsv3_weights[quant], layout=layout)
    r = G.run_layer(L)
    check_logits_close(L, r)
    check_routing_on_gpu_logits(L, r)
    if n_sample is None:
        tokens = np.arange(cfg.T)
    elif n_sample == "structural":
        idx = r.idx.cpu().numpy()
        tokens = structural_tokens(idx, cfg.T, cfg.Hs)
        assert_tile_edges_covered(idx, r.counts.cpu().numpy(), tokens, cfg.T, cfg.Hs)
        assert moe.moe_stage_kernel_name(L.shape, moe.STAGES.index("ffn_gate_up")).startswith("grouped_gemm_kernel<0")
    else:
        rng = np.random.default_rng(0)
        tokens = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, size=n_sample - 2, replace=False)]))
    x, wg, b = G.oracle_inputs(L)
    efn = prefetching_expert_fn(L.expert_fn(cache=False), [(x[tokens], wg, cfg.k, b, cfg.routing)])
    ref = oracle.layer_forward_tokens(x[tokens], wg, cfg.k, efn, L.shared_fn(), b, cfg.routing)
    np.testing.assert_array_equal(np.sort(r.idx.cpu().numpy()[tokens], 1), np.sort(ref["idx"], 1))
    ok, err, bound = G.tolerance_ok(G.to_f64(r.out)[tokens], ref["out"])
    assert ok, (err, bound)


EP_EXPERTS = 32   # one GPU's experts when the 256 are split over 8 GPUs in expert parallel


def ep_share_counts(seed=0):
    """Bucket sizes around the 2,048 rows per expert that one GPU of eight receives when each GPU
    routes 8,192 tokens, with the ragged cases of the 320-row M-tiling: an empty expert, a single
    row, an exact multiple of the tile and one row past it."""
    rng = np.random.default_rng(seed)
    c = rng.integers(1800, 2300, size=EP_EXPERTS)
    c[3], c[7], c[11], c[19] = 0, 1, 6 * M_TILE_ROWS, 6 * M_TILE_ROWS + 1
    return c


@pytest.mark.timeout(900)
def test_dsv3_ep8_share_grouped_ffn(dsv3_weights):
    """moe_grouped_ffn at one expert-parallel GPU's share of the DeepSeek-V3-shaped layer (the
    shape bench.py --ep-share 8 times): the first 32 experts over ~2,048 contiguous received rows
    each (perm_src NULL, k = 1), both bf16 weight layouts. Checked rows: the first and last row of
    every 320-row M-tile of every bucket plus a seeded sample, against the oracle's SwiGLU of each
    expert on those rows."""
    from concurrent.futures import ThreadPoolExecutor

    cfg = DSV3
    counts = ep_share_counts()
    R = int(counts.sum())
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = torch.empty(R, cfg.d, dtype=torch.bfloat16, device="cuda")
    synth.normal_device(x, 7, synth.stream_id(synth.K_X), 1.0)
    rows = set()
    for e in range(EP_EXPERTS):
        for m0 in range(int(offs[e]), int(offs[e + 1]), M_TILE_ROWS):
            rows.update((m0, min(m0 + M_TILE_ROWS, int(offs[e + 1])) - 1))
    rows.update(np.random.default_rng(1).choice(R, size=16, replace=False).tolist())
    rows = np.array(sorted(rows), dtype=np.int64)
    owner = np.searchsorted(offs, rows, side="right") - 1
    outs = {}
    for lname in ("frag16", "rowmajor"):
        print(f"[ep8-share-{lname}] moe_grouped_ffn E={EP_EXPERTS} rows={R} d={cfg.d} H={cfg.H}", flush=True)
        (g, u, dn), _, _ = dsv3_weights[lname]
        s = moe.make_shape(R, cfg.d, EP_EXPERTS, 1, cfg.H, 0, "bf16", LAYOUTS[lname])
        y = torch.empty_like(x)
        moe.moe_grouped_ffn(s, x, None, torch.from_numpy(offs.astype(np.int32)).cuda(), g[:EP_EXPERTS],
                            u[:EP_EXPERTS], dn[:EP_EXPERTS], y, moe.allocate_workspace(s))
        torch.cuda.synchronize()
        outs[lname] = G.to_f64(y[torch.from_numpy(rows).cuda()])
        del y
    x_rows = G.to_f64(x[torch.from_numpy(rows).cuda()])
    del x
    print(f"[ep8-share] oracle SwiGLU of {len(rows)} rows over {int((counts > 0).sum())} experts", flush=True)
    efn = helpers.expert_fn_host(cfg, 0, cache=False)

    def expert_rows(e):
        sel = owner == e
        return sel, oracle.swiglu(x_rows[sel], *efn(e))

    ref = np.zeros_like(x_rows)
    with ThreadPoolExecutor(8) as pool:
        for sel, r in pool.map(expert_rows, sorted(set(owner.tolist()))):
            ref[sel] = r
    for lname, out in outs.items():
        ok, err, bound = G.tolerance_ok(out, ref)
        assert ok, (lname, err, bound)


FP8_GEMM_COUNTS = [256, 0, 1, 320, 321, 300, 250, 200, 640, 33, 32, 31, 257, 100, 500, 288]


@pytest.mark.timeout(900)
def test_dsv3_fp8_grouped_gemm_at_full_width():
    """The one-byte grouped GEMM with E4M3 codes at the DeepSeek-V3 widths (d = 7168, H = 2048):
    moe_grouped_ffn over the first 16 experts (quantized on their own) and buckets of 0 to 640
    contiguous rows (mean 221, so the grouped GEMM runs; an empty and a one-row bucket, buckets of
    exactly one M-tile and one row more, two M-tiles). The layer test at T = 8192 runs the INT8
    form of the same GEMM; this one checks the E4M3 decode inside it at that size. Checked rows:
    the first and last row of every 320-row M-tile plus a seeded sample, against the oracle's SwiGLU
    on the dequantized E4M3 weights."""
    from concurrent.futures import ThreadPoolExecutor

    cfg = DSV3
    E = len(FP8_GEMM_COUNTS)
    counts = np.array(FP8_GEMM_COUNTS)
    R = int(counts.sum())
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    (g, u, dn), _, _ = G.make_weights(dataclasses.replace(cfg, E=E), 0, host_copy=False)
    q = moe.quantize_expert_weights(g, u, dn, fp8=True)
    torch.cuda.synchronize()
    del g, u, dn
    x = torch.empty(R, cfg.d, dtype=torch.bfloat16, device="cuda")
    synth.normal_device(x, 11, synth.stream_id(synth.K_X), 1.0)
    s = moe.make_shape(R, cfg.d, E, 1, cfg.H, 0, "bf16", moe.MOE_LAYOUT_FP8_FRAG)
    assert moe.moe_stage_kernel_name(s, moe.STAGES.index("ffn_gate_up")) == "grouped_gemm_kernel<0, 3>"
    print(f"[fp8-gemm] moe_grouped_ffn E={E} rows={R} d={cfg.d} H={cfg.H}", flush=True)
    y = torch.empty_like(x)
    moe.moe_grouped_ffn(s, x, None, torch.from_numpy(offs.astype(np.int32)).cuda(), q[0], q[1], q[2], y,
                        moe.allocate_workspace(s))
    torch.cuda.synchronize()
    rows = set()
    for e in range(E):
        for m0 in range(int(offs[e]), int(offs[e + 1]), M_TILE_ROWS):
            rows.update((m0, min(m0 + M_TILE_ROWS, int(offs[e + 1])) - 1))
    rows.update(np.random.default_rng(2).choice(R, size=16, replace=False).tolist())
    rows = np.array(sorted(rows), dtype=np.int64)
    owner = np.searchsorted(offs, rows, side="right") - 1
    out = G.to_f64(y[torch.from_numpy(rows).cuda()])
    x_rows = G.to_f64(x[torch.from_numpy(rows).cuda()])
    del x, y, q
    print(f"[fp8-gemm] oracle SwiGLU of {len(rows)} rows over {len(set(owner.tolist()))} experts (E4M3 weights)",
          flush=True)
    efn = helpers.expert_fn_host(dataclasses.replace(cfg, E=E), 0, cache=False, quant="fp8")

    def expert_rows(e):
        sel = owner == e
        return sel, oracle.swiglu(x_rows[sel], *efn(e))

    ref = np.zeros_like(x_rows)
    with ThreadPoolExecutor(8) as pool:
        for sel, r in pool.map(expert_rows, sorted(set(owner.tolist()))):
            ref[sel] = r
    ok, err, bound = G.tolerance_ok(out, ref)
    assert ok, (err, bound)


SKEWED = synth.CONFIG_BY_NAME["skewed_mixtral_t4096"]


@pytest.fixture(scope="module")
def skewed_runs():
    w = G.make_weights(SKEWED, 0, host_copy=False)
    weights = {"rowmajor": w, "frag16": G.packed_weights(w)}
    runs = run_cases([(SKEWED, lay) for lay in ("frag16", "rowmajor")], lambda lname: weights[lname])
    print("[skewed] oracle pass over the 8 experts", flush=True)
    L0 = next(iter(runs.values()))["L"]
    attach_oracle(runs, L0.expert_fn(cache=False), L0.shared_fn())
    yield runs, weights
    runs.clear()
    del weights, w
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layout", ["frag16", "rowmajor"])
def test_skewed_mixtral_layer(layout, skewed_runs):
    runs, _ = skewed_runs
    run = runs[f"{SKEWED.name}-{layout}"]
    counts = run["counts"]
    print(f"[skewed] expert counts {counts.tolist()}", flush=True)
    assert counts[0] > 0.4 * SKEWED.T * SKEWED.k       # the Zipf head expert is the straggler
    check_run(run)

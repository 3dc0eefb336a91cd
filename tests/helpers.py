"""Test helpers: gap screening of seeded inputs and oracle wiring (tests only)."""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

MIN_GAP = 1e-4   # tokens whose k-th and (k+1)-th router scores are closer than this are redrawn
M_TILE_ROWS = 320  # rows of one M-tile of the grouped GEMM


def screen_gaps(inp: synth.HostInputs, min_gap: float = MIN_GAP, max_rounds: int = 64) -> int:
    """Redraw activation rows whose top-k margin is below ``min_gap``: the margin between the k-th
    and (k+1)-th fp64 selection scores (the logits with any logit bias for softmax routing; the
    sigmoid affinities plus the selection bias for sigmoid routing).

    Rejection happens per token: a near-tie row is replaced by the next draw of its own redraw
    stream until every token clears the margin. Returns the number of rows redrawn.
    """
    cfg = inp.cfg
    wg = oracle.widen(inp.w_router, cfg.dtype)
    redrawn = 0
    for _ in range(max_rounds):
        L = oracle.router_logits(oracle.widen(inp.x, cfg.dtype), wg, inp.logit_bias)
        S = oracle.selection_scores(L, cfg.routing, inp.score_bias)
        bad = np.nonzero(oracle.topk_gap(S, cfg.k) < min_gap)[0]
        if bad.size == 0:
            return redrawn
        synth.redraw_rows(inp, bad)
        redrawn += int(bad.size)
    raise RuntimeError("gap screening did not converge")


def as_oracle_weight(a, dtype: str, quant=None):
    """float64 weight the oracle uses: the stored value, or the dequantized per-row one-byte code
    (quant "int8" or "fp8")."""
    w = oracle.widen(a, dtype)
    if quant == "int8":
        return oracle.dequantize_rows_int8(*oracle.quantize_rows_int8(w))
    if quant == "fp8":
        return oracle.dequantize_rows_fp8(*oracle.quantize_rows_fp8(w))
    assert quant is None, quant
    return w


def expert_fn_host(cfg: synth.LayerConfig, seed: int, stacked=None, cache: bool = True, quant=None):
    """float64 expert weights for the oracle, regenerated on the host from the generator streams
    (dequantized from their per-row one-byte codes when ``quant`` is "int8" or "fp8").

    ``cache=False`` regenerates on every call (large layers: one expert in memory at a time)."""
    store = {}

    def make(e):
        if stacked is not None:
            g, u, dn = (s[e] for s in stacked)
        else:
            g, u, dn = synth.expert_weights_host(cfg, seed, e)
        return tuple(as_oracle_weight(a, cfg.dtype, quant) for a in (g, u, dn))

    def fn(e):
        if not cache:
            return make(e)
        if e not in store:
            store[e] = make(e)
        return store[e]

    return fn


def shared_fn_host(cfg: synth.LayerConfig, seed: int, quant=None):
    if cfg.Hs == 0:
        return None
    box = {}

    def fn():
        if "w" not in box:
            box["w"] = tuple(as_oracle_weight(a, cfg.dtype, quant)
                             for a in synth.expert_weights_host(cfg, seed, 0, shared=True))
        return box["w"]

    return fn


def structural_tokens(idx, T, Hs, n_random=8, seed=0):
    """The first and last token of every M-tile of every expert bucket (a bucket lists the tokens
    that chose the expert in increasing order) and of the shared expert's rows (token order), plus
    ``n_random`` seeded tokens."""
    idx = np.asarray(idx)
    toks = set()
    for e in np.unique(idx):
        t_e = np.nonzero((idx == e).any(axis=1))[0]
        for m0 in range(0, len(t_e), M_TILE_ROWS):
            toks.update((int(t_e[m0]), int(t_e[min(m0 + M_TILE_ROWS, len(t_e)) - 1])))
    if Hs:
        for m0 in range(0, T, M_TILE_ROWS):
            toks.update((m0, min(m0 + M_TILE_ROWS, T) - 1))
    rng = np.random.default_rng(seed)
    toks.update(int(t) for t in rng.choice(T, size=min(n_random, T), replace=False))
    return np.array(sorted(toks), dtype=np.int64)


def assert_tile_edges_covered(idx, counts, tokens, T, Hs):
    """Every expert with rows (by the GPU's counts) has the first and last row of each of its
    M-tiles among the checked tokens, and so has every M-tile of the shared expert's rows."""
    idx, counts = np.asarray(idx), np.asarray(counts)
    chosen = set(np.asarray(tokens).tolist())
    missing = []
    for e in np.nonzero(counts)[0]:
        t_e = np.nonzero((idx == e).any(axis=1))[0]
        assert len(t_e) == counts[e], (e, len(t_e), counts[e])
        for m0 in range(0, int(counts[e]), M_TILE_ROWS):
            for r in (m0, min(m0 + M_TILE_ROWS, int(counts[e])) - 1):
                if int(t_e[r]) not in chosen:
                    missing.append((int(e), r))
    if Hs:
        for m0 in range(0, T, M_TILE_ROWS):
            for r in (m0, min(m0 + M_TILE_ROWS, T) - 1):
                if r not in chosen:
                    missing.append(("shared", r))
    assert not missing, missing[:10]
    n_tiles = sum((int(c) + M_TILE_ROWS - 1) // M_TILE_ROWS for c in counts) + (
        (T + M_TILE_ROWS - 1) // M_TILE_ROWS if Hs else 0)
    print(f"  checked tokens {len(chosen)} cover both edges of all {n_tiles} M-tiles "
          f"({int((counts > 0).sum())} experts{' + shared' if Hs else ''})", flush=True)


def prefetching_expert_fn(expert_fn, cases, workers: int = 8, label: str = "oracle"):
    """``expert_fn`` for an oracle pass over ``cases`` ((x_rows, w_router, k, bias, routing) each):
    the experts the pass will ask for (every expert the oracle's routing selects, in ascending
    order, as ``oracle.layer_forward_tokens`` and ``layer_forward_tokens_many`` visit them) are
    prepared ``workers`` ahead on a thread pool (numpy releases the GIL), so regenerating and
    dequantizing them on the host overlaps. Results are the same as ``expert_fn``'s; at most
    ``workers`` + 1 experts are held at once. Prints a progress line every 32 experts."""
    sel = set()
    for x_rows, w_router, k, bias, routing in cases:
        _, idx, _ = oracle.route(np.asarray(x_rows, np.float64), w_router, k, bias, routing)
        sel.update(np.unique(idx).tolist())
    order = iter(sorted(int(e) for e in sel))
    pool = ThreadPoolExecutor(workers)
    futs = {}
    seen = []

    def submit_next():
        e = next(order, None)
        if e is not None:
            futs[e] = pool.submit(expert_fn, e)

    for _ in range(workers):
        submit_next()

    def fn(e):
        e = int(e)
        seen.append(e)
        if len(seen) % 32 == 0:
            print(f"  {label}: {len(seen)} experts", flush=True)
        f = futs.pop(e, None)
        if f is None:
            return expert_fn(e)
        submit_next()
        return f.result()

    return fn

"""Test helpers: gap screening of seeded inputs and oracle wiring (tests only)."""

from __future__ import annotations

import numpy as np

import oracle
import synth

MIN_GAP = 1e-4   # tokens whose k-th and (k+1)-th router scores are closer than this are redrawn


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


def as_oracle_weight(a, dtype: str, int8: bool):
    """float64 weight the oracle uses: the stored value, or the dequantized INT8 per-row code."""
    w = oracle.widen(a, dtype)
    return oracle.dequantize_rows_int8(*oracle.quantize_rows_int8(w)) if int8 else w


def expert_fn_host(cfg: synth.LayerConfig, seed: int, stacked=None, cache: bool = True, int8: bool = False):
    """float64 expert weights for the oracle, regenerated on the host from the generator streams
    (dequantized from their per-row INT8 codes when ``int8``).

    ``cache=False`` regenerates on every call (large layers: one expert in memory at a time)."""
    store = {}

    def make(e):
        if stacked is not None:
            g, u, dn = (s[e] for s in stacked)
        else:
            g, u, dn = synth.expert_weights_host(cfg, seed, e)
        return tuple(as_oracle_weight(a, cfg.dtype, int8) for a in (g, u, dn))

    def fn(e):
        if not cache:
            return make(e)
        if e not in store:
            store[e] = make(e)
        return store[e]

    return fn


def shared_fn_host(cfg: synth.LayerConfig, seed: int, int8: bool = False):
    if cfg.Hs == 0:
        return None
    box = {}

    def fn():
        if "w" not in box:
            box["w"] = tuple(as_oracle_weight(a, cfg.dtype, int8)
                             for a in synth.expert_weights_host(cfg, seed, 0, shared=True))
        return box["w"]

    return fn

"""The structural token sample of the full-size parity tests (host logic, no GPU)."""

import numpy as np
import pytest

import oracle
from tests.helpers import M_TILE_ROWS, assert_tile_edges_covered, structural_tokens


def zipf_routing(T, E, k, seed):
    """Top-k ids of random logits with a Zipf-like per-expert bias (buckets of very different sizes)."""
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)) + 2.0 * np.log((np.arange(E) + 1.0) ** -1.2)[None, :]
    return oracle.select_topk(L, k)


@pytest.mark.parametrize("T,E,k,Hs", [(4096, 8, 2, 0), (2500, 64, 8, 16), (1400, 4, 1, 8)])
def test_structural_sample_covers_every_tile_edge(T, E, k, Hs):
    idx = zipf_routing(T, E, k, T)
    counts = np.bincount(idx.ravel(), minlength=E)
    assert counts.max() > 2 * M_TILE_ROWS          # buckets of several M-tiles
    tokens = structural_tokens(idx, T, Hs)
    assert_tile_edges_covered(idx, counts, tokens, T, Hs)
    # the sample stays small: two tokens per M-tile at most, plus the random ones
    n_tiles = sum(-(-int(c) // M_TILE_ROWS) for c in counts) + (-(-T // M_TILE_ROWS) if Hs else 0)
    assert len(tokens) <= 2 * n_tiles + 8


def test_coverage_check_names_a_missing_edge():
    idx = zipf_routing(3000, 8, 2, 1)
    counts = np.bincount(idx.ravel(), minlength=8)
    tokens = structural_tokens(idx, 3000, 0, n_random=0)
    e = int(np.argmax(counts))
    t_e = np.nonzero((idx == e).any(axis=1))[0]
    last_of_first_tile = int(t_e[M_TILE_ROWS - 1])
    with pytest.raises(AssertionError):
        assert_tile_edges_covered(idx, counts, tokens[tokens != last_of_first_tile], 3000, 0)
    with pytest.raises(AssertionError):   # counts that disagree with the ids
        assert_tile_edges_covered(idx, counts + np.eye(8, dtype=counts.dtype)[e], tokens, 3000, 0)
    with pytest.raises(AssertionError):   # a shared-expert M-tile edge left out
        assert_tile_edges_covered(idx, counts, tokens, 3000, 16)


def test_prefetching_expert_fn_returns_what_expert_fn_returns():
    """The prefetching wrapper hands the oracle the same arrays, for every expert its routing
    selects, in any order it asks for them (and for an expert it did not predict)."""
    import numpy as np

    import oracle
    from tests.helpers import prefetching_expert_fn

    rng = np.random.default_rng(3)
    T, d, E, k, H = 12, 16, 10, 3, 8
    x, wg = rng.standard_normal((T, d)), rng.standard_normal((E, d))
    weights = {e: tuple(rng.standard_normal(s) for s in ((H, d), (H, d), (d, H))) for e in range(E)}
    calls = []

    def expert_fn(e):
        calls.append(e)
        return weights[e]

    cases = [(x, wg, k, None, "softmax"), (x[:4], wg, 2, None, "sigmoid")]
    fn = prefetching_expert_fn(expert_fn, cases, workers=2)
    ref = oracle.layer_forward_tokens_many(cases, expert_fn)
    got = oracle.layer_forward_tokens_many(cases, fn)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a["out"], b["out"])
    assert fn(E - 1) is weights[E - 1]   # asked for again (or never selected): computed on the spot

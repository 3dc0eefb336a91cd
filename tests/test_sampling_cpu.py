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

"""Pins of the CPU oracle against facts fixed by the pages and by mathematics (no GPU).

Each test checks the oracle against something other than itself: hand-worked instances solved in
closed form, brute force over all k-subsets, independent library routines (torch.topk, scipy's
softmax, torch's SiLU), invariants the pages state, and the pages' own assignment counts.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def rand_layer(rng, T, d, E, H, scale=1.0):
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) * scale / math.sqrt(d)
    ex = [(rng.standard_normal((H, d)) / math.sqrt(d), rng.standard_normal((H, d)) / math.sqrt(d),
           rng.standard_normal((d, H)) / math.sqrt(H)) for _ in range(E)]
    return x, wg, ex


def screened(rng, T, d, E, k, H, min_gap=1e-3):
    """Random layer whose tokens all have a clear top-k margin (redraw rows otherwise)."""
    x, wg, ex = rand_layer(rng, T, d, E, H)
    for _ in range(200):
        bad = np.nonzero(oracle.topk_gap(oracle.router_logits(x, wg), k) < min_gap)[0]
        if bad.size == 0:
            return x, wg, ex
        x[bad] = rng.standard_normal((bad.size, d))
    raise RuntimeError


# ------------------------------------------------------------------ hand-worked instances

def w1_layer(with_shared):
    """E=4, k=2, T=2, d=2, H=1. Router rows e0=[1,2.5], e1=[3,-1], e2=[2,2], e3=[0,1];
    expert e: W_gate=[[1,1]], W_up=[[e+1,e+1]], W_down=[[1],[-1]]; x0=[1,0], x1=[0,1]."""
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    wg = np.array([[1.0, 2.5], [3.0, -1.0], [2.0, 2.0], [0.0, 1.0]])
    ex = {e: (np.array([[1.0, 1.0]]), np.array([[e + 1.0, e + 1.0]]), np.array([[1.0], [-1.0]])) for e in range(4)}
    sh = (np.array([[1.0, 1.0]]), np.array([[1.0, 1.0]]), np.array([[1.0], [1.0]]))
    return oracle.layer_forward(x, wg, 2, lambda e: ex[e], (lambda: sh) if with_shared else None)


def test_w1_routing_by_hand():
    r = w1_layer(False)
    # logits t0 = [1, 3, 2, 0], t1 = [2.5, -1, 2, 1]
    np.testing.assert_array_equal(r["logits"], [[1, 3, 2, 0], [2.5, -1, 2, 1]])
    np.testing.assert_array_equal(r["idx"], [[1, 2], [0, 2]])
    # softmax of two scores a > b is (sigmoid(a-b), sigmoid(b-a))
    np.testing.assert_allclose(r["w"], [[sig(1), sig(-1)], [sig(0.5), sig(-0.5)]], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r["counts"], [1, 1, 2, 0])           # expert 3 gets nothing
    np.testing.assert_array_equal(r["offsets"], [0, 1, 2, 4, 4])
    np.testing.assert_array_equal(r["perm_src"], [2, 0, 1, 3])
    np.testing.assert_array_equal(r["inv_perm"], [1, 2, 0, 3])


def test_w1_outputs_by_hand():
    # every expert sees gate=1, up=e+1 for both tokens: y_e = (e+1) * SiLU(1) * [1, -1], SiLU(1) = sigmoid(1)
    s1 = sig(1.0)
    out0 = (2 * sig(1) + 3 * sig(-1)) * s1
    out1 = (1 * sig(0.5) + 3 * sig(-0.5)) * s1
    r = w1_layer(False)
    np.testing.assert_allclose(r["out"], [[out0, -out0], [out1, -out1]], rtol=1e-14)
    assert abs(out0 - 1.658729090501) < 1e-11 and abs(out1 - 1.283067268043) < 1e-11
    # shared expert gate=[1,1], up=[1,1], down=[[1],[1]] adds sigmoid(1) to both features
    r = w1_layer(True)
    np.testing.assert_allclose(r["out"], [[out0 + s1, -out0 + s1], [out1 + s1, -out1 + s1]], rtol=1e-14)


def test_w2_ties_go_to_lower_index():
    L = np.array([[2.0, 2.0, 1.0, 0.0]])
    idx = oracle.select_topk(L, 1)
    assert idx.tolist() == [[0]]
    assert oracle.softmax_selected(L, idx).tolist() == [[1.0]]
    idx = oracle.select_topk(L, 2)
    assert idx.tolist() == [[0, 1]]
    np.testing.assert_allclose(oracle.softmax_selected(L, idx), [[0.5, 0.5]])
    # tie at the boundary: experts 0 and 2 both score 1, the lower index wins the last slot
    assert oracle.select_topk(np.array([[1.0, 3.0, 1.0, 0.0]]), 2).tolist() == [[1, 0]]
    # signed zeros compare equal
    assert oracle.select_topk(np.array([[-0.0, 0.0, -1.0]]), 1).tolist() == [[0]]


def test_w3_k_equals_E_identical_experts_is_dense_ffn():
    rng = np.random.default_rng(3)
    T, d, E, H = 6, 10, 4, 7
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d))
    g, u, dn = rng.standard_normal((H, d)), rng.standard_normal((H, d)), rng.standard_normal((d, H))
    r = oracle.layer_forward(x, wg, E, lambda e: (g, u, dn))
    # dense FFN via torch's own SiLU in float64 (an independent routine)
    xt = torch.from_numpy(x)
    dense = (torch.nn.functional.silu(xt @ torch.from_numpy(g).T) * (xt @ torch.from_numpy(u).T)) @ torch.from_numpy(dn).T
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["w"].sum(1), 1.0, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ selection and weights

@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 2), (8, 5), (8, 8)])
def test_topk_is_best_subset_by_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    L = rng.standard_normal((64, E))
    idx = oracle.select_topk(L, k)
    for t in range(L.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(L[t, list(s)]))
        assert set(idx[t].tolist()) == set(best)
        # in-list order: strictly decreasing scores (no ties in continuous draws)
        assert np.all(np.diff(L[t, idx[t]]) < 0)


def test_topk_matches_torch_topk_and_is_monotone_invariant():
    rng = np.random.default_rng(11)
    L = rng.standard_normal((500, 256))
    idx = oracle.select_topk(L, 8)
    tv, ti = torch.topk(torch.from_numpy(L), 8, dim=1)
    np.testing.assert_array_equal(idx, ti.numpy())
    # the selected set does not change under a monotone map of the scores
    np.testing.assert_array_equal(idx, oracle.select_topk(scipy.special.expit(L), 8))
    np.testing.assert_array_equal(idx, oracle.select_topk(scipy.special.softmax(L, axis=1), 8))


def test_topk_gap_by_hand():
    """The screening margin is the k-th largest score minus the (k+1)-th largest, per token.
    Row [3, 2, 1.5, 0]: k=1 -> 3-2 = 1, k=2 -> 2-1.5 = 0.5, k=3 -> 1.5-0 = 1.5. Row [3, 1, 2, 2]
    (unsorted, with a tie inside): k=1 -> 1, k=2 -> 0 (a tie at the cut), k=3 -> 2-1 = 1. With
    k = E nothing is left unselected, so no tie can change the selection: the margin is infinite."""
    L = np.array([[3.0, 2.0, 1.5, 0.0], [3.0, 1.0, 2.0, 2.0]])
    np.testing.assert_array_equal(oracle.topk_gap(L, 1), [1.0, 1.0])
    np.testing.assert_array_equal(oracle.topk_gap(L, 2), [0.5, 0.0])
    np.testing.assert_array_equal(oracle.topk_gap(L, 3), [1.5, 1.0])
    assert np.all(np.isinf(oracle.topk_gap(L, 4))) and np.all(oracle.topk_gap(L, 4) > 0)
    # negative scores and a single token
    np.testing.assert_array_equal(oracle.topk_gap(np.array([[-4.0, -1.0, -2.5]]), 1), [1.5])


def test_topk_gap_is_the_smallest_selected_minus_largest_unselected():
    """Brute force: for the selected set K (the k largest), the margin equals
    min_{i in K} s_i - max_{j not in K} s_j, and a permutation of the experts leaves it unchanged."""
    rng = np.random.default_rng(21)
    S = rng.standard_normal((50, 9))
    for k in range(1, 9):
        gap = oracle.topk_gap(S, k)
        for t in range(S.shape[0]):
            sel = set(oracle.select_topk(S[t:t + 1], k)[0].tolist())
            lo = min(S[t, i] for i in sel)
            hi = max(S[t, j] for j in range(9) if j not in sel)
            assert gap[t] == lo - hi
        perm = rng.permutation(9)
        np.testing.assert_array_equal(oracle.topk_gap(S[:, perm], k), gap)
    assert (oracle.topk_gap(S, 3) > 0).all()


def test_topk_gap_on_sigmoid_selection_scores():
    """Sigmoid routing screens on the scores that decide its selection, sigmoid(l) + b. Logits all
    zero and bias [0.3, 0.1, 0.2, 0]: scores [0.8, 0.6, 0.7, 0.5], so k = 2 leaves a margin of
    0.7 - 0.6 = 0.1; without the bias every score is 0.5 and the margin is 0."""
    L = np.zeros((1, 4))
    b = np.array([0.3, 0.1, 0.2, 0.0])
    gap = oracle.topk_gap(oracle.selection_scores(L, "sigmoid", b), 2)
    np.testing.assert_allclose(gap, [0.1], rtol=0, atol=1e-15)
    assert oracle.topk_gap(oracle.selection_scores(L, "sigmoid", None), 2)[0] == 0.0


def test_softmax_over_k_is_renormalised_full_softmax():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((40, 16)) * 3
    for k in (1, 2, 5, 16):
        idx = oracle.select_topk(L, k)
        w = oracle.softmax_selected(L, idx)
        full = scipy.special.softmax(L, axis=1)
        sel = np.take_along_axis(full, idx, 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13)
        np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-15)      # weights sum to 1
        if k == 1:
            assert np.all(w == 1.0)


def test_softmax_large_scores_do_not_overflow():
    L = np.array([[1000.0, 999.0, -5.0]])
    w = oracle.softmax_selected(L, oracle.select_topk(L, 2))
    np.testing.assert_allclose(w, [[sig(1), sig(-1)]], rtol=1e-14)


def test_bias_shifts_selection_and_weights():
    # bias added to logits before both selection and softmax
    L0 = np.zeros((1, 3))
    b = np.array([0.0, 1.0, 2.0])
    x = np.ones((1, 1))
    L, idx, w = oracle.route(x, np.zeros((3, 1)), 2, b)
    assert idx.tolist() == [[2, 1]]
    np.testing.assert_allclose(w, [[sig(1), sig(-1)]])
    np.testing.assert_array_equal(L, L0 + b)


# ------------------------------------------------------------------ permutation

@pytest.mark.parametrize("T,E,k", [(0, 4, 2), (1, 4, 4), (17, 8, 2), (64, 256, 8), (300, 16, 3)])
def test_permutation_invariants_and_stable_argsort_construction(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int64)
    counts, offsets, perm_src, inv_perm = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    # counts by brute force, offsets are the exclusive running sum, total T*k
    assert [int((flat == e).sum()) for e in range(E)] == counts.tolist()
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
    assert np.all(counts >= 0) and np.all(counts <= T)
    # a bijection, inverse of each other
    assert sorted(perm_src.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(inv_perm[perm_src], np.arange(T * k))
    # the listing's construction (flatten ids, argsort, bincount, cumsum), read with a stable sort
    np.testing.assert_array_equal(perm_src, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(np.bincount(flat, minlength=E), counts)
    np.testing.assert_array_equal(np.cumsum(counts), offsets[1:])
    # keys (expert, token) non-decreasing along the rows
    keys = [(flat[p], p // k) for p in perm_src]
    assert keys == sorted(keys)
    for e in range(E):
        assert np.all(flat[perm_src[offsets[e]:offsets[e + 1]]] == e)


def test_assignment_counts_from_the_pages():
    spec = json.load(open(os.path.join(GOLDEN, "assignment_counts.json")))
    rng = np.random.default_rng(0)
    for c in spec["cases"]:
        T, k, E = c["tokens"], c["k"], c["E"]
        L = rng.standard_normal((T, E))
        idx = oracle.select_topk(L, k)
        counts, offsets, perm_src, _ = oracle.permute(idx, E)
        assert offsets[-1] == c["assignments"] == len(perm_src)
        assert counts.sum() / E == pytest.approx(c["mean_per_expert"])


def test_layer_shape_example_from_the_pages():
    spec = json.load(open(os.path.join(GOLDEN, "layer_shape_example.json")))
    B, S, d = spec["input_shape"]
    rng = np.random.default_rng(1)
    x, wg, ex = rand_layer(rng, B * S, d, spec["experts"], spec["expert_width"])
    r = oracle.layer_forward(x, wg, spec["k"], lambda e: ex[e])
    assert list(r["out"].reshape(B, S, d).shape) == spec["output_shape"]


# ------------------------------------------------------------------ experts and combine

def test_single_expert_is_plain_swiglu_with_torch_silu():
    rng = np.random.default_rng(2)
    x, wg, ex = rand_layer(rng, 9, 12, 1, 20)
    r = oracle.layer_forward(x, wg, 1, lambda e: ex[e])
    g, u, dn = (torch.from_numpy(a) for a in ex[0])
    xt = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(xt @ g.T) * (xt @ u.T)) @ dn.T
    np.testing.assert_allclose(r["out"], ref.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(r["w"] == 1.0)


def test_silu_known_values():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([1.0, -1.0, 20.0])), [sig(1), -sig(-1), 20 * sig(20)], rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.linspace(-8, 8, 33)),
                               torch.nn.functional.silu(torch.linspace(-8, 8, 33, dtype=torch.float64)).numpy(),
                               rtol=1e-14)


@pytest.mark.parametrize("T,E,k", [(12, 8, 2), (20, 6, 3), (5, 4, 4)])
def test_sparse_equals_dense_masked(T, E, k):
    """Run every expert on every token and weight non-selected ones by zero: same output."""
    rng = np.random.default_rng(T * E * k)
    x, wg, ex = screened(rng, T, 16, E, k, 24)
    sh = (rng.standard_normal((24, 16)), rng.standard_normal((24, 16)), rng.standard_normal((16, 24)))
    r = oracle.layer_forward(x, wg, k, lambda e: ex[e], lambda: sh)
    L = x @ wg.T
    dense_w = np.zeros((T, E))
    for t in range(T):
        top = np.argsort(-L[t])[:k]
        z = np.exp(L[t, top] - L[t, top].max())
        dense_w[t, top] = z / z.sum()
    xt = torch.from_numpy(x)

    def ffn(g, u, dn):
        return ((torch.nn.functional.silu(xt @ torch.from_numpy(g).T) * (xt @ torch.from_numpy(u).T))
                @ torch.from_numpy(dn).T).numpy()

    dense = ffn(*sh) + sum(dense_w[:, e:e + 1] * ffn(*ex[e]) for e in range(E))
    np.testing.assert_allclose(r["out"], dense, rtol=1e-11, atol=1e-11)


def test_output_linear_in_down_projection_and_shared_only():
    rng = np.random.default_rng(9)
    x, wg, ex = screened(rng, 10, 8, 4, 2, 6)
    sh = (rng.standard_normal((5, 8)), rng.standard_normal((5, 8)), rng.standard_normal((8, 5)))
    base = oracle.layer_forward(x, wg, 2, lambda e: ex[e])["out"]
    scaled = oracle.layer_forward(x, wg, 2, lambda e: (ex[e][0], ex[e][1], 2.5 * ex[e][2]))["out"]
    np.testing.assert_allclose(scaled, 2.5 * base, rtol=1e-12, atol=1e-14)
    zero = oracle.layer_forward(x, wg, 2, lambda e: (ex[e][0], ex[e][1], 0 * ex[e][2]), lambda: sh)
    np.testing.assert_allclose(zero["out"], oracle.swiglu(x, *sh), rtol=1e-14, atol=0)
    # the shared expert adds exactly its own FFN output
    with_sh = oracle.layer_forward(x, wg, 2, lambda e: ex[e], lambda: sh)["out"]
    np.testing.assert_allclose(with_sh - base, oracle.swiglu(x, *sh), rtol=1e-10, atol=1e-12)


def test_token_sampled_forward_matches_full_forward():
    rng = np.random.default_rng(4)
    x, wg, ex = screened(rng, 15, 12, 8, 3, 10)
    sh = (rng.standard_normal((7, 12)), rng.standard_normal((7, 12)), rng.standard_normal((12, 7)))
    full = oracle.layer_forward(x, wg, 3, lambda e: ex[e], lambda: sh)
    rows = [0, 4, 14]
    part = oracle.layer_forward_tokens(x[rows], wg, 3, lambda e: ex[e], lambda: sh)
    np.testing.assert_allclose(part["out"], full["out"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(part["idx"], full["idx"][rows])


def test_token_sets_sharing_experts_match_separate_full_forwards():
    """Several token samples with their own routers, k, biases and routing rules, run with one visit
    per expert, give for each sample what its own full layer gives on those rows."""
    rng = np.random.default_rng(8)
    E, d, H = 8, 12, 10
    x1, wg1, ex = screened(rng, 14, d, E, 3, H)
    x2, wg2, _ = screened(rng, 9, d, E, 2, H)
    x3 = rng.standard_normal((6, d))
    wg3 = rng.standard_normal((E, d)) / math.sqrt(d)
    b3 = rng.standard_normal(E) * 0.05
    sh = (rng.standard_normal((7, d)), rng.standard_normal((7, d)), rng.standard_normal((d, 7)))
    visits = []

    def efn(e):
        visits.append(e)
        return ex[e]

    cases = [(x1[[0, 5, 13]], wg1, 3, None, "softmax"), (x2, wg2, 2, None, "softmax"),
             (x3, wg3, 4, b3, "sigmoid"), (x1[:0], wg1, 3, None, "softmax")]
    many = oracle.layer_forward_tokens_many(cases, efn, lambda: sh)
    assert len(visits) == len(set(visits))      # each expert generated once
    full = [oracle.layer_forward(x1, wg1, 3, lambda e: ex[e], lambda: sh)["out"][[0, 5, 13]],
            oracle.layer_forward(x2, wg2, 2, lambda e: ex[e], lambda: sh)["out"],
            oracle.layer_forward(x3, wg3, 4, lambda e: ex[e], lambda: sh, b3, "sigmoid")["out"],
            np.zeros((0, d))]
    for r, f in zip(many, full):
        np.testing.assert_allclose(r["out"], f, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(many[2]["idx"], oracle.route(x3, wg3, 4, b3, "sigmoid")[1])


def test_empty_batch():
    r = oracle.layer_forward(np.zeros((0, 4)), np.ones((3, 4)), 2, lambda e: None)
    assert r["out"].shape == (0, 4) and r["offsets"].tolist() == [0, 0, 0, 0]


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.widen(bits, "bf16"), ref)


# ------------------------------------------------------------------ sigmoid routing (MoE kernels §2.2)

def one_token_route(logits, k, bias=None, routing="sigmoid"):
    """route() on a single token whose logits are given directly (x = [1], W_g = the logits column)."""
    wg = np.asarray(logits, np.float64)[:, None]
    return oracle.route(np.ones((1, 1)), wg, k, None if bias is None else np.asarray(bias, np.float64), routing)


def test_logistic_matches_scipy_expit_without_overflow():
    z = np.concatenate([np.linspace(-800, 800, 4001), [-1e300, 1e300, 0.0]])
    np.testing.assert_allclose(oracle.logistic(z), scipy.special.expit(z), rtol=1e-15, atol=1e-300)
    assert oracle.logistic(np.array([0.0]))[0] == 0.5


def test_sigmoid_routing_without_bias_selects_like_softmax():
    """sigmoid is strictly increasing, so with no bias it ranks experts exactly as the logits do."""
    rng = np.random.default_rng(7)
    x, wg, _ = rand_layer(rng, 60, 12, 16, 4)
    _, idx_soft, _ = oracle.route(x, wg, 5)
    _, idx_sig, w_sig = oracle.route(x, wg, 5, None, "sigmoid")
    np.testing.assert_array_equal(idx_sig, idx_soft)
    np.testing.assert_allclose(w_sig.sum(1), 1.0, rtol=0, atol=1e-15)
    assert (w_sig > 0).all()


def test_sigmoid_bias_decides_selection_by_hand():
    """Logits [2, 1, 0, -1], bias +0.6 on expert 2, k = 2. Affinities sigmoid(l) are about
    [0.881, 0.731, 0.5, 0.269]; with the bias expert 2 scores 1.1 and ranks first, expert 0 second.
    (Adding the bias to the logit instead, sigmoid(0.6) = 0.646 < 0.731, would keep [0, 1]; a
    selection that ignores the bias also gives [0, 1].)"""
    _, idx, w = one_token_route([2.0, 1.0, 0.0, -1.0], 2, [0.0, 0.0, 0.6, 0.0])
    assert idx.tolist() == [[2, 0]]
    _, idx0, _ = one_token_route([2.0, 1.0, 0.0, -1.0], 2)
    assert idx0.tolist() == [[0, 1]]
    # weights: the unbiased affinities sigmoid(0) = 1/2 and sigmoid(2), normalised: 1/2 is the
    # smaller share and the two shares sum to one
    assert w[0, 0] < 0.5 < w[0, 1] and abs(w.sum() - 1.0) < 1e-15


def test_sigmoid_bias_leaves_weights_alone():
    """The bias changes which experts are picked, never their weights ([MoE kernels] §2.2): a bias
    shifted by a constant, or changed only on experts that stay unselected, gives the same ids and
    bit-identical weights."""
    rng = np.random.default_rng(11)
    x, wg, _ = rand_layer(rng, 40, 10, 12, 4)
    b = rng.standard_normal(12) * 0.3
    _, idx, w = oracle.route(x, wg, 3, b, "sigmoid")
    _, idx2, w2 = oracle.route(x, wg, 3, b + 5.0, "sigmoid")
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_allclose(w2, w, rtol=1e-15, atol=0)
    # lower the bias of experts no token selected: nothing changes
    unused = np.setdiff1d(np.arange(12), np.unique(idx))
    if unused.size:
        b3 = b.copy()
        b3[unused] -= 10.0
        _, idx3, w3 = oracle.route(x, wg, 3, b3, "sigmoid")
        np.testing.assert_array_equal(idx3, idx)
        np.testing.assert_array_equal(w3, w)


def test_sigmoid_weights_limits():
    """Large positive logits saturate every affinity at 1, so the weights tend to 1/k (a softmax
    would favour the largest logit); for very negative logits sigmoid(l) ~ e^l, so the weights tend
    to the softmax over the selected logits."""
    _, idx, w = one_token_route([30.0, 31.0, 32.0, -5.0], 3)
    assert idx.tolist() == [[2, 1, 0]]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=0, atol=1e-12)
    lg = np.array([-40.0, -37.5, -36.0, -39.0, -45.0])
    _, idx, w = one_token_route(lg, 3)
    assert idx.tolist() == [[2, 1, 3]]
    np.testing.assert_allclose(w[0], scipy.special.softmax(lg[[2, 1, 3]]), rtol=1e-14, atol=0)


@pytest.mark.parametrize("E,k", [(5, 2), (8, 3), (7, 7)])
def test_sigmoid_selection_is_best_subset_by_brute_force(E, k):
    """The selected set maximises the sum of the biased scores over all k-subsets."""
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(20):
        lg = rng.standard_normal(E) * 2
        b = rng.standard_normal(E) * 0.2
        _, idx, _ = one_token_route(lg, k, b)
        S = 1.0 / (1.0 + np.exp(-lg)) + b
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(S[list(c)]))
        assert sorted(idx[0].tolist()) == sorted(best)
        assert all(S[idx[0][i]] >= S[idx[0][i + 1]] for i in range(k - 1))


def test_sigmoid_layer_forward_uses_sigmoid_weights():
    """A whole layer with sigmoid routing: the output is the weighted sum of the selected experts
    with the sigmoid weights (the same dense-masked check as the softmax layer)."""
    rng = np.random.default_rng(3)
    T, d, E, k, H = 12, 6, 5, 2, 4
    x, wg, ex = rand_layer(rng, T, d, E, H)
    b = rng.standard_normal(E) * 0.2
    r = oracle.layer_forward(x, wg, k, lambda e: ex[e], None, b, "sigmoid")
    dense = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = r["idx"][t, j]
            dense[t] += r["w"][t, j] * oracle.swiglu(x[t:t + 1], *ex[e])[0]
    np.testing.assert_allclose(r["out"], dense, rtol=1e-12, atol=1e-12)
    tok = oracle.layer_forward_tokens(x[3:7], wg, k, lambda e: ex[e], None, b, "sigmoid")
    np.testing.assert_allclose(tok["out"], r["out"][3:7], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ INT8 weights (Inference ch.6)

def test_quantization_example_from_the_pages():
    with open(os.path.join(GOLDEN, "quantization_example.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert oracle.quantize(c["x"], c["s"], c["z"]) == c["x_q"]
        assert abs(oracle.dequantize(c["x_q"], c["s"], c["z"]) - c["x_hat"]) < 1e-12


def test_int8_rows_round_trip_within_half_a_step():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((3, 40, 96)) * rng.uniform(0.01, 10.0, (3, 40, 1))
    w[1, 7] = 0.0                                      # an all-zero row
    q, sc = oracle.quantize_rows_int8(w)
    w32 = w.astype(np.float32).astype(np.float64)
    err = np.abs(oracle.dequantize_rows_int8(q, sc) - w32)
    assert (err <= sc.astype(np.float64)[..., None] * (0.5 + 1e-6)).all()
    nz = sc > 0
    assert (np.abs(q).max(-1)[nz] == 127).all()        # the largest entry of every row maps to +-127
    assert sc[1, 7] == 0 and (q[1, 7] == 0).all()
    assert (np.sign(q) == np.sign(np.rint(w32 / np.where(nz, sc, 1)[..., None]))).all()


def test_int8_rows_match_torch_per_channel_quantization():
    """torch.quantize_per_channel (axis = output channel, zero point 0) gives the same codes, except
    where w / s sits within float rounding of a half-integer (torch divides in double)."""
    rng = np.random.default_rng(6)
    w = rng.standard_normal((64, 128)).astype(np.float32)
    q, sc = oracle.quantize_rows_int8(w)
    tq = torch.quantize_per_channel(torch.from_numpy(w), torch.from_numpy(sc.astype(np.float64)),
                                    torch.zeros(64, dtype=torch.int64), 0, torch.qint8).int_repr().numpy()
    ratio = w.astype(np.float64) / sc.astype(np.float64)[:, None]
    near_half = np.abs(np.abs(ratio - np.floor(ratio)) - 0.5) < 1e-4
    assert (q[~near_half] == tq[~near_half]).all()
    assert near_half.mean() < 1e-3


# ------------------------------------------------------------------ load statistics (MoE overview §4.1)

# ------------------------------------------------------------------ FP8 (E4M3) weights

def test_fp8_e4m3_codes_by_hand():
    """Codes from the format's definition (sign, 4 exponent bits with bias 7, 3 mantissa bits):
    1 = 2^0 -> e 7 -> 0x38; 0.5 -> 0x30; 1.125 = 1 + 1/8 -> 0x39; 3.5 = 1.75 * 2 -> 0x46; 240 = 1.875 * 2^7
    -> 0x77; 448 = 1.75 * 2^8 -> 0x7E (largest finite); 2^-6 -> 0x08 (smallest normal); 2^-9 -> 0x01
    (smallest subnormal); 7 * 2^-9 -> 0x07; the sign is the top bit (-0.0 -> 0x80)."""
    x = [1.0, -1.0, 0.5, 1.125, 3.5, 240.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, 0.0, -0.0]
    want = [0x38, 0xB8, 0x30, 0x39, 0x46, 0x77, 0x7E, 0xFE, 0x08, 0x01, 0x07, 0x00, 0x80]
    assert oracle.fp8_e4m3_encode(np.array(x, np.float32)).tolist() == want
    np.testing.assert_array_equal(oracle.fp8_e4m3_decode(np.array(want, np.uint8)), x)
    assert np.isnan(oracle.fp8_e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_fp8_e4m3_rounding_ties_and_saturation():
    """Nearest value, ties to the even code: 1.0625 lies midway between 1 (0x38) and 1.125 (0x39) and
    goes to 0x38; 1.1875 between 0x39 and 0x3A goes to 0x3A; 1.05 is nearer 1 than 1.125; on the
    subnormal grid 1.5 * 2^-9 goes
    to 0x02 and 7.5 * 2^-9 to 0x08 (= 2^-6). Past 448 the nearest finite value is 448 up to the midpoint
    464 with the absent 480; at and above it the code saturates to 448 as well."""
    x = np.array([1.0625, 1.1875, 1.05, 1.5 * 2.0 ** -9, 7.5 * 2.0 ** -9, 460.0, 464.0, 1e30, -500.0], np.float32)
    assert oracle.fp8_e4m3_encode(x).tolist() == [0x38, 0x3A, 0x38, 0x02, 0x08, 0x7E, 0x7E, 0x7E, 0xFE]


def test_fp8_e4m3_is_the_nearest_code_by_brute_force():
    """Every finite code decodes and re-encodes to itself, and for random float32 inputs within range
    the code is the finite code of least distance (ties to the even code), found by trying all 253."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = oracle.fp8_e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(vals.astype(np.float32)), codes)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 9, 4000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = oracle.fp8_e4m3_encode(x)
    pos = codes[codes < 0x80]
    pv = oracle.fp8_e4m3_decode(pos)
    for xi, gi in zip(x.astype(np.float64), got):
        d = np.abs(pv - abs(xi))
        best = pos[d == d.min()]
        best = best[best % 2 == 0] if len(best) > 1 else best      # a tie goes to the even code
        assert (gi & 0x7F) == best[0] and (gi >> 7) == (xi < 0 or (xi == 0 and np.signbit(xi)))


def test_fp8_e4m3_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-14, 9, 20000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.fp8_e4m3_encode(x), t)


def test_fp8_rows_map_each_row_maximum_to_448_and_stay_within_half_a_step():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((3, 40, 96)) * rng.uniform(1e-3, 5, (3, 40, 1))
    w[1, 7] = 0.0
    codes, s = oracle.quantize_rows_fp8(w)
    assert s.dtype == np.float32 and codes.dtype == np.uint8 and s[1, 7] == 0 and (codes[1, 7] == 0).all()
    nz = s > 0
    amax = np.abs(oracle.fp8_e4m3_decode(codes)).max(-1)
    assert (amax[nz] == 448.0).all()
    w32 = w.astype(np.float32).astype(np.float64)
    back = oracle.dequantize_rows_fp8(codes, s)
    x = w32 / np.where(s > 0, s, 1)[..., None]
    # half a step of the E4M3 grid at |x|: 2^(floor(log2|x|) - 4) for normals, 2^-10 for subnormals
    half = np.where(np.abs(x) < 2.0 ** -6, 2.0 ** -10, np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6))) - 4))
    assert (np.abs(back - w32) <= half * s[..., None] * (1 + 1e-6) + 1e-30).all()


def test_load_stats_closed_forms():
    """Uniform assignment has no penalty; everything on one expert gives coef * (E-1)/E; the loads
    are the assignment shares and sum to 1."""
    E, T, k = 8, 16, 2
    load, aux = oracle.load_stats(np.full(E, T * k // E), T, k)
    np.testing.assert_allclose(load, 1.0 / E, rtol=0, atol=1e-15)
    assert aux == 0.0
    one = np.zeros(E, np.int64)
    one[3] = T * k
    load, aux = oracle.load_stats(one, T, k, coef=0.5)
    assert load[3] == 1.0 and load.sum() == 1.0
    assert abs(aux - 0.5 * (E - 1) / E) < 1e-15


def test_load_stats_from_a_routing():
    """On a real routing the loads are the assignment shares (brute-force count over the ids)."""
    rng = np.random.default_rng(9)
    x, wg, _ = rand_layer(rng, 50, 8, 6, 4)
    _, idx, _ = oracle.route(x, wg, 2)
    counts, _, _, _ = oracle.permute(idx, 6)
    load, aux = oracle.load_stats(counts, 50, 2, coef=0.01)
    for e in range(6):
        assert load[e] == sum(1 for t in range(50) for j in range(2) if idx[t, j] == e) / 100
    assert abs(load.sum() - 1.0) < 1e-15
    assert abs(aux - 0.01 * sum((load[e] - 1 / 6) ** 2 for e in range(6))) < 1e-15


# ------------------------------------------------------------------ GELU expert variant

def test_gelu_known_values():
    """GELU(z) = z Phi(z): Phi(0) = 1/2, Phi(1) and Phi(2) from the standard normal table; GELU(z) -
    GELU(-z) = z (as Phi(z) + Phi(-z) = 1); against scipy's normal CDF and torch's exact GELU."""
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.gelu(np.array([1.0, -1.0, 2.0])),
                               [0.8413447460685429, -0.15865525393145707, 2 * 0.9772498680518208], rtol=1e-15)
    z = np.linspace(-7, 7, 57)
    np.testing.assert_allclose(oracle.gelu(z) - oracle.gelu(-z), z, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu(z), z * scipy.special.ndtr(z), rtol=1e-14, atol=1e-300)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(z), ref, rtol=1e-14, atol=1e-15)   # torch's 1 + erf cancels for z << 0


def test_gelu_mlp_by_hand():
    """Two rows through a 3 -> 2 -> 3 expert with both biases, in plain Python."""
    X = [[0.5, -1.0, 2.0], [1.5, 0.25, -0.75]]
    w1 = [[0.2, -0.4, 0.1], [-0.3, 0.5, 0.6]]
    b1 = [0.05, -0.1]
    w2 = [[1.0, -2.0], [0.5, 0.25], [-1.5, 0.75]]
    b2 = [0.3, -0.2, 0.1]
    got = oracle.gelu_mlp(np.array(X), np.array(w1), np.array(b1), np.array(w2), np.array(b2))
    for r in range(2):
        h = []
        for o in range(2):
            z = sum(X[r][i] * w1[o][i] for i in range(3)) + b1[o]
            h.append(z * 0.5 * (1 + math.erf(z / math.sqrt(2))))
        for o in range(3):
            assert abs(got[r, o] - (sum(h[i] * w2[o][i] for i in range(2)) + b2[o])) < 1e-14


def _gelu_experts(E, d, H, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal((H, d)) / math.sqrt(d), rng.standard_normal(H) * 0.1,
             rng.standard_normal((d, H)) / math.sqrt(H), rng.standard_normal(d) * 0.1) for _ in range(E)]


def test_gelu_single_expert_layer_is_torch_linear_gelu_linear():
    """E = k = 1: the layer is the listing's expert block itself (weight 1), built from torch modules."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 6))
    (w1, b1, w2, b2), = _gelu_experts(1, 6, 10, 6)
    r = oracle.layer_forward_gelu(x, rng.standard_normal((1, 6)), 1, lambda e: (w1, b1, w2, b2))
    blk = torch.nn.Sequential(torch.nn.Linear(6, 10), torch.nn.GELU(), torch.nn.Linear(10, 6)).double()
    with torch.no_grad():
        blk[0].weight.copy_(torch.from_numpy(w1)); blk[0].bias.copy_(torch.from_numpy(b1))
        blk[2].weight.copy_(torch.from_numpy(w2)); blk[2].bias.copy_(torch.from_numpy(b2))
        ref = blk(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_gelu_layer_is_the_weighted_sum_over_the_selected_experts():
    """Every token: sum over its k selected experts of weight x expert(x_t), experts from torch modules."""
    rng = np.random.default_rng(7)
    T, d, E, k, H = 13, 8, 5, 2, 12
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d))
    b = rng.standard_normal(E) * 0.3
    ex = _gelu_experts(E, d, H, 8)
    r = oracle.layer_forward_gelu(x, wg, k, lambda e: ex[e], b)
    mods = []
    for (w1, b1, w2, b2) in ex:
        m = torch.nn.Sequential(torch.nn.Linear(d, H), torch.nn.GELU(), torch.nn.Linear(H, d)).double()
        with torch.no_grad():
            m[0].weight.copy_(torch.from_numpy(w1)); m[0].bias.copy_(torch.from_numpy(b1))
            m[2].weight.copy_(torch.from_numpy(w2)); m[2].bias.copy_(torch.from_numpy(b2))
        mods.append(m)
    L = x @ wg.T + b
    for t in range(T):
        top = sorted(range(E), key=lambda e: (-L[t, e], e))[:k]
        w = np.exp(L[t, top] - L[t, top].max())
        w /= w.sum()
        with torch.no_grad():
            ref = sum(w[j] * mods[e](torch.from_numpy(x[t:t + 1])).numpy()[0] for j, e in enumerate(top))
        np.testing.assert_allclose(r["out"][t], ref, rtol=1e-12, atol=1e-13)


def _gelu_tanh(z):
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


def _gelu_mlp_without_b2(X, w1, b1, w2, b2):
    return _GELU_MLP(X, w1, b1, w2, None)


def _gelu_mlp_bias_after_activation(X, w1, b1, w2, b2):
    X = np.asarray(X, np.float64)
    H = om.gelu(X @ np.asarray(w1).T) + (0 if b1 is None else np.asarray(b1)[None, :])
    return H @ np.asarray(w2).T + (0 if b2 is None else np.asarray(b2)[None, :])


# ------------------------------------------------------------------ planted mistakes are caught

def _plant(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _swiglu_swapped(X, g, u, dn):
    X = np.asarray(X, np.float64)
    return (om.silu(X @ np.asarray(u).T) * (X @ np.asarray(g).T)) @ np.asarray(dn).T


def _combine_no_shared(y, inv, w, shared=None):
    return _COMBINE(y, inv, w, None)


def _combine_with_perm(y, inv, w, shared=None):
    inv = np.asarray(inv)
    perm = np.empty_like(inv)
    perm[inv] = np.arange(len(inv))
    return _COMBINE(y, perm, w, shared)


def _softmax_unnormalised_over_k(L, idx):
    return np.take_along_axis(scipy.special.softmax(np.asarray(L), axis=1), idx, 1)


def _perm_reversed(idx, E):
    c, o, p, _ = _PERMUTE(idx, E)
    p = p.copy()
    for e in range(E):
        p[o[e]:o[e + 1]] = p[o[e]:o[e + 1]][::-1].copy()
    inv = np.empty_like(p)
    inv[p] = np.arange(len(p))
    return c, o, p, inv


def _route_bias_weights_only(x, w_router, k, bias=None, routing="softmax"):
    L0 = om.router_logits(x, w_router, None)
    idx = om.select_topk(L0, k)
    L = om.router_logits(x, w_router, bias)
    return L, idx, om.softmax_selected(L, idx)


def _sigmoid_scores_of_biased_logit(L, routing="softmax", bias=None):
    if routing != "sigmoid":
        return _SELECTION(L, routing, bias)
    L = np.asarray(L, np.float64)
    return om.logistic(L + (0.0 if bias is None else np.asarray(bias)[None, :]))


def _sigmoid_scores_without_bias(L, routing="softmax", bias=None):
    return _SELECTION(L, routing, None)


def _sigmoid_weights_with_bias(x, w_router, k, bias=None, routing="softmax"):
    if routing != "sigmoid":
        return _ROUTE(x, w_router, k, bias, routing)
    L = om.router_logits(x, w_router, None)
    S = om.selection_scores(L, "sigmoid", bias)
    idx = om.select_topk(S, k)
    s = np.take_along_axis(S, idx, 1)
    return L, idx, s / s.sum(1, keepdims=True)


def _logistic_sign_flipped(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(np.asarray(z, np.float64)))


def _sigmoid_weights_softmax(L, idx):
    return om.softmax_selected(L, idx)


def _quant_rows_div128(w):
    w32 = np.asarray(w, np.float64).astype(np.float32)
    sc = (np.abs(w32).max(-1) / np.float32(128.0)).astype(np.float32)
    q = np.clip(np.rint(w32 / np.where(sc > 0, sc, 1)[..., None]), -127, 127)
    return q.astype(np.int8), sc


def _quant_rows_truncating(w):
    w32 = np.asarray(w, np.float64).astype(np.float32)
    sc = (np.abs(w32).max(-1) / np.float32(127.0)).astype(np.float32)
    q = np.trunc(w32 / np.where(sc > 0, sc, 1)[..., None])
    return q.astype(np.int8), sc


def _quant_cols(w):
    w32 = np.asarray(w, np.float64).astype(np.float32)
    sc = (np.abs(w32).max(-2) / np.float32(127.0)).astype(np.float32)
    q = np.rint(w32 / np.where(sc > 0, sc, 1)[..., None, :])
    return q.astype(np.int8), (np.abs(w32).max(-1) / np.float32(127.0)).astype(np.float32)


def _gap_one_past(L, k):
    """Margin measured one place too far down: (k+1)-th minus (k+2)-th score."""
    s = -np.sort(-np.asarray(L, np.float64), axis=1)
    out = np.full(s.shape[0], np.inf)
    if k + 1 < s.shape[1]:
        out = s[:, k] - s[:, k + 1]
    return out


def _gap_one_short(L, k):
    """Margin measured one place too high: (k-1)-th minus k-th score (the first gap for k = 1)."""
    s = -np.sort(-np.asarray(L, np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, max(k - 2, 0)] - s[:, max(k - 1, 1)]


def _gap_always_inf(L, k):
    return np.full(np.asarray(L).shape[0], np.inf)


def _e4m3_truncating(x):
    x = np.asarray(x, np.float32).astype(np.float64)
    a = np.abs(x)
    frac, ex = np.frexp(np.where(a > 0, a, 1.0))
    code = np.where(a < 2.0 ** -6, np.floor(a * 512.0), ((ex + 6) * 8 + np.floor((2 * frac - 1) * 8)))
    code = np.where(a >= 448, 0x7E, code).astype(np.int64) | (np.signbit(x).astype(np.int64) << 7)
    return code.astype(np.uint8)


def _e4m3_decode_bias8(code):
    c = np.asarray(code, np.uint8).astype(np.int64)
    e, m = (c >> 3) & 15, (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -10, (1 + m / 8) * np.exp2(e - 8.0))
    return np.where(c & 0x80, -mag, mag)


def _e4m3_decode_no_subnormals(code):
    c = np.asarray(code, np.uint8).astype(np.int64)
    e, m = (c >> 3) & 15, (c & 7).astype(np.float64)
    mag = (1 + m / 8) * np.exp2(e - 7.0)
    return np.where(c & 0x80, -mag, mag)


def _fp8_rows_scale_127(w):
    w32 = np.asarray(w, np.float64).astype(np.float32)
    sc = (np.abs(w32).max(-1) / np.float32(127.0)).astype(np.float32)
    return om.fp8_e4m3_encode((w32 / np.where(sc > 0, sc, 1)[..., None]).astype(np.float32)), sc


def _load_over_tokens(counts, T, k, coef=0.01):
    load = np.asarray(counts, np.float64) / T
    return load, coef * float(((load - 1.0 / len(load)) ** 2).sum())


_COMBINE = om.combine
_GELU_MLP = om.gelu_mlp
_PERMUTE = om.permute
_SELECTION = om.selection_scores
_ROUTE = om.route

MUTATIONS = {
    "silu_as_sigmoid": ("silu", lambda z: 1.0 / (1.0 + np.exp(-np.asarray(z))),
                        test_single_expert_is_plain_swiglu_with_torch_silu),
    "gate_and_up_swapped": ("swiglu", _swiglu_swapped, test_single_expert_is_plain_swiglu_with_torch_silu),
    "softmax_over_all_E": ("softmax_selected", _softmax_unnormalised_over_k,
                           test_softmax_over_k_is_renormalised_full_softmax),
    "topk_ascending": ("select_topk", lambda L, k: np.argsort(np.asarray(L), axis=1, kind="stable")[:, :k],
                       lambda: test_topk_is_best_subset_by_brute_force(8, 2)),
    "perm_reversed_within_expert": ("permute", _perm_reversed, test_w1_routing_by_hand),
    "shared_expert_dropped": ("combine", _combine_no_shared, test_w1_outputs_by_hand),
    "combine_gathers_with_perm_src": ("combine", _combine_with_perm, test_w1_outputs_by_hand),
    "bias_only_in_weights": ("route", _route_bias_weights_only, test_bias_shifts_selection_and_weights),
    "sigmoid_of_biased_logit": ("selection_scores", _sigmoid_scores_of_biased_logit,
                                test_sigmoid_bias_decides_selection_by_hand),
    "sigmoid_selection_ignores_bias": ("selection_scores", _sigmoid_scores_without_bias,
                                       test_sigmoid_bias_decides_selection_by_hand),
    "sigmoid_bias_in_weights": ("route", _sigmoid_weights_with_bias, test_sigmoid_bias_leaves_weights_alone),
    "sigmoid_weights_as_softmax": ("sigmoid_weights_selected", _sigmoid_weights_softmax,
                                   test_sigmoid_weights_limits),
    "logistic_sign_flipped": ("logistic", _logistic_sign_flipped, test_logistic_matches_scipy_expit_without_overflow),
    "int8_scale_over_128": ("quantize_rows_int8", _quant_rows_div128, test_int8_rows_round_trip_within_half_a_step),
    "int8_truncating": ("quantize_rows_int8", _quant_rows_truncating, test_int8_rows_round_trip_within_half_a_step),
    "int8_scale_per_column": ("quantize_rows_int8", _quant_cols, test_int8_rows_match_torch_per_channel_quantization),
    "dequantize_without_zero_point": ("dequantize", lambda q, s, z=0: np.asarray(q, np.float64) * s,
                                      test_quantization_example_from_the_pages),
    "load_over_tokens_not_slots": ("load_stats", _load_over_tokens, test_load_stats_closed_forms),
    "fp8_truncating": ("fp8_e4m3_encode", _e4m3_truncating, test_fp8_e4m3_rounding_ties_and_saturation),
    "fp8_exponent_bias_8": ("fp8_e4m3_decode", _e4m3_decode_bias8, test_fp8_e4m3_codes_by_hand),
    "fp8_subnormals_as_normals": ("fp8_e4m3_decode", _e4m3_decode_no_subnormals, test_fp8_e4m3_codes_by_hand),
    "fp8_scale_over_127": ("quantize_rows_fp8", _fp8_rows_scale_127,
                           test_fp8_rows_map_each_row_maximum_to_448_and_stay_within_half_a_step),
    "topk_gap_one_place_too_far": ("topk_gap", _gap_one_past, test_topk_gap_by_hand),
    "topk_gap_one_place_too_high": ("topk_gap", _gap_one_short, test_topk_gap_by_hand),
    "topk_gap_never_rejects": ("topk_gap", _gap_always_inf, test_topk_gap_is_the_smallest_selected_minus_largest_unselected),
    "gelu_tanh_approximation": ("gelu", _gelu_tanh, test_gelu_known_values),
    "gelu_as_silu": ("gelu", lambda z: om.silu(z), test_gelu_known_values),
    "gelu_expert_drops_output_bias": ("gelu_mlp", _gelu_mlp_without_b2,
                                      test_gelu_single_expert_layer_is_torch_linear_gelu_linear),
    "gelu_expert_bias_after_activation": ("gelu_mlp", _gelu_mlp_bias_after_activation, test_gelu_mlp_by_hand),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistakes_fail_a_pin(mutation, monkeypatch):
    """A plausible slip planted in the oracle makes the named pin fail."""
    name, fn, pin = MUTATIONS[mutation]
    _plant(monkeypatch, name, fn)
    with pytest.raises(AssertionError):
        pin()

"""Pins of the oracle's post-processing and selection steps.

Pooling is pinned to SciPy's filters (a library special case), pages, clusters,
top-k and the block union to hand-built cases with answers worked out by hand
(tests/golden/selection_cases.json), top-k also to brute force over tiny
arrays, block selection to closed forms (one dominant block; uniform blocks).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.ndimage
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "selection_cases.json")))


def _arr(rows):
    conv = {"nan": np.nan, "-0": -0.0}
    return np.array([[conv.get(v, v) if isinstance(v, str) else v for v in r] for r in rows],
                    dtype=np.float32)


# ---------------------------------------------------------------- pooling
@pytest.mark.parametrize("n,k", [(1, 7), (5, 7), (50, 7), (49, 3), (33, 1), (100, 9)])
def test_pool_max_is_scipy_maximum_filter(n, k):
    x = synth.score_array(7, 3, n, signed=True)
    y = oracle.pool(x, oracle.RED_MAX, k)
    ref = scipy.ndimage.maximum_filter1d(x.astype(np.float64), size=k, axis=1, mode="constant",
                                         cval=-np.inf)
    np.testing.assert_array_equal(y, ref)


@pytest.mark.parametrize("n,k", [(1, 7), (5, 7), (50, 7), (33, 5)])
def test_pool_mean_divides_by_in_range_count(n, k):
    x = synth.score_array(8, 2, n).astype(np.float64)
    y = oracle.pool(x, 3, k)
    s = scipy.ndimage.uniform_filter1d(x, size=k, axis=1, mode="constant", cval=0.0) * k
    c = scipy.ndimage.uniform_filter1d(np.ones(n), size=k, mode="constant", cval=0.0) * k
    np.testing.assert_allclose(y, s / c[None, :], rtol=1e-12)


# ---------------------------------------------------------------- pages
def test_pages_golden():
    case = GOLD["pages"][0]
    x = np.array(case["x"], dtype=np.float64)
    zmax, arg = oracle.pages(x, case["P"], 2)
    zsum, _ = oracle.pages(x, case["P"], 1)
    np.testing.assert_array_equal(zmax, case["max"])
    np.testing.assert_array_equal(arg, case["argmax"])
    np.testing.assert_array_equal(zsum, case["sum"])


def test_head_reduce_then_pool_then_page_order():
    x = np.array([[0, 0, 5, 0, 0, 0, 0, 0], [0, 0, 0, 0, 0, 0, 0, 9]], dtype=np.float64)
    y, z, arg = oracle.pool_pages(x, head_mode=2, pool_mode=2, pool_k=3, P=4, page_mode=1)
    # max over heads -> [0,0,5,0,0,0,0,9]; max-pool 3 -> [0,5,5,5,0,0,9,9]; page sums 15, 18
    np.testing.assert_array_equal(y, [[0, 5, 5, 5, 0, 0, 9, 9]])
    np.testing.assert_array_equal(z, [[15, 18]])
    np.testing.assert_array_equal(arg, [[1, 6]])


def test_head_reduce_hand_worked():
    """Head reduction over the rows, worked by hand: SUM (the per-layer score summed
    over all heads, CLAA "Three design decisions"), MEAN (the mean over lookahead
    queries, CLAA Speculative Prefill) and MAX ([DELTA] key design 2).  Summing
    along the token axis, or keeping one row, fails every line."""
    x = np.array([[1.0, 2.0, -3.0, 0.5],
                  [4.0, -1.0, 3.0, 0.25],
                  [0.0, 0.0, 1.0, 0.25]])
    np.testing.assert_array_equal(oracle.head_reduce(x, oracle.RED_SUM), [[5.0, 1.0, 1.0, 1.0]])
    np.testing.assert_array_equal(oracle.head_reduce(x, oracle.RED_MAX), [[4.0, 2.0, 3.0, 0.5]])
    np.testing.assert_allclose(oracle.head_reduce(x, oracle.RED_MEAN),
                               [[5.0 / 3, 1.0 / 3, 1.0 / 3, 1.0 / 3]], rtol=1e-15)
    np.testing.assert_array_equal(oracle.head_reduce(x, oracle.RED_NONE), x)
    # SUM over heads, then max-pool 3 ([5, 5, 1, 1]), then page sums with P = 2
    y, z, arg = oracle.pool_pages(x, head_mode=oracle.RED_SUM, pool_mode=oracle.RED_MAX, pool_k=3,
                                  P=2, page_mode=oracle.RED_SUM)
    np.testing.assert_array_equal(y, [[5.0, 5.0, 1.0, 1.0]])
    np.testing.assert_array_equal(z, [[10.0, 2.0]])
    np.testing.assert_array_equal(arg, [[0, 2]])


# ---------------------------------------------------------------- layers
def test_aggregate_identical_layers():
    s = synth.score_array(3, 4, 64)
    one = oracle.aggregate_layers([s], 4)
    np.testing.assert_allclose(one.sum(), 1.0, rtol=1e-12)
    many = oracle.aggregate_layers([s] * 5, 4)
    np.testing.assert_allclose(many, 5 * one, rtol=1e-12)
    np.testing.assert_allclose(oracle.aggregate_layers([s] * 3, 2), s.astype(np.float64).sum(axis=0))


def test_aggregate_hand_built():
    a = np.array([[1.0, 3.0], [0.0, 0.0]])      # head sum [1, 3], norm 4
    b = np.array([[2.0, 0.0], [0.0, 2.0]])      # head sum [2, 2], norm 4
    np.testing.assert_allclose(oracle.aggregate_layers([a, b], 4), [0.75, 1.25])
    np.testing.assert_allclose(oracle.aggregate_layers([a, b], 2), [2.0, 3.0])


# ---------------------------------------------------------------- clusters
def test_cluster_golden():
    c = GOLD["cluster"][0]
    p = oracle.cluster_priority(np.array(c["page"]), np.array(c["page_arg"]), c["n"], c["theta"], c["r"])
    np.testing.assert_array_equal(p, c["priority"])


def test_cluster_theta_edges_and_r0():
    page = np.array([[0.5, 0.7]])
    arg = np.array([[3, 6]])
    assert oracle.cluster_priority(page, arg, 8, 0.7000001, 1).sum() == 0
    np.testing.assert_array_equal(oracle.cluster_priority(page, arg, 8, 0.7, 1), [[0, 0, 0, 0, 0, 1, 1, 1]])
    np.testing.assert_array_equal(oracle.cluster_priority(page, arg, 8, 0.0, 0), [[0, 0, 0, 1, 0, 0, 1, 0]])


# ---------------------------------------------------------------- top-k
def test_topk_golden():
    for block in GOLD["topk"]:
        S = _arr(block["S"])
        prio = np.array(block["priority"], dtype=np.uint8) if "priority" in block else None
        for case in block["cases"]:
            got = oracle.topk(S, case["budget"], prio, case.get("n_forced", 0))
            np.testing.assert_array_equal(got, case["idx"])


@settings(max_examples=200, deadline=None)
@given(st.lists(st.sampled_from([0.0, -0.0, 1.0, 2.0, 2.5, -1.0, float("inf"), float("-inf"), float("nan")]),
                min_size=1, max_size=24),
       st.data())
def test_topk_brute_force(vals, data):
    n = len(vals)
    S = np.array([vals], dtype=np.float32)
    prio = np.array([data.draw(st.lists(st.integers(0, 1), min_size=n, max_size=n))], dtype=np.uint8)
    budget = data.draw(st.integers(0, n))

    def key(i):
        v = vals[i]
        return (-int(prio[0, i]), 1 if math.isnan(v) else 0, 0.0 if math.isnan(v) else -v, i)

    want = sorted(sorted(range(n), key=key)[:budget])
    got = oracle.topk(S, budget, prio, 2)
    assert list(got[0, :budget]) == want
    assert list(got[0, budget:]) == [n, n + 1]


# ---------------------------------------------------------------- block select
def _chunk(Qf, Kf):
    return synth.to_bf16(Qf), synth.to_bf16(Kf)


def test_block_select_dominant_block():
    """One block holding >= 0.9 of the mass is the only block kept."""
    d_k, blk, L, Lq = 64, 4, 32, 8
    Kf = np.zeros((1, L, d_k), dtype=np.float32)
    Kf[0, 8:12, 0] = 8.0                 # block 2 points along axis 0
    Qf = np.zeros((1, Lq, d_k), dtype=np.float32)
    Qf[0, :, 0] = 8.0
    Q, K = _chunk(Qf, Kf)
    M = oracle.block_select(Q, K, Lq=Lq, L=L, d_k=d_k, H_q=1, H_kv=1, q_pos0=L - Lq, block=blk)
    assert M.shape == (1, 2, 8)
    np.testing.assert_array_equal(M[0, :, 2], [1, 1])
    assert M.sum() == 2


@pytest.mark.parametrize("V", [1, 2, 3, 7, 13, 21])
def test_block_select_uniform_blocks(V):
    """V equally likely visible blocks keep ceil(0.9 V) of them, lowest j first."""
    d_k, blk = 64, 4
    L = V * blk
    Lq = blk
    Kf = np.ones((1, L, d_k), dtype=np.float32)
    Qf = np.ones((1, Lq, d_k), dtype=np.float32)
    Q, K = _chunk(Qf, Kf)
    M = oracle.block_select(Q, K, Lq=Lq, L=L, d_k=d_k, H_q=1, H_kv=1, q_pos0=L - Lq, block=blk)
    kept = int(M.sum())
    want = math.ceil(0.9 * V)      # 0.9 V is not an integer for these V
    assert kept == want, (kept, want)
    np.testing.assert_array_equal(np.nonzero(M[0, 0])[0], np.arange(want))


@pytest.mark.parametrize("q_lo,q_hi,want", [(1.5, 2.5, [1, 1]), (2.0, 3.0, [1, 0])])
def test_block_select_mass_closed_form(q_lo, q_hi, want):
    """Two visible key blocks with block-mean logits x and 0: the first holds e^x / (e^x + 1)
    of the softmax mass, and the second is kept iff that is below 0.9.  Query rows alternate
    q_lo, q_hi (mean x/8 on axis 0), key block 0 alternates 7, 9 (mean 8), block 1 is zero, and
    scale = 1/sqrt(64), so x = 2.0 (mass 0.881: keep both) or x = 2.5 (mass 0.924: keep one).
    Block sums instead of means, a missing scale, or the last query row instead of the mean
    block query all flip the first case; a base-2 softmax flips the second."""
    d_k, blk, L, Lq = 64, 4, 8, 4
    Kf = np.zeros((1, L, d_k), dtype=np.float32)
    Kf[0, 0:4, 0] = [7.0, 9.0, 7.0, 9.0]
    Qf = np.zeros((1, Lq, d_k), dtype=np.float32)
    Qf[0, :, 0] = [q_lo, q_hi, q_lo, q_hi]
    Q, K = _chunk(Qf, Kf)
    x = 0.125 * 8.0 * (q_lo + q_hi) / 2
    assert (math.exp(x) / (math.exp(x) + 1) < 0.9) == (want == [1, 1])
    M = oracle.block_select(Q, K, Lq=Lq, L=L, d_k=d_k, H_q=1, H_kv=1, q_pos0=L - Lq, block=blk)
    np.testing.assert_array_equal(M[0, 0], want)


def test_block_select_causal_visibility():
    """Query block i sees KV blocks j with first token <= its last position."""
    d_k, blk, L, Lq = 64, 4, 24, 8
    Kf = np.ones((1, L, d_k), dtype=np.float32)
    Qf = np.ones((1, Lq, d_k), dtype=np.float32)
    Q, K = _chunk(Qf, Kf)
    M = oracle.block_select(Q, K, Lq=Lq, L=L, d_k=d_k, H_q=1, H_kv=1, q_pos0=L - Lq, block=blk,
                            p_mass=1.01)
    # block i=0 ends at position 19 -> blocks 0..4 visible; i=1 ends at 23 -> 0..5
    np.testing.assert_array_equal(M[0, 0], [1, 1, 1, 1, 1, 0])
    np.testing.assert_array_equal(M[0, 1], [1, 1, 1, 1, 1, 1])


# ---------------------------------------------------------------- union
def test_union_golden():
    c = GOLD["union"][0]
    indptr, idx = oracle.block_union_pagetable(np.array(c["M"], dtype=np.uint8), H_q=c["H_q"], H_kv=c["H_kv"])
    np.testing.assert_array_equal(indptr, c["kv_indptr"])
    np.testing.assert_array_equal(idx, c["kv_indices"])


@pytest.mark.parametrize("sub", [0, 2, 1])
def test_union_minimal_and_covering(sub):
    """Every selected (h, i, j) is covered by its group's table and every listed
    page has a witness: the table is the unique smallest one."""
    H_q, H_kv, n_qb, n_kvb = 8, 2, 5, 40
    M = synth.block_mask(9, H_q, n_qb, n_kvb, density_den=12)
    indptr, idx = oracle.block_union_pagetable(M, H_q=H_q, H_kv=H_kv, sub_group=sub)
    sg = (H_q // H_kv) if sub == 0 else sub
    for s in range(H_q // sg):
        T = idx[indptr[s]:indptr[s + 1]]
        assert np.all(np.diff(T) > 0)
        heads = range(s * sg, (s + 1) * sg)
        for h in heads:
            for i in range(n_qb):
                assert set(np.nonzero(M[h, i])[0]) <= set(T)
        for j in T:
            assert any(M[h, i, j] for h in heads for i in range(n_qb))


# ---------------------------------------------------------------- token page tables
def test_token_pagetable_hand_worked():
    """[CompactAttention] per-group page table from kept token positions, worked by
    hand with P = 4 and 5 pages (20 tokens): -1 padding and a token past the
    cache name no page, repeats collapse, lists are ascending."""
    idx = np.array([[0, 3, 9, 17, -1],
                    [2, 8, 19, 25, 11],
                    [4, 5, 6, 7, -1],
                    [-1, -1, -1, -1, -1]])
    ptr, ind = oracle.token_pagetable(idx, P=4, n_pages=5, rows_per_group=2)
    np.testing.assert_array_equal(ptr, [0, 3, 4])
    np.testing.assert_array_equal(ind, [0, 2, 4, 1])
    ptr, ind = oracle.token_pagetable(idx, P=4, n_pages=5, rows_per_group=1)
    np.testing.assert_array_equal(ptr, [0, 3, 6, 7, 7])
    np.testing.assert_array_equal(ind, [0, 2, 4, 0, 2, 4, 1])
    # P = 1: the table is the sorted set of valid tokens itself
    ptr, ind = oracle.token_pagetable(idx[:1], P=1, n_pages=20)
    np.testing.assert_array_equal(ind, [0, 3, 9, 17])


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 6), st.integers(1, 40), st.integers(1, 9), st.integers(1, 3), st.data())
def test_token_pagetable_covers_minimally(H0, n, P, rpg, data):
    """Coverage and minimality: every valid token's page is listed for its group,
    every listed page holds a kept token of the group, lists strictly ascending."""
    H = H0 * rpg
    n_pages = data.draw(st.integers(1, 12))
    idx = np.array(data.draw(st.lists(st.lists(st.integers(-2, n_pages * P + 3), min_size=n,
                                               max_size=n), min_size=H, max_size=H)))
    ptr, ind = oracle.token_pagetable(idx, P=P, n_pages=n_pages, rows_per_group=rpg)
    for s in range(H0):
        lst = ind[ptr[s]:ptr[s + 1]]
        assert np.all(np.diff(lst) > 0)
        toks = idx[s * rpg:(s + 1) * rpg].reshape(-1)
        toks = toks[(toks >= 0) & (toks < n_pages * P)]
        for t in toks:
            assert t // P in lst
        for pg in lst:
            assert np.any((toks >= pg * P) & (toks < pg * P + P))

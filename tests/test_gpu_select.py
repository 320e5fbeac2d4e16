"""GPU parity of the selection kernels on seeded arrays (no score kernel involved).

Integer outputs (top-k indices, page argmax, cluster priority, block-union page
tables) must equal the oracle's exactly; float outputs (pooled values, page
sums, layer aggregates) agree within float32 rounding of the same sums.  Inputs
include forced ties, +-0, NaN, ragged sizes and the full 32K and 128K layer sizes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "selection_cases.json")))


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available()
    return k


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# ------------------------------------------------------------------ pool / pages
POOL_CASES = [
    # H, n, head_reduce, pool, k, P, page_reduce
    (1, 496, 0, 2, 7, 0, 1),          # Tiny: max-pool 7, no pages
    (8, 32736, 0, 2, 7, 0, 1),        # Llama 32K prefix
    (8, 131040, 0, 0, 7, 16, 2),      # Mistral 128K: page max + argmax
    (32, 5000, 2, 0, 7, 16, 1),       # DELTA: max over heads, page sum
    (3, 2049, 1, 3, 5, 16, 1),        # head sum, mean pool, page sum
    (2, 1000, 0, 3, 7, 7, 2),         # odd page size
    (4, 37, 0, 2, 9, 16, 2),          # shorter than a page + halo
    (1, 1, 0, 2, 7, 16, 1),
    (5, 4100, 2, 2, 3, 0, 1),
]


@pytest.mark.parametrize("H,n,hr,pool,k,P,pr", POOL_CASES)
def test_pool_pages(kvs, H, n, hr, pool, k, P, pr):
    x = synth.score_array(1000 + n, H, n)
    pooled, page, arg = kvs.kvs_pool_pages(dev(x), n, head_reduce=hr, pool=pool, pool_k=k, P=P,
                                           page_reduce=pr)
    torch.cuda.synchronize()
    y, z, a = oracle.pool_pages(x, head_mode=hr, pool_mode=pool, pool_k=k, P=P, page_mode=pr)
    np.testing.assert_allclose(pooled.cpu().numpy(), y, rtol=5e-6, atol=0)
    if P:
        np.testing.assert_allclose(page.cpu().numpy(), z, rtol=5e-6, atol=0)
        if hr != 1 and pool != 3:   # values are exact copies of the input: argmax is exact
            np.testing.assert_array_equal(arg.cpu().numpy(), a)


def test_pages_golden(kvs):
    c = GOLD["pages"][0]
    x = np.array(c["x"], dtype=np.float32)
    for pr, key in ((2, "max"), (1, "sum")):
        _, page, arg = kvs.kvs_pool_pages(dev(x), x.shape[1], P=c["P"], page_reduce=pr)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(page.cpu().numpy(), c[key])
        np.testing.assert_array_equal(arg.cpu().numpy(), c["argmax"])


# ------------------------------------------------------------------ top-k
TOPK_CASES = [
    # H, n, budget, n_forced, levels, with_priority
    (1, 1, 1, 0, 0, False),
    (1, 7, 3, 2, 3, True),
    (1, 496, 64, 16, 0, False),
    (1, 496, 64, 16, 5, False),
    (8, 32736, 1024, 32, 0, False),
    (8, 131040, 1024, 32, 0, True),
    (8, 131040, 1024, 32, 9, True),      # heavy ties inside and outside the priority set
    (1, 16384, 3276, 0, 0, False),
    (3, 4097, 0, 5, 0, False),
    (3, 4097, 4097, 0, 4, True),
    (2, 2048, 1000, 0, 2, False),        # two values only: ties decide almost everything
    (4, 3001, 1500, 0, 0, True),
    # rows selected across all their parts (more candidates than one workgroup holds)
    (1, 131072, 26214, 0, 0, False),     # 20% of a 128K row
    (2, 40000, 6000, 3, 7, True),        # ties, NaN, +-inf, priority; three parts
    (3, 50000, 20000, 2, 2, False),      # two values only: ties spread over the parts
    (2, 32769, 16385, 0, 5, True),       # last part of one element
    (1, 262144, 100000, 0, 0, False),    # the most parts this path takes
    (1, 262145, 100000, 0, 3, False),    # one part more: the single-workgroup merge
    # stage-1 parts of 8192 elements (the candidates of all parts fit one merge)
    (1, 16385, 1000, 0, 3, True),        # last part of one element
    (2, 40000, 3000, 2, 5, True),        # five parts, ties across part edges
    (2, 131040, 1025, 0, 0, False),      # one slot too many for small parts: parts of 16384
    # two values only: the first pass leaves thousands of keys in the threshold bin
    (1, 16384, 3000, 0, 2, False),       # one part: later passes over the registers
    (2, 40000, 3000, 2, 2, True),        # small parts and a merge of tied candidates
    (100, 20000, 500, 0, 3, True),       # many rows: workgroup i takes row i % 100
]


@pytest.mark.parametrize("H,n,budget,nf,levels,use_prio", TOPK_CASES)
def test_topk_bit_exact(kvs, H, n, budget, nf, levels, use_prio):
    x = synth.score_array(2000 + n + budget, H, n, levels=levels, signed=levels > 0,
                          with_zeros=levels > 0)
    if levels > 0 and n > 10:
        x[0, 3] = np.nan
        x[-1, n // 2] = np.float32(-np.inf)
        x[-1, n // 3] = np.float32(np.inf)
    prio = synth.priority_array(n, H, n) if use_prio else None
    got = kvs.kvs_topk(dev(x), n, budget, priority=dev(prio) if use_prio else None, n_forced=nf)
    torch.cuda.synchronize()
    want = oracle.topk(x, budget, prio, nf)
    np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_topk_golden(kvs):
    for block in GOLD["topk"]:
        conv = {"nan": np.nan, "-0": -0.0}
        S = np.array([[conv.get(v, v) if isinstance(v, str) else v for v in r] for r in block["S"]],
                     dtype=np.float32)
        prio = np.array(block["priority"], dtype=np.uint8) if "priority" in block else None
        for case in block["cases"]:
            got = kvs.kvs_topk(dev(S), S.shape[1], case["budget"],
                               priority=dev(prio) if prio is not None else None,
                               n_forced=case.get("n_forced", 0))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got.cpu().numpy(), case["idx"])


def test_topk_row_stride(kvs):
    """Rows read through ld > n (candidate prefix of a longer score row)."""
    H, L, n = 4, 3000, 2968
    x = synth.score_array(77, H, L)
    got = kvs.kvs_topk(dev(x), n, 300, n_forced=32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.topk(x[:, :n], 300, None, 32))


@pytest.mark.parametrize("H,n,budget,nf,ld", [(3, 5000, 700, 16, 5000), (2, 40000, 3000, 2, 40008),
                                              (1, 131040, 26208, 0, 131072), (4, 300, 0, 5, 300)])
def test_topk_values(kvs, H, n, budget, nf, ld):
    """kvs_topk's val output: the input scores at the oracle's indices, bit for bit,
    in index order; NaN for the forced suffix (one-part, merged and wide rows)."""
    x = synth.score_array(5100 + n, H, ld, levels=5, signed=True, with_zeros=True)
    idx, val = kvs.kvs_topk(dev(x), n, budget, n_forced=nf, ld=ld, want_val=True)
    torch.cuda.synchronize()
    want = oracle.topk(x[:, :n], budget, None, nf)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    v = val.cpu().numpy()
    gathered = np.take_along_axis(x, want[:, :budget], axis=1)
    assert np.array_equal(v[:, :budget].view(np.uint32), gathered.view(np.uint32))
    assert np.isnan(v[:, budget:]).all()


# ------------------------------------------------------------------ clusters
@pytest.mark.parametrize("H,n,P,theta,r", [(8, 131040, 16, 2e-3, 3), (2, 1000, 16, 1.5, 3),
                                           (1, 100, 7, 0.0, 0), (3, 5000, 16, 3.0, 20)])
def test_cluster_priority_bit_exact(kvs, H, n, P, theta, r):
    x = synth.score_array(3000 + n, H, n)
    if theta == 2e-3:
        x = x * np.float32(1e-3)          # page maxima straddle theta
    z, arg = oracle.pages(x, P, oracle.RED_MAX)
    z32 = z.astype(np.float32)
    prio = kvs.kvs_cluster_priority(dev(z32), dev(arg.astype(np.int32)), P, n, theta, r)
    torch.cuda.synchronize()
    want = oracle.cluster_priority(z32, arg, n, float(np.float32(theta)), r)
    np.testing.assert_array_equal(prio.cpu().numpy(), want)


def test_cluster_golden(kvs):
    c = GOLD["cluster"][0]
    page = np.array(c["page"], dtype=np.float32)
    prio = kvs.kvs_cluster_priority(dev(page), dev(np.array(c["page_arg"], dtype=np.int32)), c["P"], c["n"],
                                    c["theta"], c["r"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(prio.cpu().numpy(), c["priority"])


# ------------------------------------------------------------------ layers
@pytest.mark.parametrize("mode", [4, 2], ids=["sum_l1", "max"])
@pytest.mark.parametrize("H,n,layers", [(8, 16384, 5), (1, 777, 3), (3, 70000, 2)])
def test_aggregate_layers(kvs, mode, H, n, layers):
    xs = [synth.score_array(4000 + l, H, n) for l in range(layers)]
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    for l, x in enumerate(xs):
        kvs.kvs_aggregate_layers(acc, dev(x), n, mode, first_layer=(l == 0))
    torch.cuda.synchronize()
    want = oracle.aggregate_layers(xs, mode)
    np.testing.assert_allclose(acc.cpu().numpy(), want, rtol=1e-5, atol=0)


# ------------------------------------------------------------------ union
@pytest.mark.parametrize("H_q,H_kv,sub,n_qb,n_kvb,den", [
    (32, 8, 0, 16, 2048, 40), (32, 8, 2, 16, 2048, 40), (8, 1, 4, 3, 777, 5),
    (4, 4, 0, 1, 10, 3), (16, 2, 1, 5, 4096, 200), (8, 2, 0, 2, 33, 1000)])
def test_union_bit_exact(kvs, H_q, H_kv, sub, n_qb, n_kvb, den):
    M = synth.block_mask(5000 + n_kvb, H_q, n_qb, n_kvb, density_den=den)
    indptr, indices = kvs.kvs_block_union_pagetable(dev(M), H_q, H_kv, sub)
    torch.cuda.synchronize()
    want_ptr, want_idx = oracle.block_union_pagetable(M, H_q=H_q, H_kv=H_kv, sub_group=sub)
    got_ptr = indptr.cpu().numpy()
    np.testing.assert_array_equal(got_ptr, want_ptr)
    np.testing.assert_array_equal(indices.cpu().numpy()[:got_ptr[-1]], want_idx)


def test_union_golden(kvs):
    c = GOLD["union"][0]
    M = np.array(c["M"], dtype=np.uint8)
    indptr, indices = kvs.kvs_block_union_pagetable(dev(M), c["H_q"], c["H_kv"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(indptr.cpu().numpy(), c["kv_indptr"])
    np.testing.assert_array_equal(indices.cpu().numpy()[:c["kv_indptr"][-1]], c["kv_indices"])


@pytest.mark.parametrize("n,budget", [(5000, 700), (131040, 1024), (20000, 19999)])
def test_topk_equal_values(kvs, n, budget):
    """Every value of a class equal: no radix pass, ties decided by index."""
    x = np.full((2, n), np.float32(0.25), dtype=np.float32)
    x[1, ::7] = np.float32(0.5)
    prio = synth.priority_array(77, 2, n)
    for pr in (None, prio):
        got = kvs.kvs_topk(dev(x), n, budget, priority=dev(pr) if pr is not None else None,
                           n_forced=3)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), oracle.topk(x, budget, pr, 3))


@pytest.mark.parametrize("n,top,budget", [(5000, 200, 1200), (131040, 200, 1200),
                                           (131072, 10000, 26214)],
                         ids=["one_part", "parts_and_merge", "wide_rows"])
def test_topk_whole_bin(kvs, n, top, budget):
    """The budget ends exactly at the edge of a radix bin, after the first, second and third
    digit (rows 0, 1, 2: below a block of 4.0 the next values are 2.0, 1 + 2^-12 and
    1 + 2^-22 over a floor of 1.0), so the selection stops at that bin; the chosen set must
    still be the oracle's, in one part, through the candidate merge and across wide rows."""
    x = np.ones((3, n), dtype=np.float32)
    nxt = [np.float32(2.0), np.float32(1.0 + 2.0 ** -12), np.float32(1.0 + 2.0 ** -22)]
    for r in range(3):
        order = np.argsort(synth.u64(500 + r, 1, np.arange(n)))   # a seeded placement
        x[r, order[:top]] = np.float32(4.0)
        x[r, order[top:budget]] = nxt[r]
    got = kvs.kvs_topk(dev(x), n, budget, n_forced=5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.topk(x, budget, None, 5))


@pytest.mark.parametrize("n,budget", [(16000, 1600), (131040, 1024), (60000, 20000)])
def test_topk_narrow_values(kvs, n, budget):
    """Values within a few ulps of each other share all their leading bits."""
    steps = (synth.u64(91, 1, np.arange(2 * n)) % np.uint64(37)).astype(np.float32)
    x = (np.float32(1.0) + steps * np.float32(2.0 ** -20)).reshape(2, n).astype(np.float32)
    x[1] = np.float32(-3.0) - steps.reshape(2, n)[1] * np.float32(2.0 ** -18)
    prio = synth.priority_array(92, 2, n, 1, 50)
    for pr in (None, prio):
        got = kvs.kvs_topk(dev(x), n, budget, priority=dev(pr) if pr is not None else None)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), oracle.topk(x, budget, pr, 0))


def test_deterministic_selection(kvs):
    x = synth.score_array(9, 8, 131040, levels=50)
    a = kvs.kvs_topk(dev(x), 131040, 1024, n_forced=32).cpu().numpy()
    b = kvs.kvs_topk(dev(x), 131040, 1024, n_forced=32).cpu().numpy()
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ fused select
SELECT_POOL_CASES = [
    # H, n, budget, n_forced, k, levels
    (1, 496, 64, 16, 7, 0),            # Tiny: max-pool 7 + window
    (8, 32736, 1024, 32, 7, 0),        # Llama 32K prefix
    (8, 131040, 1024, 32, 7, 0),       # Mistral 128K prefix
    (3, 4097, 700, 3, 9, 6),           # ragged tail, ties, NaN / inf
    (2, 5, 2, 0, 7, 0),                # window wider than the row
    (2, 9000, 4500, 0, 1, 4),          # k = 1: plain top-k
    (1, 20000, 100, 0, 2049, 0),       # widest supported window
    (2, 8, 3, 0, 7, 0),                # register window wider than the row
    (3, 12, 5, 1, 31, 0),              # widest register-window pooling
    (2, 48, 10, 0, 33, 3),             # beyond the register window: staged path
    (2, 16388, 500, 0, 7, 5),          # second part of four elements
    (1, 131072, 26214, 0, 7, 0),       # GemFilter keep rate 20%, across all parts
    (2, 40000, 9000, 5, 7, 6),         # across all parts, with ties
]


@pytest.mark.parametrize("H,n,budget,nf,k,levels", SELECT_POOL_CASES)
def test_select_max_pool_bit_exact(kvs, H, n, budget, nf, k, levels):
    """Max-pooled values are exact float32 copies: the selection is unique."""
    x = synth.score_array(6000 + n + k, H, n, levels=levels, signed=levels > 0,
                          with_zeros=levels > 0)
    if levels > 0:
        x[0, 17] = np.nan
        x[-1, n // 2] = np.float32(np.inf)
        x[-1, n // 3] = np.float32(-np.inf)
    a = kvs.select_args(budget=budget, n_forced=nf, pool=kvs.RED_MAX, pool_k=k)
    got = kvs.kvs_select(dev(x), n, a)
    torch.cuda.synchronize()
    want = oracle.topk(oracle.pool(x, oracle.RED_MAX, k), budget, None, nf)
    np.testing.assert_array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("H,n,budget,k", [(8, 32736, 1024, 7), (2, 3001, 1500, 5), (1, 70, 9, 31),
                                          (2, 16, 4, 31), (3, 32768, 100, 33), (2, 40000, 900, 9)])
def test_select_mean_pool(kvs, H, n, budget, k):
    """float32 left-to-right means against fp64 ones: decided elements agree."""
    from helpers import assert_topk_parity
    x = synth.score_array(6100 + n, H, n)
    a = kvs.select_args(budget=budget, n_forced=4, pool=kvs.RED_MEAN, pool_k=k)
    got = kvs.kvs_select(dev(x), n, a).cpu().numpy()
    assert np.array_equal(got[:, budget:], np.tile(np.arange(n, n + 4), (H, 1)))
    assert_topk_parity(got, oracle.pool(x, oracle.RED_MEAN, k), budget, rel=1e-5)


SELECT_CLUSTER_CASES = [
    # H, n, budget, n_forced, P, theta, r, scale
    (8, 131040, 1024, 32, 16, 2e-3, 3, 1e-3),   # Mistral 128K shape; maxima straddle theta
    (2, 1000, 100, 0, 16, 1.5, 3, 1.0),
    (1, 100, 10, 3, 7, 0.0, 0, 1.0),
    (3, 5000, 400, 0, 16, 3.0, 20, 1.0),
    (2, 9000, 300, 0, 1, 2.0, 2, 1.0),          # every token a page
    (2, 12000, 2000, 0, 24, 2.5, 1000, 1.0),    # P + r at the halo limit
    (1, 4096, 4096, 0, 16, 1.0, 3, 1.0),        # budget = n
    (2, 20, 5, 0, 16, 0.5, 3, 1.0),             # partial last page, one thread
    (1, 48, 7, 2, 16, 1.0, 16, 1.0),            # widest register-window radius
    (3, 16388, 500, 0, 16, 2.0, 3, 1.0),        # second part of four elements
    (2, 16390, 500, 0, 16, 2.0, 3, 1.0),        # n % 4 != 0: staged path
    (2, 60000, 20000, 4, 16, 2.0, 3, 1.0),      # across all parts
    (3, 70000, 1024, 4, 16, 1.0, 16, 1.0),      # parts of 8192: centres reach across part edges
]


@pytest.mark.parametrize("H,n,budget,nf,P,theta,r,scale", SELECT_CLUSTER_CASES)
def test_select_cluster_bit_exact(kvs, H, n, budget, nf, P, theta, r, scale):
    x = synth.score_array(6200 + n + r, H, n) * np.float32(scale)
    x[0, min(5, n - 1)] = np.nan                   # its page has no centre
    a = kvs.select_args(budget=budget, n_forced=nf, cluster_P=P, cluster_theta=theta, cluster_r=r)
    got = kvs.kvs_select(dev(x), n, a)
    torch.cuda.synchronize()
    z, arg = oracle.pages(x, P, oracle.RED_MAX)
    prio = oracle.cluster_priority(z, arg, n, float(np.float32(theta)), r)
    want = oracle.topk(x, budget, prio, nf)
    np.testing.assert_array_equal(got.cpu().numpy(), want)


def test_select_workspace_reuse(kvs):
    """One workspace, sized for the largest call, serves calls of different
    shapes, budgets and transforms back to back (stale candidates of an
    earlier call never leak into a later one)."""
    calls = [
        (8, 131040, dict(budget=1024, n_forced=32, cluster_P=16, cluster_theta=2e-3, cluster_r=3)),
        (3, 50000, dict(budget=77)),
        (8, 32736, dict(budget=1024, pool=kvs.RED_MAX, pool_k=7)),
        (1, 1, dict(budget=1)),
        (5, 131040, dict(budget=0, n_forced=7)),
        (8, 131040, dict(budget=131040)),                   # every part keeps everything
        (2, 131040, dict(budget=3000)),                     # candidates exceed one tile
        (8, 131040, dict(budget=1024, n_forced=32)),
    ]
    nbytes = max(kvs.library().kvs_select_workspace(H, n, kw["budget"]) for H, n, kw in calls)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    for i, (H, n, kw) in enumerate(calls):
        x = synth.score_array(6300 + i, H, n, levels=0 if i % 2 else 40) * np.float32(1e-3)
        got = kvs.kvs_select(dev(x), n, kvs.select_args(**kw), ws=ws)
        torch.cuda.synchronize()
        if kw.get("cluster_P"):
            z, arg = oracle.pages(x, 16, oracle.RED_MAX)
            prio = oracle.cluster_priority(z, arg, n, float(np.float32(2e-3)), 3)
            want = oracle.topk(x, kw["budget"], prio, kw.get("n_forced", 0))
        elif kw.get("pool"):
            want = oracle.topk(oracle.pool(x, oracle.RED_MAX, 7), kw["budget"], None, 0)
        else:
            want = oracle.topk(x, kw["budget"], None, kw.get("n_forced", 0))
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"call {i}")


def test_select_matches_three_call_path(kvs):
    """The fused cluster select equals page max -> cluster priority -> top-k."""
    H, n, P, theta, r = 8, 131040, 16, 2e-3, 3
    x = dev(synth.score_array(6400, H, n) * np.float32(1e-3))
    _, page, parg = kvs.kvs_pool_pages(x, n, P=P, page_reduce=kvs.RED_MAX, want_pooled=False)
    prio = kvs.kvs_cluster_priority(page, parg, P, n, theta, r)
    a = kvs.kvs_topk(x, n, 1024, priority=prio, n_forced=32)
    b = kvs.kvs_select(x, n, kvs.select_args(budget=1024, n_forced=32, cluster_P=P,
                                             cluster_theta=theta, cluster_r=r))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kind,budget", [("plain", 6000), ("plain", 20000), ("pool", 8000),
                                         ("cluster", 6000)])
def test_one_launch_select_late_part_path(kvs, kind, budget):
    """Wide rows (more candidates than one merge holds) run in one launch whose parts exchange
    their statistics, digit histograms and counts.  With the wait bound at 0, every part that
    finds a word of its row missing computes the late parts' words itself: the indices must
    equal the default run's and the oracle's."""
    print(f"late-part select {kind} budget={budget}", flush=True)
    H, n, nf = 3, 50000, 4
    x = synth.score_array(7100 + budget, H, n, levels=6 if kind == "plain" else 0,
                          signed=kind == "plain", with_zeros=kind == "plain")
    prio = synth.priority_array(n, H, n) if kind == "plain" else None
    if kind == "plain":
        run = lambda: kvs.kvs_topk(dev(x), n, budget, priority=dev(prio), n_forced=nf)
        want = oracle.topk(x, budget, prio, nf)
    elif kind == "pool":
        a = kvs.select_args(budget=budget, n_forced=nf, pool=kvs.RED_MAX, pool_k=7)
        run = lambda: kvs.kvs_select(dev(x), n, a)
        want = oracle.topk(oracle.pool(x, oracle.RED_MAX, 7), budget, None, nf)
    else:
        x = x * np.float32(1e-3)
        a = kvs.select_args(budget=budget, n_forced=nf, cluster_P=16, cluster_theta=2e-3,
                            cluster_r=3)
        run = lambda: kvs.kvs_select(dev(x), n, a)
        z, arg = oracle.pages(x, 16, oracle.RED_MAX)
        want = oracle.topk(x, budget, oracle.cluster_priority(z, arg, n, float(np.float32(2e-3)), 3),
                           nf)
    base = run().cpu().numpy()
    prev = kvs.kvs_wait_limit(0)
    try:
        late = [run().cpu().numpy() for _ in range(2)]
    finally:
        assert kvs.kvs_wait_limit(prev) == 0
    np.testing.assert_array_equal(base, want)
    for got in late:
        np.testing.assert_array_equal(got, want)


def test_select_grid_larger_than_device(kvs):
    """130 wide rows of three parts each: more workgroups than the device holds at once, so the
    selection takes the launch-per-phase form."""
    H, n, budget = 130, 40000, 10000
    x = synth.score_array(7300, H, n, levels=4, signed=True, with_zeros=True)
    got = kvs.kvs_topk(dev(x), n, budget, n_forced=3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.topk(x, budget, None, 3))

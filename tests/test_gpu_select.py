"""GPU parity of the selection kernels on seeded arrays (no score kernel involved).

Integer outputs (top-k indices, page argmax, cluster priority, block-union page
tables) must equal the oracle's exactly; float outputs (pooled values, page
sums, layer aggregates) agree within float32 rounding of the same sums.  Inputs
include forced ties, +-0, NaN, ragged sizes and the full BASELINE sizes.
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


def test_deterministic_selection(kvs):
    x = synth.score_array(9, 8, 131040, levels=50)
    a = kvs.kvs_topk(dev(x), 131040, 1024, n_forced=32).cpu().numpy()
    b = kvs.kvs_topk(dev(x), 131040, 1024, n_forced=32).cpu().numpy()
    assert np.array_equal(a, b)

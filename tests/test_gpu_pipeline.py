"""End-to-end GPU pipelines for the five workloads against the fp64 oracle.

Each pipeline runs only library kernels on the GPU and only oracle functions on
the host, from the same seeded inputs.  Scores agree within 2e-3; a selection
must agree on every element whose oracle quantity lies more than 2e-3
(relative) away from the selection boundary (the k-th value, theta, or the
0.9 cumulative mass), and the counts must be equal.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_scores_close, assert_topk_parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
REL = 2e-3


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available()
    return k


def _score(kvs, ly):
    a = kvs.score_args(L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv, q_pos0=ly.q_pos0)
    return kvs.kvs_score(kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K), a)


def _oscore(ly):
    return oracle.score(ly.Q, ly.K, L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                        q_pos0=ly.q_pos0)


@pytest.mark.parametrize("which,budget", [("tiny", 64), ("llama32k", 1024)])
def test_window_maxpool_topk(kvs, which, budget):
    """Tiny layer and Llama 32K layer: score -> max-pool 7 over the prefix -> top-budget + window."""
    print(f"pipeline {which}", flush=True)
    ly = synth.tiny() if which == "tiny" else synth.llama_layer()
    n = ly.L - ly.W
    S = _score(kvs, ly)
    pooled, _, _ = kvs.kvs_pool_pages(S, n, pool=kvs.RED_MAX, pool_k=7, ld=ly.L)
    idx = kvs.kvs_topk(pooled, n, budget, n_forced=ly.W)
    torch.cuda.synchronize()
    So = _oscore(ly)
    yo = oracle.pool(So[:, :n], oracle.RED_MAX, 7)
    assert_scores_close(pooled.cpu().numpy(), yo, ly.W * ly.G, ly.L, "pooled")
    got = idx.cpu().numpy()
    assert_topk_parity(got, yo, budget)
    assert np.array_equal(got[:, budget:], np.tile(np.arange(n, ly.L), (ly.H_kv, 1)))
    if ly.spans:   # planted spans dominate the selection
        in_span = np.zeros(n, dtype=bool)
        for a, b in ly.spans:
            in_span[max(0, a - 3):b + 3] = True
        assert in_span[got[:, :budget]].mean() > 0.9


def _robust_priority(So_pref, P, theta, r):
    """Tokens whose cluster priority cannot flip under a 2e-3 relative change."""
    H, n = So_pref.shape
    z, arg = oracle.pages(So_pref, P, oracle.RED_MAX)
    robust = np.ones((H, n), dtype=bool)
    for h in range(H):
        for u in range(z.shape[1]):
            seg = So_pref[h, u * P:min(n, u * P + P)]
            zmax = z[h, u]
            near_theta = abs(zmax - theta) <= REL * theta
            cands = np.nonzero(seg >= zmax * (1 - REL))[0] + u * P
            if near_theta or (len(cands) > 1 and zmax >= theta * (1 - REL)):
                for c in cands:
                    robust[h, max(0, c - r):min(n, c + r + 1)] = False
    return z, arg, robust


def test_cluster_topk_128k(kvs):
    """Mistral 128K layer: score -> page max P=16 -> clusters (theta 2e-3, r 3) -> top-1024 + window."""
    ly = synth.mistral_layer()
    n, P, theta, r, budget = ly.L - ly.W, 16, 2e-3, 3, 1024
    S = _score(kvs, ly)
    _, page, parg = kvs.kvs_pool_pages(S, n, P=P, page_reduce=kvs.RED_MAX, ld=ly.L, want_pooled=False)
    prio = kvs.kvs_cluster_priority(page, parg, P, n, theta, r)
    idx = kvs.kvs_topk(S, n, budget, priority=prio, n_forced=ly.W, ld=ly.L)
    torch.cuda.synchronize()
    So = _oscore(ly)
    Sp = So[:, :n]
    assert_scores_close(S.cpu().numpy(), So, ly.W * ly.G, ly.L, "scores")
    z, arg, robust = _robust_priority(Sp, P, theta, r)
    po = oracle.cluster_priority(z, arg, n, float(np.float32(theta)), r)
    pg = prio.cpu().numpy()
    assert np.array_equal(pg[robust], po[robust]), "cluster priority differs on robust tokens"
    got = idx.cpu().numpy()
    # priority flips (all on non-robust tokens) can move the boundary by that many ranks
    for h in range(ly.H_kv):
        flips = int((pg[h] != po[h]).sum())
        order = np.lexsort((np.arange(n), -Sp[h], -po[h].astype(np.int64)))
        k = budget - 1
        cls = po[h, order[k]]
        lo_rank, hi_rank = max(0, k - flips), min(n - 1, k + flips)
        v_hi, v_lo = Sp[h, order[lo_rank]], Sp[h, order[hi_rank]]
        band = (Sp[h] <= v_hi * (1 + REL)) & (Sp[h] >= v_lo * (1 - REL)) & (po[h] == cls)
        chosen_o = np.zeros(n, bool)
        chosen_o[order[:budget]] = True
        chosen_g = np.zeros(n, bool)
        chosen_g[got[h, :budget]] = True
        decidable = robust[h] & ~band
        assert not (decidable & (chosen_o != chosen_g)).any(), f"row {h}"
        assert np.all(np.diff(got[h, :budget]) > 0)
    assert np.array_equal(got[:, budget:], np.tile(np.arange(n, ly.L), (ly.H_kv, 1)))
    # the clusters capture the planted spans: most kept tokens lie in them
    in_span = np.zeros(n, dtype=bool)
    for a, b in ly.spans:
        in_span[max(0, a - r):b + r] = True
    assert in_span[got[:, :budget]].mean() > 0.9


def test_cross_layer_l1_sum(kvs):
    """32 layers x 16K: per-layer L1-normalised sums, top 20% of all tokens."""
    layers, L = 32, 16384
    budget = int(0.2 * L)
    acc = torch.empty(L, dtype=torch.float32, device="cuda")
    per_layer = []
    for l in range(layers):
        ly = synth.cross_layer(l, L=L)
        S = _score(kvs, ly)
        kvs.kvs_aggregate_layers(acc, S, L, kvs.RED_SUM_L1, first_layer=(l == 0))
        per_layer.append(_oscore(ly))
        if l % 8 == 0:
            print(f"layer {l}", flush=True)
    idx = kvs.kvs_topk(acc.view(1, L), L, budget)
    torch.cuda.synchronize()
    Ao = oracle.aggregate_layers(per_layer, oracle.RED_SUM_L1)
    np.testing.assert_allclose(acc.cpu().numpy(), Ao, rtol=REL, atol=REL * 1e-3 * layers / L)
    np.testing.assert_allclose(Ao.sum(), layers, rtol=1e-9)
    assert_topk_parity(idx.cpu().numpy(), Ao[None, :], budget)


def test_chunk_block_union(kvs):
    """Chunked prefill at 128K: block select (64, top-p 0.9) -> Q-block union -> group union -> CSR."""
    ch = synth.chunk_select()
    a = kvs.block_select_args(Lq=ch.Lq, L=ch.L, d_k=ch.d_k, H_q=ch.H_q, H_kv=ch.H_kv,
                              q_pos0=ch.q_pos0, block=ch.block, p_mass=0.9)
    M = kvs.kvs_block_select(kvs.bf16_from_bits(ch.Qc), kvs.bf16_from_bits(ch.K), a)
    indptr, indices = kvs.kvs_block_union_pagetable(M, ch.H_q, ch.H_kv)
    torch.cuda.synchronize()
    Mo, before = oracle.block_select(ch.Qc, ch.K, Lq=ch.Lq, L=ch.L, d_k=ch.d_k, H_q=ch.H_q,
                                     H_kv=ch.H_kv, q_pos0=ch.q_pos0, block=ch.block, p_mass=0.9,
                                     return_before=True)
    Mg = M.cpu().numpy()
    decidable = np.abs(before - 0.9) > REL * 0.9
    assert np.array_equal(Mg[decidable], Mo[decidable]), "block mask differs on decidable blocks"
    ptr_o, idx_o = oracle.block_union_pagetable(Mo, H_q=ch.H_q, H_kv=ch.H_kv)
    ptr = indptr.cpu().numpy()
    idx = indices.cpu().numpy()
    G = ch.H_q // ch.H_kv
    n_kvb = Mg.shape[2]
    for s in range(ch.H_kv):
        T_g = np.zeros(n_kvb, bool)
        T_g[idx[ptr[s]:ptr[s + 1]]] = True
        T_o = np.zeros(n_kvb, bool)
        T_o[idx_o[ptr_o[s]:ptr_o[s + 1]]] = True
        assert np.all(np.diff(idx[ptr[s]:ptr[s + 1]]) > 0)
        # the table is exactly the union of the mask the GPU produced
        assert np.array_equal(T_g, Mg[s * G:(s + 1) * G].any(axis=(0, 1)))
        # where it differs from the oracle's table, a boundary decision explains it
        for j in np.nonzero(T_g != T_o)[0]:
            assert (~decidable[s * G:(s + 1) * G, :, j]).any(), (s, j)
    # each planted span is found by its (head, query-block) pairs: its KV blocks are kept
    for g in range(ch.H_kv):
        T = set(idx[ptr[g]:ptr[g + 1]].tolist())
        for (a0, b0) in ch.spans[g]:
            inside = range((a0 + ch.block - 1) // ch.block, b0 // ch.block)
            assert all(j in T for j in inside), (g, a0)

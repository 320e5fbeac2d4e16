"""Streaming selector state (GPU): key-block means cached across prefill chunks
(kvs_block_select_cached) and the CLAA rolling buffer of per-layer scores.

The cached block select must equal the uncached one bit for bit, including
when the keys of the cached blocks have been overwritten (so they are
provably not read again).  The rolling buffer chain (per-layer score ->
sum over heads into slot l mod n -> max over the buffer at the pruning layer
-> top-k) is checked against the oracle's max over the last n layers with
the selection-parity rule.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_topk_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


@pytest.mark.parametrize("L_total,Lq,block,H_q,H_kv,d_k", [(8229, 1024, 64, 32, 8, 128),
                                                        (3000, 512, 64, 8, 2, 64),
                                                        (1000, 300, 32, 4, 4, 128)])
def test_block_select_cached_matches_uncached(kvs, L_total, Lq, block, H_q, H_kv, d_k):
    print(f"chunked prefill L={L_total} Lq={Lq}", flush=True)
    ly = synth.gaussian_layer(17, L=L_total, W=Lq, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=0)
    K = kvs.bf16_from_bits(ly.K)
    rng = np.random.default_rng(3)
    n_kvb_total = (L_total + block - 1) // block
    Kb = torch.empty(H_kv, n_kvb_total, d_k, dtype=torch.float32, device="cuda")
    n_cached = 0
    for c0 in range(0, L_total, Lq):
        L = min(c0 + Lq, L_total)
        rows = L - c0
        Qc = kvs.bf16_from_bits(synth.to_bf16(rng.standard_normal((H_q, rows, d_k)).astype(np.float32)))
        a = kvs.block_select_args(Lq=rows, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=c0, block=block,
                                  k_head_stride=L_total * d_k)
        want = kvs.kvs_block_select(Qc, K, a)
        # the cached call must not read the keys of its cached blocks: overwrite them
        Kc = K.clone()
        Kc[:, :n_cached * block, :] = float("nan")
        got = kvs.kvs_block_select_cached(Qc, Kc, a, Kb, n_cached)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"chunk at {c0}"
        n_cached = L // block


@pytest.mark.parametrize("L_total,Lq,block,H_q,H_kv,d_k", [(6000, 1024, 64, 8, 2, 128),
                                                        (4100, 512, 64, 16, 4, 64)])
def test_block_select_cached_matches_oracle(kvs, L_total, Lq, block, H_q, H_kv, d_k):
    """A chunked prefill (5-8 chunks, growing L) through the cached select, every
    chunk's mask checked against the oracle's block select on the same keys
    (decidable blocks: preceding mass more than 2e-3 relative away from 0.9)."""
    print(f"chunked prefill vs oracle L={L_total} Lq={Lq}", flush=True)
    ly = synth.gaussian_layer(23, L=L_total, W=Lq, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=0)
    K = kvs.bf16_from_bits(ly.K)
    rng = np.random.default_rng(5)
    Kb = torch.empty(H_kv, (L_total + block - 1) // block, d_k, dtype=torch.float32, device="cuda")
    n_cached, chunks = 0, 0
    for c0 in range(0, L_total, Lq):
        L = min(c0 + Lq, L_total)
        rows = L - c0
        qbits = synth.to_bf16(rng.standard_normal((H_q, rows, d_k)).astype(np.float32))
        a = kvs.block_select_args(Lq=rows, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=c0, block=block,
                                  k_head_stride=L_total * d_k)
        got = kvs.kvs_block_select_cached(kvs.bf16_from_bits(qbits), K, a, Kb, n_cached)
        torch.cuda.synchronize()
        want, before = oracle.block_select(qbits, np.ascontiguousarray(ly.K[:, :L]), Lq=rows, L=L,
                                           d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=c0, block=block,
                                           return_before=True)
        dec = np.abs(before - 0.9) > 2e-3 * 0.9
        g = got.cpu().numpy()
        assert np.array_equal(g[dec], want[dec]), f"chunk at {c0}"
        n_cached = L // block
        chunks += 1
    assert chunks >= 5


def test_claa_rolling_buffer(kvs):
    """CLAA: per-layer window scores summed over heads, a buffer of the last n = 4
    layers, the token-wise max at the pruning layer (Eq. 6), then top 20%."""
    L, W, n_buf, layers = 4096, 8, 4, 7
    ring = torch.empty(n_buf, L, dtype=torch.float32, device="cuda")
    kept = []
    for l in range(layers):
        ly = synth.gaussian_layer(90 + l, L=L, W=W, d_k=128, H_q=32, H_kv=8, n_spans=4, span_len=64,
                                  lift=2.0, fixed_span_seed=90, n_fixed=2)
        a = kvs.score_args(L=L, W=W, d_k=128, H_q=32, H_kv=8, q_pos0=ly.q_pos0)
        S = kvs.kvs_score(kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K), a)
        kvs.kvs_pool_pages(S, L, head_reduce=kvs.RED_SUM, out=ring[l % n_buf:l % n_buf + 1])
        kept.append(oracle.score(ly.Q, ly.K, L=L, W=W, d_k=128, H_q=32, H_kv=8, q_pos0=ly.q_pos0))
    agg, _, _ = kvs.kvs_pool_pages(ring, L, head_reduce=kvs.RED_MAX)
    budget = L // 5
    idx = kvs.kvs_topk(agg, L, budget)
    torch.cuda.synchronize()
    want = oracle.aggregate_layers(kept[-n_buf:], oracle.RED_MAX)
    np.testing.assert_allclose(agg.cpu().numpy()[0], want, rtol=2e-3, atol=1e-6)
    assert_topk_parity(idx.cpu().numpy(), want[None, :], budget)


@pytest.mark.slow
def test_claa_ring_all_heads_32k(kvs):
    """CLAA at 32K: each of 9 layers' window scores summed over every head straight into
    slot l mod 4 of the ring (kvs_score ALL_SUM), Eq. 6's token-wise max over the ring at
    the pruning layer, then the top 20%, against the oracle (selection parity)."""
    L, W, n_buf, layers = 32768, 8, 4, 9
    ring = torch.empty(n_buf, L, dtype=torch.float32, device="cuda")
    kept = []
    for l in range(layers):
        ly = synth.gaussian_layer(600 + l, L=L, W=W, d_k=128, H_q=32, H_kv=8, n_spans=8,
                                  span_len=256, lift=2.0, fixed_span_seed=600, n_fixed=4)
        a = kvs.score_args(L=L, W=W, d_k=128, H_q=32, H_kv=8, q_pos0=ly.q_pos0,
                           heads=kvs.HEADS_ALL_SUM)
        kvs.kvs_score(kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K), a,
                      S=ring[l % n_buf:l % n_buf + 1])
        if l >= layers - n_buf:
            kept.append(oracle.score(ly.Q, ly.K, L=L, W=W, d_k=128, H_q=32, H_kv=8,
                                     q_pos0=ly.q_pos0, heads=oracle.HEADS_ALL_SUM))
    acc = torch.empty(L, dtype=torch.float32, device="cuda")
    for i in range(n_buf):
        kvs.kvs_aggregate_layers(acc, ring[i:i + 1], L, kvs.RED_MAX, first_layer=(i == 0))
    budget = L // 5
    idx = kvs.kvs_topk(acc.view(1, L), L, budget)
    torch.cuda.synchronize()
    want = oracle.aggregate_layers(kept, oracle.RED_MAX)
    np.testing.assert_allclose(acc.cpu().numpy(), want, rtol=2e-3, atol=2e-3 * 1e-3 * W * 32 / L)
    assert_topk_parity(idx.cpu().numpy(), want[None, :], budget)

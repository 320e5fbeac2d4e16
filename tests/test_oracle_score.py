"""Pins of the fp64 oracle's scoring step to facts fixed by the pages and mathematics.

Each test is chosen so that a plausible mistake fails it:
* softmax over the wrong axis / missing normalisation -> mass invariant;
* causal-mask off-by-one or rows all at one position -> identical-key closed form
  and the single-row decomposition;
* missing or wrong 1/sqrt(d_k) -> SciPy softmax special case;
* wrong query-head -> KV-head mapping -> GQA routing case;
* position-dependent bugs -> permutation and shift invariance;
* the score failing to find what the window looks for -> planted spans.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _layer(seed, L, W, d_k, H_q, H_kv):
    return synth.gaussian_layer(seed, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)


@pytest.mark.parametrize("L,W,d_k,H_q,H_kv,q_pos0", [
    (512, 16, 64, 4, 1, 496),     # Tiny shape (window at the end)
    (300, 7, 64, 6, 2, 293),      # ragged sizes
    (128, 8, 128, 8, 8, 120),     # MHA, G = 1
    (200, 5, 64, 4, 2, 250),      # lookahead queries: q_pos0 >= L, all visible
    (64, 64, 64, 2, 1, 0),        # window covers the whole prompt
])
def test_mass_equals_rows(L, W, d_k, H_q, H_kv, q_pos0):
    """Each softmax row is a distribution over keys, so a group's mass is W*G."""
    ly = _layer(11, L, W, d_k, H_q, H_kv)
    G = H_q // H_kv
    S = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0)
    assert S.shape == (H_kv, L)
    np.testing.assert_allclose(S.sum(axis=1), W * G, rtol=1e-12)
    N = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0,
                     heads=oracle.HEADS_NONE)
    np.testing.assert_allclose(N.sum(axis=1), W, rtol=1e-12)
    A = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0,
                     heads=oracle.HEADS_ALL_SUM)
    assert A.shape == (1, L)
    np.testing.assert_allclose(A.sum(), W * H_q, rtol=1e-12)   # every row of every head
    assert (S >= 0).all()


@pytest.mark.parametrize("L,W,G", [(512, 16, 4), (97, 13, 3), (40, 40, 1)])
def test_identical_keys_closed_form(L, W, G):
    """All keys equal: row j is uniform over its q_pos0 + j + 1 visible keys.

    Prefix column: G * sum_j 1/(q_pos0 + j + 1).  Window column q_pos0 + i is
    seen only by rows j >= i: G * sum_{j >= i} 1/(q_pos0 + j + 1).
    """
    d_k = 64
    q_pos0 = L - W
    ly = _layer(5, L, W, d_k, G, 1)
    K = np.repeat(ly.K[:, :1, :], L, axis=1)          # every key = key 0
    S = oracle.score(ly.Q, K, L=L, W=W, d_k=d_k, H_q=G, H_kv=1, q_pos0=q_pos0)[0]
    inv = np.array([1.0 / (q_pos0 + j + 1) for j in range(W)])
    prefix = G * inv.sum()
    np.testing.assert_allclose(S[:q_pos0], prefix, rtol=1e-12)
    for i in range(W):
        np.testing.assert_allclose(S[q_pos0 + i], G * inv[i:].sum(), rtol=1e-12)
    # the per-head maximum equals one head's value when all heads agree
    M = oracle.score(ly.Q, K, L=L, W=W, d_k=d_k, H_q=G, H_kv=1, q_pos0=q_pos0,
                     heads=oracle.HEADS_GROUP_MAX)[0]
    np.testing.assert_allclose(M, S / G, rtol=1e-12)
    # two KV heads with identical keys: the sum over every head of the layer
    # doubles the one-group closed form
    K2 = np.concatenate([K, K], axis=0)
    Q2 = np.concatenate([ly.Q, ly.Q[::-1]], axis=0)
    A = oracle.score(Q2, K2, L=L, W=W, d_k=d_k, H_q=2 * G, H_kv=2, q_pos0=q_pos0,
                     heads=oracle.HEADS_ALL_SUM)[0]
    np.testing.assert_allclose(A[:q_pos0], 2 * prefix, rtol=1e-12)
    for i in range(W):
        np.testing.assert_allclose(A[q_pos0 + i], 2 * G * inv[i:].sum(), rtol=1e-12)


@pytest.mark.parametrize("d_k", [64, 128])
def test_single_query_is_scipy_softmax(d_k):
    """W = G = 1 with every key visible reduces to softmax(q K^T / sqrt(d_k))."""
    L = 257
    ly = _layer(3, L, 1, d_k, 1, 1)
    S = oracle.score(ly.Q, ly.K, L=L, W=1, d_k=d_k, H_q=1, H_kv=1, q_pos0=L - 1)[0]
    q = synth.bf16_to_f32(ly.Q).astype(np.float64).reshape(d_k)
    k = synth.bf16_to_f32(ly.K).astype(np.float64).reshape(L, d_k)
    ref = scipy.special.softmax(k @ q / math.sqrt(d_k))
    np.testing.assert_allclose(S, ref, rtol=1e-12)
    # an explicit scale is honoured
    S2 = oracle.score(ly.Q, ly.K, L=L, W=1, d_k=d_k, H_q=1, H_kv=1, q_pos0=L - 1, scale=0.25)[0]
    np.testing.assert_allclose(S2, scipy.special.softmax(0.25 * (k @ q)), rtol=1e-12)


def test_gqa_routing():
    """Query head h must read KV head h // G: a strong key at column 10*g of KV
    head g, aligned with the queries of heads gG..gG+G-1 only."""
    L, W, d_k, H_q, H_kv = 64, 4, 64, 8, 4
    G = H_q // H_kv
    K = np.zeros((H_kv, L, d_k), dtype=np.float32)
    Q = np.zeros((H_q, W, d_k), dtype=np.float32)
    for g in range(H_kv):
        K[g, 10 * g, g] = 16.0               # key 10g of KV head g points along axis g
    for h in range(H_q):
        Q[h, :, h // G] = 16.0               # queries of group g point along axis g
    S = oracle.score(synth.to_bf16(Q), synth.to_bf16(K), L=L, W=W, d_k=d_k, H_q=H_q,
                     H_kv=H_kv, q_pos0=L - W, heads=oracle.HEADS_NONE)
    for h in range(H_q):
        assert int(np.argmax(S[h])) == 10 * (h // G)
        assert S[h, 10 * (h // G)] > 0.99 * W
    # group sum adds the heads of each group
    GS = oracle.score(synth.to_bf16(Q), synth.to_bf16(K), L=L, W=W, d_k=d_k, H_q=H_q,
                      H_kv=H_kv, q_pos0=L - W)
    np.testing.assert_allclose(GS, S.reshape(H_kv, G, L).sum(axis=1), rtol=1e-12)


def test_rows_decompose_by_position():
    """The W-row score is the sum of single-row scores at positions q_pos0 + j."""
    L, W, d_k = 150, 9, 64
    q_pos0 = 140
    ly = _layer(8, L, W, d_k, 2, 1)
    S = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=2, H_kv=1, q_pos0=q_pos0)
    acc = np.zeros_like(S)
    for j in range(W):
        acc += oracle.score(ly.Q[:, j:j + 1], ly.K, L=L, W=1, d_k=d_k, H_q=2, H_kv=1,
                            q_pos0=q_pos0 + j)
    np.testing.assert_allclose(S, acc, rtol=1e-12, atol=1e-15)


def test_prefix_permutation_and_shift_invariance():
    """Permuting keys seen by every row permutes their scores; adding one vector
    to every key leaves all scores unchanged (small integers keep bf16 exact)."""
    L, W, d_k = 80, 6, 64
    q_pos0 = L - W
    rng = np.random.default_rng(0)          # test-local integers, not method arithmetic
    Qf = rng.integers(-2, 3, size=(2, W, d_k)).astype(np.float32)
    Kf = rng.integers(-2, 3, size=(1, L, d_k)).astype(np.float32)
    Q, K = synth.to_bf16(Qf), synth.to_bf16(Kf)
    S = oracle.score(Q, K, L=L, W=W, d_k=d_k, H_q=2, H_kv=1, q_pos0=q_pos0)[0]
    perm = np.concatenate([rng.permutation(q_pos0), np.arange(q_pos0, L)])
    Sp = oracle.score(Q, K[:, perm], L=L, W=W, d_k=d_k, H_q=2, H_kv=1, q_pos0=q_pos0)[0]
    np.testing.assert_allclose(Sp, S[perm], rtol=1e-12)
    w = rng.integers(-3, 4, size=(d_k,)).astype(np.float32)
    Ks = synth.to_bf16(Kf + w[None, None, :])
    Ss = oracle.score(Q, Ks, L=L, W=W, d_k=d_k, H_q=2, H_kv=1, q_pos0=q_pos0)[0]
    np.testing.assert_allclose(Ss, S, rtol=1e-10)


def test_causal_rows_ignore_later_keys():
    """Changing a key after row j's position does not change row j's attention."""
    L, W, d_k = 60, 8, 64
    ly = _layer(21, L, W, d_k, 1, 1)
    q_pos0 = L - W
    A = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=1, H_kv=1, q_pos0=q_pos0, per_row=True)[0]
    K2 = ly.K.copy()
    K2[0, q_pos0 + 3:] = synth.to_bf16(np.full((L - q_pos0 - 3, d_k), 3.0, dtype=np.float32))
    A2 = oracle.score(ly.Q, K2, L=L, W=W, d_k=d_k, H_q=1, H_kv=1, q_pos0=q_pos0, per_row=True)[0]
    np.testing.assert_allclose(A2[:3], A[:3], rtol=1e-12)
    assert np.all(A[:, :][np.arange(L)[None, :] > (q_pos0 + np.arange(W))[:, None]] == 0)


def test_planted_spans_rank_first():
    """Keys sharing a direction with the window queries take the top ranks."""
    ly = synth.llama_layer(L=4096, seed=1, n_spans=4, span_len=64)
    S = oracle.score(ly.Q, ly.K, L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                     q_pos0=ly.q_pos0)
    n = ly.L - ly.W
    in_span = np.zeros(n, dtype=bool)
    for a, b in ly.spans:
        in_span[a:b] = True
    budget = int(in_span.sum())
    idx = oracle.topk(S[:, :n], budget)
    frac = in_span[idx].mean()
    assert frac > 0.9, frac
    # and a span token out-scores an unplanted token on average by a wide margin
    assert S[:, :n][:, in_span].mean() > 4 * S[:, :n][:, ~in_span].mean()


def test_brute_force_tiny():
    """Pure-Python loops on a tiny case agree with the vectorised definition."""
    L, W, d_k, H_q, H_kv = 11, 3, 64, 4, 2
    ly = _layer(2, L, W, d_k, H_q, H_kv)
    q = synth.bf16_to_f32(ly.Q).astype(np.float64)
    k = synth.bf16_to_f32(ly.K).astype(np.float64)
    q_pos0 = 9
    G = H_q // H_kv
    out = [[0.0] * L for _ in range(H_kv)]
    for h in range(H_q):
        for j in range(W):
            vis = [t for t in range(L) if t <= q_pos0 + j]
            logits = {t: sum(q[h, j, c] * k[h // G, t, c] for c in range(d_k)) / math.sqrt(d_k) for t in vis}
            m = max(logits.values())
            z = sum(math.exp(v - m) for v in logits.values())
            for t in vis:
                out[h // G][t] += math.exp(logits[t] - m) / z
    S = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0)
    np.testing.assert_allclose(S, np.array(out), rtol=1e-12)
    A = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0,
                     heads=oracle.HEADS_ALL_SUM)
    every = [sum(out[g][t] for g in range(H_kv)) for t in range(L)]
    np.testing.assert_allclose(A[0], np.array(every), rtol=1e-12)

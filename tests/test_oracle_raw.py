"""Pins of the oracle's raw (pre-softmax) scoring and its Speculative-Prefill aggregation.

Each test is chosen so that a plausible mistake fails it:
* wrong query-head -> KV-head mapping -> one-hot GQA closed form;
* a dropped head, a sum taken as a max or the reverse -> integer closed forms and
  the linearity identity;
* a missing or wrong default scale -> the 1/sqrt(d_k) check;
* max over layers and mean over queries applied in the wrong order -> the
  hand-worked aggregation case, where the two orders differ;
* anything else -> brute-force loops on a tiny case.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _bits(x):
    return synth.to_bf16(np.asarray(x, dtype=np.float32))


def test_sum_is_linear_in_the_queries():
    """Sum over heads of q_h . k_g(h) equals (sum of a group's queries) . k_g, summed over groups."""
    H_q, H_kv, W, L, d_k = 8, 2, 3, 50, 64
    ly = synth.gaussian_layer(21, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L)
    R = oracle.score_raw(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, reduce=oracle.RED_SUM)
    q = oracle.bf16_to_f64(ly.Q).reshape(H_q, W, d_k)
    k = oracle.bf16_to_f64(ly.K).reshape(H_kv, L, d_k)
    G = H_q // H_kv
    want = sum(q[g * G:(g + 1) * G].sum(axis=0) @ k[g].T for g in range(H_kv)) / math.sqrt(d_k)
    np.testing.assert_allclose(R, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("H_q,H_kv", [(8, 4), (6, 3), (4, 4)])
def test_one_hot_gqa_closed_form(H_q, H_kv):
    """q[h][j] = (j+1) e_{h // G}, k[g][t] = c[g][t] e_g: only the own KV head contributes.

    SUM = G (j+1) sum_g c[g][t]; MAX = (j+1) max_g c[g][t] with c[g][t] = 1 + (g*5 + t) % 7.
    A head read against the wrong KV head would see a zero logit."""
    G = H_q // H_kv
    W, L, d_k = 3, 11, 16
    q = np.zeros((H_q, W, d_k))
    for h in range(H_q):
        for j in range(W):
            q[h, j, h // G] = j + 1
    c = np.array([[1 + (g * 5 + t) % 7 for t in range(L)] for g in range(H_kv)], dtype=np.float64)
    k = np.zeros((H_kv, L, d_k))
    for g in range(H_kv):
        k[g, :, g] = c[g]
    Q, K = _bits(q), _bits(k)
    j1 = np.arange(1, W + 1)[:, None]
    S = oracle.score_raw(Q, K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, reduce=oracle.RED_SUM, scale=1.0)
    np.testing.assert_array_equal(S, G * j1 * c.sum(axis=0)[None, :])
    M = oracle.score_raw(Q, K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, reduce=oracle.RED_MAX, scale=1.0)
    np.testing.assert_array_equal(M, j1 * c.max(axis=0)[None, :])


def test_integer_sum_and_max_over_heads():
    """q[h][j] = (h+1)(j+1) (1,1,1,1), k[0][t] = (t+1) e_{t mod 4}: logit (h+1)(j+1)(t+1).

    SUM over H_q heads = (j+1)(t+1) H_q (H_q+1) / 2; MAX = (j+1)(t+1) H_q."""
    H_q, W, L, d_k = 5, 2, 9, 4
    q = np.array([[[(h + 1) * (j + 1)] * 4 for j in range(W)] for h in range(H_q)], dtype=np.float64)
    k = np.zeros((1, L, d_k))
    for t in range(L):
        k[0, t, t % 4] = t + 1
    Q, K = _bits(q), _bits(k)
    jt = np.outer(np.arange(1, W + 1), np.arange(1, L + 1)).astype(np.float64)
    S = oracle.score_raw(Q, K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=1, reduce=oracle.RED_SUM, scale=1.0)
    np.testing.assert_array_equal(S, jt * H_q * (H_q + 1) / 2)
    M = oracle.score_raw(Q, K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=1, reduce=oracle.RED_MAX, scale=1.0)
    np.testing.assert_array_equal(M, jt * H_q)


def test_default_scale_is_inverse_sqrt_dk():
    """GemFilter divides the raw logit by sqrt(d_k), the standard attention scale; d_k = 64 -> 1/8."""
    q = np.zeros((1, 1, 64))
    q[0, 0, 0] = 3.0
    k = np.zeros((1, 2, 64))
    k[0, 0, 0] = 2.0
    k[0, 1, 0] = -4.0
    S = oracle.score_raw(_bits(q), _bits(k), L=2, W=1, d_k=64, H_q=1, H_kv=1)
    np.testing.assert_array_equal(S, [[6.0 / 8.0, -12.0 / 8.0]])


@pytest.mark.parametrize("reduce", [1, 2])
def test_brute_force_tiny(reduce):
    """Pure-Python loops over heads, rows, keys and channels on a tiny GQA case."""
    H_q, H_kv, W, L, d_k = 4, 2, 3, 6, 5
    G = H_q // H_kv
    rng = np.random.default_rng(7)
    Q = _bits(rng.standard_normal((H_q, W, d_k)))
    K = _bits(rng.standard_normal((H_kv, L, d_k)))
    q = oracle.bf16_to_f64(Q).reshape(H_q, W, d_k).tolist()
    k = oracle.bf16_to_f64(K).reshape(H_kv, L, d_k).tolist()
    scale = 0.37
    want = [[None] * L for _ in range(W)]
    for j in range(W):
        for t in range(L):
            acc = None
            for h in range(H_q):
                v = 0.0
                for c in range(d_k):
                    v += q[h][j][c] * k[h // G][t][c]
                v *= scale
                acc = v if acc is None else (acc + v if reduce == 1 else max(acc, v))
            want[j][t] = acc
    got = oracle.score_raw(Q, K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, reduce=reduce, scale=scale)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-14)


def test_aggregate_max_over_layers_before_mean_over_queries():
    """Worked by hand.  Layers A = [[4,0,1],[0,0,1]], B = [[0,0,1],[4,0,1]] (rows = queries).

    Max over layers: [[4,0,1],[4,0,1]]; mean over queries: [4, 0, 1]; average
    pooling k = 3 clipped to the row: [(4+0)/2, (4+0+1)/3, (0+1)/2] = [2, 5/3, 1/2].
    Averaging over queries first would give [2, 0, 1] and then [1, 1, 1/2]."""
    A = np.array([[4.0, 0, 1], [0, 0, 1]])
    B = np.array([[0.0, 0, 1], [4, 0, 1]])
    np.testing.assert_allclose(oracle.aggregate_raw([A, B], pool_k=0), [4.0, 0.0, 1.0], rtol=0)
    np.testing.assert_allclose(oracle.aggregate_raw([A, B], pool_k=3), [2.0, 5.0 / 3.0, 0.5],
                               rtol=1e-15)


def test_head_reduce_mean_worked_example():
    """Mean over rows: [[1, 2], [3, 6], [5, 1]] -> [3, 3]."""
    x = np.array([[1.0, 2.0], [3.0, 6.0], [5.0, 1.0]])
    np.testing.assert_array_equal(oracle.head_reduce(x, oracle.RED_MEAN), [[3.0, 3.0]])


def test_last_token_raw_score_finds_planted_spans():
    """GemFilter on a layer whose last-token query shares each KV head's planted direction:
    the 2% best tokens by the summed raw logit are mostly planted ones."""
    L, d_k, H_q, H_kv = 4096, 128, 8, 2
    ly = synth.gaussian_layer(31, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1,
                              n_spans=4, span_len=64, lift=2.0, span_region=L - 1)
    R = oracle.score_raw(ly.Q, ly.K, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv)[0]
    planted = np.zeros(L, dtype=bool)
    for a, b in ly.spans:
        planted[a:b] = True
    top = np.argsort(-R, kind="stable")[: planted.sum()]
    assert planted[top].mean() > 0.9

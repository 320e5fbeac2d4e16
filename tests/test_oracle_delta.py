"""Pins of the oracle's DELTA page selection (max over heads -> page sums ->
recent pages + top older pages).

Each test is chosen so that a plausible mistake fails it:
* mean instead of max over heads -> the one-sharp-head case;
* pages cut at the wrong boundary or the partial last page mishandled -> the
  identical-key closed form;
* recency pages dropped or taken from the wrong end -> the zero-score recency case;
* anything else -> brute-force loops on a tiny case.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _bits(x):
    return synth.to_bf16(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("L,P,K,Lr", [(300, 16, 8, 2), (1000, 16, 64, 8), (37, 16, 64, 8), (5, 4, 3, 1)])
def test_identical_keys_closed_form(L, P, K, Lr):
    """Identical keys: every head attends uniformly, s_t = 1/L, a full page scores P/L and the
    partial last page (L mod P)/L; ties go to the lower page index."""
    H_q, H_kv, d_k = 4, 2, 64
    ly = synth.gaussian_layer(3, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1)
    Kb = np.repeat(ly.K[:, :1, :], L, axis=1)
    rho, z = oracle.delta_pages(ly.Q[:, 0, :], Kb, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P,
                                K_pages=K, L_recent=Lr)
    n_pages = math.ceil(L / P)
    want_z = np.full(n_pages, P / L)
    if L % P:
        want_z[-1] = (L % P) / L
    np.testing.assert_allclose(z, want_z, rtol=1e-12)
    n_recent = min(Lr, n_pages)
    n_cand = n_pages - n_recent
    keep = min(K - Lr, n_cand)
    want = list(range(keep)) + list(range(n_cand, n_pages))
    assert list(rho[:len(want)]) == want
    assert (rho[len(want):] == -1).all()


def test_one_sharp_head_wins_by_max():
    """Head 0 puts almost all its mass on token 40 (page 2); heads 1-3 spread over pages 5-6.
    The max over heads keeps page 2 on top; a mean over heads would rank it below them."""
    H_q, H_kv, d_k, L, P = 4, 1, 16, 128, 16
    q = np.zeros((H_q, d_k))
    k = np.zeros((1, L, d_k))
    q[0, 0] = 8.0                      # head 0: logit 8*8/4 = 16 at token 40, 0 elsewhere
    k[0, 40, 0] = 8.0
    for h in range(1, H_q):            # heads 1-3: logit 2 on tokens 80..111
        q[h, 1] = 4.0
    k[0, 80:112, 1] = 2.0
    rho, z = oracle.delta_pages(_bits(q), _bits(k), L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P,
                                K_pages=2, L_recent=0)
    assert z[2] > 0.99 and z[2] == z.max()
    assert list(rho) == [2, 5] or list(rho) == [2, 6]
    # a mean over heads would give page 2 about 1/4 and pages 5-6 about 0.37 each
    assert z[2] > z[5] and z[2] > z[6]


def test_recent_pages_are_kept_with_zero_score():
    """The last L pages enter rho even when every key there is invisible to the query's focus."""
    H_q, H_kv, d_k, L, P = 2, 1, 8, 160, 16
    q = np.zeros((H_q, d_k))
    q[:, 0] = 8.0
    k = np.zeros((1, L, d_k))
    k[0, 0:16, 0] = 4.0                # page 0 holds nearly all the mass
    k[0, 128:160, 0] = -8.0            # pages 8, 9 (the recent ones) hold almost none
    rho, z = oracle.delta_pages(_bits(q), _bits(k), L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P,
                                K_pages=4, L_recent=2)
    assert z[8] < 1e-6 and z[9] < 1e-6
    assert list(rho[2:]) == [8, 9]
    assert rho[0] == 0


def test_brute_force_tiny():
    """Pure-Python softmax per head, max over heads, page sums and an explicit ranking."""
    H_q, H_kv, d_k, L, P, K, Lr = 4, 2, 5, 23, 4, 4, 1
    G = H_q // H_kv
    rng = np.random.default_rng(11)
    Q = _bits(rng.standard_normal((H_q, d_k)))
    Kb = _bits(rng.standard_normal((H_kv, L, d_k)))
    q = oracle.bf16_to_f64(Q).reshape(H_q, d_k).tolist()
    k = oracle.bf16_to_f64(Kb).reshape(H_kv, L, d_k).tolist()
    scale = 1.0 / math.sqrt(d_k)
    s = [0.0] * L
    for h in range(H_q):
        logits = [scale * sum(q[h][c] * k[h // G][t][c] for c in range(d_k)) for t in range(L)]
        m = max(logits)
        e = [math.exp(x - m) for x in logits]
        Z = sum(e)
        for t in range(L):
            s[t] = max(s[t], e[t] / Z)
    n_pages = (L + P - 1) // P
    z = [sum(s[u * P:min(u * P + P, L)]) for u in range(n_pages)]
    n_cand = n_pages - Lr
    order = sorted(range(n_cand), key=lambda u: (-z[u], u))
    want = sorted(order[:K - Lr]) + list(range(n_cand, n_pages))
    rho, zz = oracle.delta_pages(Q, Kb, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P, K_pages=K, L_recent=Lr)
    np.testing.assert_allclose(zz, z, rtol=1e-12)
    assert list(rho) == want

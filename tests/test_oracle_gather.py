"""Pins of the oracle's KV gather (a copy, so pinned by construction).

Every element of X carries a code of its (head, token, channel), so a gathered
row names the token it came from: a wrong head, token, unit offset or list
stride fails exactly.  Negative entries, tokens past L and rows past a head's
list must be zero.
"""
import numpy as np

import oracle


def _coded(H, L, d):
    g, t, c = np.meshgrid(np.arange(H), np.arange(L), np.arange(d), indexing="ij")
    return ((g * 7919 + t * 31 + c * 3 + 1) % 65521).astype(np.uint16)


def test_per_head_tokens():
    H, L, d = 3, 50, 8
    X = _coded(H, L, d)
    idx = np.array([[0, 7, 49, -1], [3, 3, 10, 60], [1, 2, 3, 4]], dtype=np.int32)
    out = oracle.gather_kv(X, L=L, indices=idx, n=4, idx_ld=4)
    for g in range(H):
        for r in range(4):
            i = idx[g, r]
            want = X[g, i] if 0 <= i < L else np.zeros(d, np.uint16)
            assert np.array_equal(out[g, r], want), (g, r)


def test_shared_list_pages_with_partial_last_page():
    """unit = 16 (pages): page 3 of a 60-token row holds tokens 48..59, then 4 zero rows."""
    H, L, d = 2, 60, 4
    X = _coded(H, L, d)
    out = oracle.gather_kv(X, L=L, indices=np.array([3, 0, -1], np.int32), n=3, unit=16)
    assert out.shape == (H, 48, d)
    for g in range(H):
        assert np.array_equal(out[g, 0:12], X[g, 48:60])
        assert not out[g, 12:16].any()
        assert np.array_equal(out[g, 16:32], X[g, 0:16])
        assert not out[g, 32:48].any()


def test_csr_lists():
    """CSR lists of different lengths: head 0 two blocks, head 1 none, head 2 one (capped at n)."""
    H, L, d = 3, 40, 4
    X = _coded(H, L, d)
    indptr = np.array([0, 2, 2, 5], np.int32)
    indices = np.array([4, 1, 0, 2, 3], np.int32)
    out = oracle.gather_kv(X, L=L, indices=indices, n=2, unit=8, indptr=indptr)
    assert np.array_equal(out[0, 0:8], X[0, 32:40]) and np.array_equal(out[0, 8:16], X[0, 8:16])
    assert not out[1].any()
    assert np.array_equal(out[2, 0:8], X[2, 0:8]) and np.array_equal(out[2, 8:16], X[2, 16:24])

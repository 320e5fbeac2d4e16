"""Pin (viii): two independent fp64 oracles of the window score agree.

The NumPy oracle (oracle/kvs.py: one matrix product per head, masked softmax
over the key axis, sums along axes) and a plain C one (oracle/score_ref.c:
scalar loops, one row at a time) are written separately; they must agree to
1e-12 relative on every head mode and on shapes with causal windows, lookahead
queries, GQA groups and ragged sizes.  A transposed operand, a wrong head
mapping or an off-by-one mask in either fails here."""
import ctypes
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import build_ref


@pytest.fixture(scope="module")
def ref():
    return build_ref.load()


def _ref_score(ref, ly, q_pos0, heads):
    rows = {0: ly.H_q, 3: 1}.get(heads, ly.H_kv)
    out = np.empty((rows, ly.L), dtype=np.float64)
    Q = np.ascontiguousarray(ly.Q)
    K = np.ascontiguousarray(ly.K)
    st = ref.kvs_ref_score(Q.ctypes.data, K.ctypes.data, ly.L, ly.W, ly.d_k, ly.H_q, ly.H_kv,
                           q_pos0, heads, 1.0 / math.sqrt(ly.d_k), out.ctypes.data)
    assert st == 0
    return out


@pytest.mark.parametrize("L,W,d_k,H_q,H_kv,off", [(300, 16, 64, 4, 1, 0), (257, 7, 128, 6, 2, 0),
                                                  (200, 5, 64, 8, 4, 30), (64, 64, 64, 2, 1, 0),
                                                  (1, 1, 64, 2, 1, 0)])
@pytest.mark.parametrize("heads", [0, 1, 2, 3])
def test_two_fp64_oracles_agree(ref, L, W, d_k, H_q, H_kv, off, heads):
    ly = synth.gaussian_layer(900 + L, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, n_spans=0)
    q_pos0 = max(L - W, 0) + off
    got = _ref_score(ref, ly, q_pos0, heads)
    want = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0,
                        heads=heads)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)

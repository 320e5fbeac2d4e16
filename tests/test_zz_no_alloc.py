"""kvs_score_noalloc: kvs_score with the library's static per-GPU scratch in place of
a caller workspace.  Through the C ABI, two calls in a row (the second on a
smaller input) must equal kvs_score with a caller workspace bit for bit, the split
phase-1 / phase-2 calls must equal one call, and a call needing more than the
static scratch is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _inputs(kvs, seed, L, W, d_k, H_q, H_kv):
    ly = synth.gaussian_layer(seed, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, n_spans=4,
                              span_len=64, lift=2.0)
    return ly, kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K)


def _noalloc(kvs, Q, K, a, S):
    st = kvs.library().kvs_score_noalloc(ctypes.byref(a), ctypes.c_void_p(Q.data_ptr()),
                                         ctypes.c_void_p(K.data_ptr()),
                                         ctypes.c_void_p(S.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kvs.library().kvs_status_string(st)


@pytest.mark.parametrize("heads", [1, 0, 2], ids=["group_sum", "none", "group_max"])
def test_noalloc_matches_workspace_call_twice(kvs, heads):
    shapes = [(6001, 32, 128, 32, 8), (1000, 16, 64, 8, 2)]   # second call: a smaller input
    for i, (L, W, d_k, H_q, H_kv) in enumerate(shapes):
        print(f"noalloc call {i} L={L} heads={heads}", flush=True)
        ly, Q, K = _inputs(kvs, 70 + i, L, W, d_k, H_q, H_kv)
        a = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, heads=heads)
        want = kvs.kvs_score(Q, K, a)
        got = torch.full_like(want, float("nan"))
        _noalloc(kvs, Q, K, a, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))


def test_noalloc_phase_split_and_all_heads(kvs):
    L, W, d_k, H_q, H_kv = 4113, 32, 128, 64, 8           # two row groups
    ly, Q, K = _inputs(kvs, 90, L, W, d_k, H_q, H_kv)
    shape = dict(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0)
    want = kvs.kvs_score(Q, K, kvs.score_args(**shape))
    got = torch.full_like(want, float("nan"))
    _noalloc(kvs, Q, K, kvs.score_args(**shape, phase=1), got)
    _noalloc(kvs, Q, K, kvs.score_args(**shape, phase=2), got)
    a = kvs.score_args(**shape, heads=kvs.HEADS_ALL_SUM)
    all_want = kvs.kvs_score(Q, K, a)
    all_got = torch.full_like(all_want, float("nan"))
    _noalloc(kvs, Q, K, a, all_got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    assert torch.equal(all_got.view(torch.int32), all_want.view(torch.int32))


def test_noalloc_refuses_beyond_scratch(kvs):
    """ALL_SUM at 1M tokens with 8 KV heads needs 32 MiB of per-head rows: refused
    with KVS_ESCRATCH before any pointer is used."""
    a = kvs.score_args(L=1 << 20, W=32, d_k=128, H_q=32, H_kv=8, q_pos0=(1 << 20) - 32,
                       heads=kvs.HEADS_ALL_SUM)
    assert kvs.kvs_score_workspace(a) > 8 << 20
    P = ctypes.c_void_p
    assert kvs.library().kvs_score_noalloc(ctypes.byref(a), P(16), P(16), P(16), None) == -5
    assert kvs.library().kvs_score_noalloc(None, P(16), P(16), P(16), None) == -1

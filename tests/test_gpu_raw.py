"""GPU parity of kvs_score_raw (raw pre-softmax logits reduced over all heads)
against the fp64 oracle, and of the GemFilter / Speculative-Prefill selection
chains built on it.

Tolerance, from the arithmetic: each logit is a 32x32x16 MFMA sum of exact
bf16 products in fp32 (d_k terms), scaled in fp32, and the reduction over
heads adds at most H_q more fp32 roundings.  The error is therefore below
(d_k + H_q + 2) * 2^-24 * A, where A = sum over heads of scale * |q| . |k| (the
same score on absolute values).  The test allows 2^-16 * A + 1e-30, a factor
above that bound for every shape here.  MAX picks one head's value, whose error
is below the same bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_topk_parity

pytestmark = pytest.mark.gpu

RAW_REL = 2.0 ** -16


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _abs_bits(bits):
    return (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


def _oracle(ly, reduce, scale=None, Q=None, K=None, L=None):
    Q = ly.Q if Q is None else Q
    K = ly.K if K is None else K
    L = ly.L if L is None else L
    kw = dict(L=L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv, scale=scale)
    want = oracle.score_raw(Q, K, reduce=reduce, **kw)
    bound = oracle.score_raw(_abs_bits(Q), _abs_bits(K), reduce=oracle.RED_SUM, **kw)
    return want, bound


def _assert_raw_close(got, want, bound, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    tol = RAW_REL * bound + 1e-30
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} out of tolerance; worst at {i}: "
                             f"got {got[i]:.9g} want {want[i]:.9g} tol {tol[i]:.3g}")


def _run(kvs, ly, reduce, q_pos0=None, S=None, **kw):
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    a = kvs.raw_args(L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                     q_pos0=ly.L if q_pos0 is None else q_pos0, reduce=reduce, **kw)
    out = kvs.kvs_score_raw(Q, K, a, S=S)
    torch.cuda.synchronize()
    return out


CASES = [
    # (name, L, W, d_k, H_q, H_kv): several tiles and splits, ragged tails
    ("gemfilter_ragged", 1000, 1, 128, 8, 2),
    ("gqa_w8", 4113, 8, 128, 32, 8),
    ("ragged64", 777, 8, 64, 8, 2),
    ("g2_w3", 300, 3, 128, 6, 3),
    ("g8_w16", 2048, 16, 128, 8, 1),            # 4 row tiles per KV head
    ("mha_w32", 513, 32, 64, 4, 4),
    ("g3_w5", 1234, 5, 128, 12, 4),             # padding rows inside the row tile
    ("d64_many_heads", 3001, 8, 64, 56, 14),    # 14 KV heads of rows in LDS
    ("one_key", 1, 1, 128, 4, 1),
    ("sub_tile", 31, 4, 64, 4, 2),
    ("tile_plus_one", 33, 2, 128, 8, 8),
]


@pytest.mark.parametrize("name,L,W,d_k,H_q,H_kv", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("reduce", [1, 2], ids=["sum", "max"])
def test_raw_parity(kvs, name, L, W, d_k, H_q, H_kv, reduce):
    print(f"raw case {name} reduce={reduce}", flush=True)
    ly = synth.gaussian_layer(300 + L, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L)
    got = _run(kvs, ly, reduce).cpu().numpy()
    want, bound = _oracle(ly, reduce)
    _assert_raw_close(got, want, bound, name)


@pytest.mark.parametrize("acc", [0, 1, 2], ids=["write", "add", "max"])
def test_raw_accumulate_strides_and_last_token(kvs, acc):
    """Sequence-major K, strided Q and S, q_pos0 = L - 1 (GemFilter's last prompt
    token), and the three ways of combining with S."""
    L, W, d_k, H_q, H_kv = 2500, 4, 128, 8, 2
    print(f"raw accumulate {acc}", flush=True)
    ly = synth.gaussian_layer(77, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1)
    K_seq = np.ascontiguousarray(ly.K.transpose(1, 0, 2))          # [L][H_kv][d_k]
    Qpad = np.zeros((H_q, W + 3, d_k + 8), dtype=np.uint16)
    Qpad[:, :W, :d_k] = ly.Q
    s_ld = L + 37
    prior = synth.score_array(5, W, s_ld, signed=True) * 50.0
    S = torch.from_numpy(prior).cuda()
    Q = kvs.bf16_from_bits(Qpad)
    K = kvs.bf16_from_bits(K_seq)
    a = kvs.raw_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1, reduce=kvs.RED_MAX,
                     accumulate=acc, q_head_stride=(W + 3) * (d_k + 8), q_row_stride=d_k + 8,
                     k_head_stride=d_k, k_tok_stride=H_kv * d_k, s_ld=s_ld)
    kvs.kvs_score_raw(Q, K, a, S=S)
    torch.cuda.synchronize()
    got = S.cpu().numpy().astype(np.float64)
    want, bound = _oracle(ly, oracle.RED_MAX)
    p = prior[:, :L].astype(np.float64)
    if acc == 1:
        want = p + want
        bound = bound + np.abs(p) * 2.0 ** -6     # one more fp32 rounding: |p| 2^-22 after scaling
    elif acc == 2:
        want = np.maximum(p, want)
    _assert_raw_close(got[:, :L], want, bound, f"acc={acc}")
    np.testing.assert_array_equal(got[:, L:], prior[:, L:])      # columns past L untouched


def test_raw_deterministic(kvs):
    ly = synth.gaussian_layer(9, L=8192, W=8, d_k=128, H_q=32, H_kv=8, q_pos0=8192)
    a = _run(kvs, ly, 1).cpu().numpy()
    b = _run(kvs, ly, 1).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.slow
@pytest.mark.parametrize("W,reduce", [(1, 1), (8, 2)], ids=["gemfilter", "specprefill"])
def test_raw_full_size(kvs, W, reduce):
    """Mistral-7B GQA layer at L = 131072 in the launch configuration the bench
    uses, every key column against the oracle."""
    L = 131072
    print(f"raw full size W={W}", flush=True)
    ly = synth.gaussian_layer(5 + W, L=L, W=W, d_k=128, H_q=32, H_kv=8, q_pos0=L - 1,
                              n_spans=16, span_len=512, lift=2.0, span_region=L - 1)
    got = _run(kvs, ly, reduce, q_pos0=L - 1).cpu().numpy()
    want, bound = _oracle(ly, reduce)
    _assert_raw_close(got[:, :L], want, bound, "every column")
    assert np.isfinite(got).all()


def test_gemfilter_selection_chain(kvs):
    """GemFilter: last-token raw logits summed over heads -> average pool 7 ->
    top 20% + nothing forced, against the oracle's chain (selection parity)."""
    L, W = 16384, 1
    ly = synth.gaussian_layer(41, L=L, W=W, d_k=128, H_q=32, H_kv=8, q_pos0=L - 1,
                              n_spans=8, span_len=256, lift=2.0, span_region=L - 1)
    R = _run(kvs, ly, kvs.RED_SUM, q_pos0=L - 1)
    pooled, _, _ = kvs.kvs_pool_pages(R, L, pool=kvs.RED_MEAN, pool_k=7)
    budget = L // 5
    idx = kvs.kvs_topk(pooled, L, budget)
    torch.cuda.synchronize()
    want = oracle.pool(oracle.score_raw(ly.Q, ly.K, L=L, W=W, d_k=128, H_q=32, H_kv=8),
                       oracle.RED_MEAN, 7)
    assert_topk_parity(idx.cpu().numpy(), want, budget)


def test_specprefill_selection_chain(kvs):
    """Speculative Prefill / answer oracle over 4 layers and 8 lookahead queries:
    per layer raw max over heads (S = R, then S = max(S, R)), mean over the
    queries and average pool 7 in one kvs_pool_pages call, top 10%."""
    L, W, layers = 16384, 8, 4
    S = None
    per_layer = []
    for l in range(layers):
        ly = synth.gaussian_layer(50 + l, L=L, W=W, d_k=128, H_q=32, H_kv=8, q_pos0=L,
                                  n_spans=8, span_len=256, lift=2.0, span_region=L,
                                  fixed_span_seed=50, n_fixed=4)
        S = _run(kvs, ly, kvs.RED_MAX, S=S, accumulate=kvs.ACC_WRITE if l == 0 else kvs.ACC_MAX)
        per_layer.append(oracle.score_raw(ly.Q, ly.K, L=L, W=W, d_k=128, H_q=32, H_kv=8,
                                          reduce=oracle.RED_MAX))
    pooled, _, _ = kvs.kvs_pool_pages(S, L, head_reduce=kvs.RED_MEAN, pool=kvs.RED_MEAN, pool_k=7)
    budget = L // 10
    idx = kvs.kvs_topk(pooled, L, budget)
    torch.cuda.synchronize()
    want = oracle.aggregate_raw(per_layer, pool_k=7)
    np.testing.assert_allclose(pooled.cpu().numpy()[0], want, rtol=1e-4, atol=1e-4)
    assert_topk_parity(idx.cpu().numpy(), want[None, :], budget)

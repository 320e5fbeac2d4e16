"""GPU parity of kvs_delta_pages (DELTA decode-time page sets, batched) against
the fp64 oracle.

Page scores: |gpu - oracle| <= 1e-4 |oracle| + 1e-9 (fp32 logits from bf16
products, exp2 and sums of at most P probabilities against fp64).  Page sets:
every page whose oracle score is more than 1e-4 (relative) away from the
K - L-th score must be classified the same, the recent pages and the -1
padding must match exactly, and rows are ascending within each part.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_topk_parity

pytestmark = pytest.mark.gpu

REL = 1e-4


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _run_batch(kvs, lens, H_q, H_kv, d_k, P, K_pages, L_recent, seq_major=False, seed=0,
               spans=0):
    B = len(lens)
    L_max = max(max(lens), 1)
    layers, Ks = [], []
    for b, L in enumerate(lens):
        Lg = max(L, 1)
        ns = spans if Lg >= spans * 64 * 2 and spans else 0
        ly = synth.gaussian_layer(seed * 1000 + b, L=Lg, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv,
                                  q_pos0=Lg - 1, n_spans=ns, span_len=64, lift=2.0, span_region=Lg - 1)
        layers.append(ly)
        Kb = ly.K.transpose(1, 0, 2) if seq_major else ly.K
        Ks.append(kvs.bf16_from_bits(np.ascontiguousarray(Kb)))
    Q = kvs.bf16_from_bits(np.stack([ly.Q[:, 0, :] for ly in layers]))
    ptrs = torch.tensor([k.data_ptr() for k in Ks], dtype=torch.int64, device="cuda")
    Lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kw = dict(k_head_stride=d_k, k_tok_stride=H_kv * d_k) if seq_major else {}
    a = kvs.delta_args(B=B, d_k=d_k, H_q=H_q, H_kv=H_kv, L_max=L_max, P=P, K_pages=K_pages,
                       L_recent=L_recent, **kw)
    n_pages_max = (L_max + P - 1) // P
    S = torch.full((B, n_pages_max), -7.0, dtype=torch.float32, device="cuda")
    rho = kvs.kvs_delta_pages(Q, ptrs, Lt, a, page_scores=S)
    torch.cuda.synchronize()
    return layers, rho.cpu().numpy(), S.cpu().numpy()


def _check(layers, lens, rho, S, H_q, H_kv, d_k, P, K_pages, L_recent):
    for b, L in enumerate(lens):
        row = rho[b]
        if L == 0:
            assert (row == -1).all()
            continue
        ly = layers[b]
        want_rho, z = oracle.delta_pages(ly.Q[:, 0, :], ly.K, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P,
                                         K_pages=K_pages, L_recent=L_recent)
        n_pages = len(z)
        np.testing.assert_allclose(S[b, :n_pages], z, rtol=REL, atol=1e-9)
        assert (S[b, n_pages:] == -7.0).all(), "entries past the sequence's pages were written"
        n_recent = min(L_recent, n_pages)
        n_cand = n_pages - n_recent
        keep = min(K_pages - L_recent, n_cand)
        np.testing.assert_array_equal(row[keep:keep + n_recent], np.arange(n_cand, n_pages))
        assert (row[keep + n_recent:] == -1).all()
        if keep:
            assert_topk_parity(row[None, :keep], z[None, :n_cand], keep, rel=REL)


CASES = [
    # lens, H_q, H_kv, d_k, P, K_pages, L_recent
    ([1, 15, 16, 17, 100, 1000, 5000, 0], 32, 8, 128, 16, 8, 2),   # ragged batch, empty sequence
    ([3000, 2999, 257], 8, 2, 64, 16, 64, 8),                       # fewer pages than K
    ([4100, 700], 48, 8, 128, 16, 16, 4),                           # G = 6: heads straddle row tiles
    ([2048, 4096], 64, 8, 128, 16, 64, 8),                          # two row tiles
    ([1500], 32, 1, 64, 8, 20, 3),                                  # one KV head, P = 8
    ([777, 1234], 16, 16, 128, 32, 10, 0),                          # MHA, no recent pages
    ([900, 2049], 96, 8, 64, 16, 8, 2),                             # three row tiles, G = 12
    ([1500, 700], 128, 8, 128, 16, 16, 4),                          # four row tiles, G = 16
    ([1, 15, 16, 17, 100, 1000, 2500, 0], 32, 8, 128, 16, 8, 2),   # ragged, in one launch
    ([5000, 3000], 32, 8, 64, 512, 4, 1),                           # pages longer than a chunk
    ([16512, 16528, 16496], 32, 8, 128, 16, 64, 8),   # 1 024 / 1 025 / 1 023 candidate pages:
                                                      # the one-wave selection's edge
]


@pytest.mark.parametrize("lens,H_q,H_kv,d_k,P,K_pages,L_recent", CASES)
def test_delta_parity(kvs, lens, H_q, H_kv, d_k, P, K_pages, L_recent):
    print(f"delta case lens={lens} H_q={H_q} H_kv={H_kv} d_k={d_k}", flush=True)
    layers, rho, S = _run_batch(kvs, lens, H_q, H_kv, d_k, P, K_pages, L_recent)
    _check(layers, lens, rho, S, H_q, H_kv, d_k, P, K_pages, L_recent)


def test_delta_sequence_major_and_deterministic(kvs):
    lens = [2500, 1111]
    a = _run_batch(kvs, lens, 32, 8, 128, 16, 64, 8, seq_major=True, seed=3)
    _check(a[0], lens, a[1], a[2], 32, 8, 128, 16, 64, 8)
    b = _run_batch(kvs, lens, 32, 8, 128, 16, 64, 8, seq_major=True, seed=3)
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))


@pytest.mark.parametrize("H_q,H_kv", [(32, 8), (64, 8)], ids=["one_launch", "three_kernels"])
def test_delta_tied_page_scores(kvs, H_q, H_kv):
    """Zero keys give every token of a sequence the same logit, so all of its full pages
    score the same: rho must hold the lowest-index older pages.  The sequences cover the
    one-wave selection (504 and 86 candidate pages), the workgroup one (1 242) and, with 64
    query heads, the separate selection kernel; the page scores still match the oracle."""
    lens, d_k, P, K_pages, L_recent = [8192, 1500, 20000, 8192], 128, 16, 64, 8
    print(f"delta tied pages lens={lens} H_q={H_q}", flush=True)
    B, L_max = len(lens), max(lens)
    Qs, Ks, Kbits = [], [], []
    for b, L in enumerate(lens):
        ly = synth.gaussian_layer(700 + b, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1)
        Qs.append(ly.Q[:, 0, :])
        Kbits.append(np.zeros((H_kv, L, d_k), dtype=np.uint16))
        Ks.append(kvs.bf16_from_bits(Kbits[-1]))
    Q = kvs.bf16_from_bits(np.stack(Qs))
    ptrs = torch.tensor([k.data_ptr() for k in Ks], dtype=torch.int64, device="cuda")
    Lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    a = kvs.delta_args(B=B, d_k=d_k, H_q=H_q, H_kv=H_kv, L_max=L_max, P=P, K_pages=K_pages,
                       L_recent=L_recent)
    S = torch.full((B, (L_max + P - 1) // P), -7.0, dtype=torch.float32, device="cuda")
    rho = kvs.kvs_delta_pages(Q, ptrs, Lt, a, page_scores=S).cpu().numpy()
    S = S.cpu().numpy()
    for b, L in enumerate(lens):
        n_pages = (L + P - 1) // P
        n_recent = min(L_recent, n_pages)
        n_cand = n_pages - n_recent
        keep = min(K_pages - L_recent, n_cand)
        assert (S[b, :n_cand] == S[b, 0]).all(), "full pages of equal tokens must tie exactly"
        want = list(range(keep)) + list(range(n_cand, n_pages))
        want += [-1] * (K_pages - len(want))
        np.testing.assert_array_equal(rho[b], want)
        _, z = oracle.delta_pages(Qs[b], Kbits[b], L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P,
                                  K_pages=K_pages, L_recent=L_recent)
        np.testing.assert_allclose(S[b, :n_pages], z, rtol=REL, atol=1e-9)


@pytest.mark.parametrize("lens,H_q,H_kv,d_k,P", [
    ([3000, 17, 2600, 0, 1024], 32, 8, 128, 16),
    ([1500], 32, 1, 64, 8),
    ([777, 1234], 16, 16, 128, 32),
], ids=["ragged", "one_kv_head", "mha"])
def test_delta_one_launch_late_chunk_path(kvs, lens, H_q, H_kv, d_k, P):
    """With the wait bound at 0, every workgroup of the one-launch form that finds its
    sequence incomplete computes the missing chunks' statistics itself: the page scores and
    page sets must equal the default run's bit for bit, and the oracle's."""
    print(f"delta late-chunk path lens={lens} H_q={H_q}", flush=True)
    want = _run_batch(kvs, lens, H_q, H_kv, d_k, P, 16, 4, seed=5)
    prev = kvs.kvs_wait_limit(0)
    try:
        got = [_run_batch(kvs, lens, H_q, H_kv, d_k, P, 16, 4, seed=5) for _ in range(2)]
    finally:
        assert kvs.kvs_wait_limit(prev) == 0
    for g in got:
        assert np.array_equal(want[1], g[1])
        assert np.array_equal(want[2].view(np.uint32), g[2].view(np.uint32))
    _check(want[0], lens, want[1], want[2], H_q, H_kv, d_k, P, 16, 4)


@pytest.mark.slow
@pytest.mark.parametrize("lens", [[8192] * 32, [131072]], ids=["batch32x8k", "one128k"])
def test_delta_full_size(kvs, lens):
    """The decode batch the bench times (32 sequences of 8K tokens, Llama-3.1-8B
    heads), and one 128K-token sequence, with planted spans."""
    print(f"delta full size {len(lens)} x {lens[0]}", flush=True)
    layers, rho, S = _run_batch(kvs, lens, 32, 8, 128, 16, 64, 8, seed=9, spans=8)
    _check(layers, lens, rho, S, 32, 8, 128, 16, 64, 8)

"""GPU parity of kvs_gather_kv against the oracle's gather: a copy, so bit-exact.

Elements carry codes of their (head, token, channel), so any misplaced row
shows.  Lists come from the selection kernels themselves (per-head top-k
lists, a shared DELTA-style page list with -1 padding, CompactAttention CSR
page tables) as well as hand-made ones with out-of-range entries.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _coded(H, L, d, salt=0):
    g, t, c = np.meshgrid(np.arange(H), np.arange(L), np.arange(d), indexing="ij")
    return ((g * 7919 + t * 31 + c * 3 + salt) % 65521).astype(np.uint16)


def _dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def _dev32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("H,L,d,n,unit", [(8, 4096, 128, 300, 1), (3, 1000, 64, 77, 1),
                                          (2, 999, 128, 20, 16), (4, 130, 64, 9, 16),
                                          (2, 300, 256, 40, 1), (1, 50, 2048, 5, 2), (2, 77, 96, 13, 3)])
def test_gather_per_head_lists(kvs, H, L, d, n, unit):
    K, V = _coded(H, L, d, 1), _coded(H, L, d, 5)
    rng = np.random.default_rng(H * L + n)
    hi = (L + unit - 1) // unit
    idx = rng.integers(-2, hi + 2, size=(H, n + 3)).astype(np.int32)   # some out of range
    Ko, Vo = kvs.kvs_gather_kv(_dev16(K), _dev32(idx), n, V=_dev16(V), unit=unit, idx_ld=n + 3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(Ko), oracle.gather_kv(K, L=L, indices=idx, n=n, unit=unit, idx_ld=n + 3))
    np.testing.assert_array_equal(_bits(Vo), oracle.gather_kv(V, L=L, indices=idx, n=n, unit=unit, idx_ld=n + 3))


def test_gather_selection_lists(kvs):
    """The kept tokens of a kvs_select call (per KV head, window appended), K only."""
    H, L, d, budget, nf = 8, 20000, 128, 1000, 32
    n = L - nf
    x = synth.score_array(33, H, n)
    sel = kvs.kvs_select(torch.from_numpy(x).cuda(), n, kvs.select_args(budget=budget, n_forced=nf,
                                                                          pool=kvs.RED_MAX, pool_k=7))
    K = _coded(H, L, d, 2)
    Ko, _ = kvs.kvs_gather_kv(_dev16(K), sel, budget + nf, idx_ld=budget + nf)
    torch.cuda.synchronize()
    want = oracle.gather_kv(K, L=L, indices=sel.cpu().numpy(), n=budget + nf, idx_ld=budget + nf)
    np.testing.assert_array_equal(_bits(Ko), want)


def test_gather_shared_pages_sequence_major(kvs):
    """A DELTA-style page list (-1 padding) shared by every head, over sequence-major K."""
    H, L, d, P = 8, 5000, 128, 16
    Kh = _coded(H, L, d, 3)
    Ks = np.ascontiguousarray(Kh.transpose(1, 0, 2))             # [L][H][d]
    pages = np.array([0, 5, 17, 200, 312, -1, -1, 400], dtype=np.int32)   # 312 is the partial last page
    Ko, _ = kvs.kvs_gather_kv(_dev16(Ks), _dev32(pages), len(pages), unit=P, L=L, H=H,
                              head_stride=d, tok_stride=H * d,
                              K_out=torch.empty(H, len(pages) * P, d, dtype=torch.int16, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(Ko), oracle.gather_kv(Kh, L=L, indices=pages, n=len(pages), unit=P))


def test_gather_csr_block_tables(kvs):
    """CompactAttention's copy path: the per-group block lists of kvs_block_union_pagetable."""
    H_q, H_kv, n_qb, n_kvb, blk, d = 32, 8, 4, 64, 64, 128
    L = n_kvb * blk - 17                                         # ragged last block
    M = synth.block_mask(5, H_q, n_qb, n_kvb, density_den=8)
    indptr, indices = kvs.kvs_block_union_pagetable(torch.from_numpy(M).cuda(), H_q=H_q, H_kv=H_kv)
    K, V = _coded(H_kv, L, d, 7), _coded(H_kv, L, d, 9)
    Ko, Vo = kvs.kvs_gather_kv(_dev16(K), indices, n_kvb, V=_dev16(V), unit=blk, indptr=indptr)
    torch.cuda.synchronize()
    ip, ix = indptr.cpu().numpy(), indices.cpu().numpy()
    np.testing.assert_array_equal(_bits(Ko), oracle.gather_kv(K, L=L, indices=ix, n=n_kvb, unit=blk, indptr=ip))
    np.testing.assert_array_equal(_bits(Vo), oracle.gather_kv(V, L=L, indices=ix, n=n_kvb, unit=blk, indptr=ip))


@pytest.mark.slow
def test_gather_full_size(kvs):
    """20% of every KV head of a 128K-token Mistral-7B layer, K and V."""
    H, L, d = 8, 131072, 128
    n = L // 5
    K, V = _coded(H, L, d, 11), _coded(H, L, d, 13)
    rng = np.random.default_rng(0)
    idx = np.sort(np.stack([rng.choice(L, n, replace=False) for _ in range(H)]), axis=1).astype(np.int32)
    Ko, Vo = kvs.kvs_gather_kv(_dev16(K), _dev32(idx), n, V=_dev16(V), idx_ld=n)
    torch.cuda.synchronize()
    for g in range(H):
        np.testing.assert_array_equal(_bits(Ko)[g], K[g, idx[g]])
        np.testing.assert_array_equal(_bits(Vo)[g], V[g, idx[g]])

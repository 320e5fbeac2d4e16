"""GPU parity of kvs_token_pagetable (per-group page tables from kept token
positions) against the oracle: bit-exact CSR, on seeded lists with repeats,
-1 padding and positions past the cache, on a top-k selection with its window,
and at the Mistral-7B 128K shape (8 KV heads, 8190 pages of 16 tokens)."""
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


def _check(kvs, idx, P, n_pages, rpg, n=None):
    n = idx.shape[1] if n is None else n
    d = torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))).cuda()
    ptr, ind = kvs.kvs_token_pagetable(d, P, n_pages, rows_per_group=rpg, n=n)
    torch.cuda.synchronize()
    wptr, wind = oracle.token_pagetable(idx[:, :n], P=P, n_pages=n_pages, rows_per_group=rpg)
    np.testing.assert_array_equal(ptr.cpu().numpy(), wptr)
    np.testing.assert_array_equal(ind.cpu().numpy()[:wptr[-1]], wind)


@pytest.mark.parametrize("H,n,P,n_pages,rpg", [(8, 1056, 16, 8190, 1), (8, 500, 16, 100, 2),
                                               (6, 77, 1, 300, 3), (4, 3000, 64, 40, 4),
                                               (3, 1, 16, 1, 1), (2, 0, 16, 50, 1),
                                               (64, 200, 8, 1000, 8)])
def test_token_pagetable_parity(kvs, H, n, P, n_pages, rpg):
    r = synth.u64(H * 1000 + n, synth.STREAM_SCORES + 500, np.arange(max(H * n, 1)))
    idx = (r % np.uint64(n_pages * P + 40)).astype(np.int64).reshape(-1)[:H * n] - 20
    idx = idx.reshape(H, n)              # repeats, negative entries and positions past the cache
    _check(kvs, idx, P, n_pages, rpg)


def test_token_pagetable_of_a_selection(kvs):
    """The pages of a kvs_select row (top 1024 of 131040 with the 32-token window
    appended) per KV head, and the union over pairs of heads."""
    H, n, L = 8, 131040, 131072
    x = synth.score_array(91, H, n)
    idx = kvs.kvs_topk(torch.from_numpy(x).cuda(), n, 1024, n_forced=32)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    for rpg in (1, 2):
        _check(kvs, sel, 16, L // 16, rpg)


def test_token_pagetable_row_stride(kvs):
    """Rows read through idx_ld > n: entries past n are ignored."""
    idx = np.full((4, 64), 7, dtype=np.int64)
    idx[:, :40] = np.arange(40)[None, :] * 5
    d = torch.from_numpy(idx.astype(np.int32)).cuda()
    ptr, ind = kvs.kvs_token_pagetable(d, 16, 20, n=40)
    torch.cuda.synchronize()
    wptr, wind = oracle.token_pagetable(idx[:, :40], P=16, n_pages=20)
    np.testing.assert_array_equal(ptr.cpu().numpy(), wptr)
    np.testing.assert_array_equal(ind.cpu().numpy()[:wptr[-1]], wind)

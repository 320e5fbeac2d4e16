"""The C-ABI library loads, exports every symbol include/kvs.h declares, and
rejects invalid arguments on the host before anything is enqueued (no GPU
needed: every call here fails validation, so no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    return k


def test_every_declared_symbol_is_exported(kvs):
    names = _declared()
    assert "kvs_score" in names and "kvs_topk" in names
    lib = kvs.library()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kvs.EXPORTED)


def test_status_strings(kvs):
    lib = kvs.library()
    for st in (0, -1, -2, -3, -4, 7):
        assert lib.kvs_status_string(st)
    assert lib.kvs_version() >= 100


def _score_args(kvs, **kw):
    base = dict(L=512, W=16, d_k=64, H_q=4, H_kv=1, q_pos0=496)
    base.update(kw)
    return kvs.score_args(**base)


def test_score_workspace_is_shape_only(kvs):
    a = _score_args(kvs)
    assert kvs.kvs_score_workspace(a) > 0
    big = _score_args(kvs, L=131072, W=32, d_k=128, H_q=32, H_kv=8, q_pos0=131040)
    assert kvs.kvs_score_workspace(big) > kvs.kvs_score_workspace(a)
    assert kvs.kvs_score_workspace(_score_args(kvs, d_k=96)) == 0


def test_score_row_limit(kvs):
    """Up to 256 padded rows per KV head (two row groups); GROUP_MAX over two
    groups also keeps every query head's column sums in the workspace."""
    ok = dict(L=4096, W=32, d_k=128, H_q=64, H_kv=8, q_pos0=4064)
    ws_sum = kvs.kvs_score_workspace(_score_args(kvs, **ok))
    ws_max = kvs.kvs_score_workspace(_score_args(kvs, **ok, heads=kvs.HEADS_GROUP_MAX))
    assert ws_sum > 0 and ws_max >= ws_sum + 64 * 4096 * 4
    assert kvs.kvs_score_workspace(_score_args(kvs, L=4096, W=200, d_k=128, H_q=2, H_kv=2,
                                               q_pos0=3896)) > 0
    for bad in (dict(W=33, H_q=8, H_kv=1), dict(W=16, H_q=17, H_kv=1), dict(W=257, H_q=1, H_kv=1)):
        assert kvs.kvs_score_workspace(_score_args(kvs, **bad)) == 0, bad


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), -1), (dict(W=0), -1), (dict(H_q=3, H_kv=2), -1), (dict(q_pos0=-1), -1),
    (dict(heads=4), -1), (dict(scale=-1.0), -1), (dict(d_k=96), -2),
    (dict(W=64, H_q=8, H_kv=1), -2), (dict(W=33, H_q=8, H_kv=1), -2), (dict(q_row_stride=65), -1), (dict(s_ld=100), -1),
])
def test_score_rejects(kvs, kw, status):
    lib = kvs.library()
    a = _score_args(kvs, **kw)
    st = lib.kvs_score(ctypes.byref(a), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                       ctypes.c_void_p(256), 1 << 20, None)
    assert st == status


def test_score_rejects_null_misaligned_and_small_workspace(kvs):
    lib = kvs.library()
    a = _score_args(kvs)
    P = ctypes.c_void_p
    assert lib.kvs_score(ctypes.byref(a), None, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_score(ctypes.byref(a), P(18), P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_score(ctypes.byref(a), P(16), P(16), P(16), P(256), 8, None) == -3
    assert lib.kvs_score(ctypes.byref(a), P(16), P(16), P(16), None, 1 << 20, None) == -3
    assert lib.kvs_score(None, P(16), P(16), P(16), P(256), 1 << 20, None) == -1


def _raw_args(kvs, **kw):
    base = dict(L=4096, W=8, d_k=128, H_q=32, H_kv=8, q_pos0=4096, reduce=kvs.RED_MAX)
    base.update(kw)
    return kvs.raw_args(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), -1), (dict(W=0), -1), (dict(H_q=3, H_kv=2), -1), (dict(reduce=0), -1),
    (dict(reduce=3), -1), (dict(accumulate=3), -1), (dict(scale=-1.0), -1),
    (dict(q_pos0=4094), -2), (dict(d_k=96), -2), (dict(W=33), -2),
    (dict(H_q=16, H_kv=1, W=16), -2),             # 16 heads x 16 padded rows > 128
    (dict(H_q=64, H_kv=16), -2),                  # 16 KV heads of query rows exceed the LDS share
    (dict(d_k=64, H_q=120, H_kv=30, W=8), -2),    # 30 row tiles > 28 at d_k 64
    (dict(q_row_stride=65), -1), (dict(s_ld=100), -1),
])
def test_score_raw_rejects(kvs, kw, status):
    lib = kvs.library()
    a = _raw_args(kvs, **kw)
    P = ctypes.c_void_p
    assert lib.kvs_score_raw(ctypes.byref(a), P(16), P(16), P(16), None) == status


def test_score_raw_rejects_null_and_misaligned(kvs):
    lib = kvs.library()
    a = _raw_args(kvs)
    P = ctypes.c_void_p
    assert lib.kvs_score_raw(ctypes.byref(a), None, P(16), P(16), None) == -1
    assert lib.kvs_score_raw(ctypes.byref(a), P(16), P(24), P(16), None) == -1
    assert lib.kvs_score_raw(ctypes.byref(a), P(16), P(16), P(18), None) == -1
    assert lib.kvs_score_raw(None, P(16), P(16), P(16), None) == -1


def _delta_args(kvs, **kw):
    base = dict(B=4, d_k=128, H_q=32, H_kv=8, L_max=8192)
    base.update(kw)
    return kvs.delta_args(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -1), (dict(H_q=30), -1), (dict(P=0), -1), (dict(L_max=0), -1),
    (dict(L_recent=65), -1), (dict(K_pages=0, L_recent=0), -1), (dict(scale=-1.0), -1),
    (dict(k_tok_stride=12), -1), (dict(d_k=96), -2), (dict(H_q=256, H_kv=8), -2),
    (dict(P=24), -2), (dict(P=1024), -2), (dict(L_max=300000), -2),
])
def test_delta_rejects(kvs, kw, status):
    lib = kvs.library()
    a = _delta_args(kvs, **kw)
    P = ctypes.c_void_p
    assert lib.kvs_delta_pages(ctypes.byref(a), P(16), P(16), P(16), P(16), None, P(256), 1 << 40,
                               None) == status
    assert (kvs.kvs_delta_workspace(a) == 0) == (status != 0)


def test_delta_rejects_pointers_and_workspace(kvs):
    lib = kvs.library()
    a = _delta_args(kvs)
    need = kvs.kvs_delta_workspace(a)
    assert need >= 4 * 32 * 8192 * 4           # every head's logits of every cached token
    P = ctypes.c_void_p
    assert lib.kvs_delta_pages(ctypes.byref(a), None, P(16), P(16), P(16), None, P(256), need, None) == -1
    assert lib.kvs_delta_pages(ctypes.byref(a), P(8), P(16), P(16), P(16), None, P(256), need, None) == -1
    assert lib.kvs_delta_pages(ctypes.byref(a), P(16), P(16), P(16), P(16), None, P(256), need - 1,
                               None) == -3
    assert lib.kvs_delta_pages(ctypes.byref(a), P(16), P(16), P(16), P(16), None, None, need, None) == -3
    b0 = _delta_args(kvs, B=0)
    assert lib.kvs_delta_pages(ctypes.byref(b0), None, None, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("args,status", [
    # H, L, d_k, head_stride, tok_stride, idx_ld, n, unit
    ((-1, 10, 128, 0, 0, 0, 4, 1), -1), ((2, 10, 128, 0, 0, 0, 4, 0), -1),
    ((2, 10, 12, 0, 0, 0, 4, 1), -1), ((2, 10, 2056, 0, 0, 0, 4, 1), -1),
    ((2, 10, 128, 12, 0, 0, 4, 1), -1), ((2, 10, 128, 0, 0, -1, 4, 1), -1),
    ((2, -1, 128, 0, 0, 0, 4, 1), -1),
])
def test_gather_rejects(kvs, args, status):
    lib = kvs.library()
    H, L, d, hs, ts, ld, n, unit = args
    P = ctypes.c_void_p
    assert lib.kvs_gather_kv(P(16), None, H, L, d, hs, ts, P(16), ld, None, n, unit, P(16), None,
                             None) == status


def test_gather_rejects_pointers(kvs):
    lib = kvs.library()
    P = ctypes.c_void_p

    def call(K, V, idx, K_out, V_out, H=2, n=4):
        return lib.kvs_gather_kv(K, V, H, 10, 128, 0, 0, idx, 0, None, n, 1, K_out, V_out, None)

    assert call(None, None, P(16), P(16), None) == -1          # no K
    assert call(P(16), P(16), P(16), P(16), None) == -1        # V without V_out
    assert call(P(16), None, P(16), P(16), P(16)) == -1        # V_out without V
    assert call(P(18), None, P(16), P(16), None) == -1         # misaligned K
    assert call(P(16), None, P(18), P(16), None) == -1         # misaligned indices
    assert call(P(16), None, None, P(16), None) == -1          # no indices
    # nothing to copy: accepted without touching memory
    assert call(None, None, None, None, None, H=0) == 0
    assert call(None, None, None, None, None, n=0) == 0


def test_token_pagetable_rejects(kvs):
    lib = kvs.library()
    P = ctypes.c_void_p
    ws = lib.kvs_token_pagetable_workspace(8, 1, 8192)
    assert ws > 0
    assert lib.kvs_token_pagetable_workspace(8, 3, 100) == 0          # 3 does not divide 8
    assert lib.kvs_token_pagetable(P(16), 8, 10, 10, 3, 16, 100, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_token_pagetable(P(16), 8, 10, 9, 1, 16, 100, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_token_pagetable(P(16), 8, 10, 10, 1, 0, 100, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_token_pagetable(P(16), 8, 10, 10, 1, 16, 100, None, P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_token_pagetable(P(18), 8, 10, 10, 1, 16, 100, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_token_pagetable(P(16), 8, 10, 10, 1, 1 << 20, 1 << 12, P(16), P(16), P(256), 1 << 20,
                                   None) == -1                          # n_pages * P >= 2^31
    assert lib.kvs_token_pagetable(P(16), 8, 10, 10, 1, 16, 100, P(16), P(16), P(256), 8, None) == -3


def test_other_entry_points_reject(kvs):
    lib = kvs.library()
    P = ctypes.c_void_p
    # pool: even kernel, bad reductions, no outputs, ld < n
    assert lib.kvs_pool_pages(P(16), 2, 10, 10, 0, 2, 6, 0, 1, P(16), None, None, None) == -1
    assert lib.kvs_pool_pages(P(16), 2, 10, 10, 5, 2, 7, 0, 1, P(16), None, None, None) == -1
    assert lib.kvs_pool_pages(P(16), 2, 10, 10, 0, 2, 7, 0, 1, None, None, None, None) == -1
    assert lib.kvs_pool_pages(P(16), 2, 10, 9, 0, 2, 7, 0, 1, P(16), None, None, None) == -1
    assert lib.kvs_pool_pages(P(16), 2, 10, 10, 0, 2, 7, 4, 3, None, P(16), None, None) == -1
    # top-k: budget > n, negative forced, null output
    assert lib.kvs_topk(P(16), 1, 10, 10, 11, None, 0, P(16), None, None, 0, None) == -1
    assert lib.kvs_topk(P(16), 1, 10, 10, 5, None, -1, P(16), None, None, 0, None) == -1
    assert lib.kvs_topk(P(16), 1, 10, 10, 5, None, 0, None, None, None, 0, None) == -1
    assert lib.kvs_topk(P(16), 1, 10, 10, 5, None, 0, P(16), P(18), None, 0, None) == -1
    # union: H_q not a multiple of H_kv, sub_group not dividing G, tiny workspace
    assert lib.kvs_block_union_pagetable(P(16), 6, 4, 0, 2, 8, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_block_union_pagetable(P(16), 8, 2, 3, 2, 8, P(16), P(16), P(256), 1 << 20, None) == -1
    assert lib.kvs_block_union_pagetable(P(16), 8, 2, 0, 2, 8, P(16), P(16), P(256), 4, None) == -3
    # aggregate: bad mode, tiny workspace for SUM_L1
    assert lib.kvs_aggregate_layers(P(16), P(16), 2, 10, 10, 3, 1, P(256), 1 << 20, None) == -1
    assert lib.kvs_aggregate_layers(P(16), P(16), 2, 10, 10, 4, 1, P(256), 1, None) == -3
    # cluster: page count inconsistent with n and P
    assert lib.kvs_cluster_priority(P(16), P(16), 1, 3, 16, 100, 1e-3, 3, P(16), None) == -1
    # block select: chunk beyond the keys, p_mass out of range, unsupported d_k
    a = kvs.block_select_args(Lq=64, L=128, d_k=128, H_q=4, H_kv=1, q_pos0=100)
    assert lib.kvs_block_select(ctypes.byref(a), P(16), P(16), P(16), P(256), 1 << 24, None) == -1
    a = kvs.block_select_args(Lq=64, L=128, d_k=128, H_q=4, H_kv=1, q_pos0=64, p_mass=1.5)
    assert lib.kvs_block_select(ctypes.byref(a), P(16), P(16), P(16), P(256), 1 << 24, None) == -1
    a = kvs.block_select_args(Lq=64, L=128, d_k=80, H_q=4, H_kv=1, q_pos0=64)
    assert lib.kvs_block_select(ctypes.byref(a), P(16), P(16), P(16), P(256), 1 << 24, None) == -2
    a = kvs.block_select_args(Lq=64, L=1 << 20, d_k=128, H_q=4, H_kv=1, q_pos0=64, block=64)
    assert lib.kvs_block_select(ctypes.byref(a), P(16), P(16), P(16), P(256), 1 << 30, None) == -2
    # cached block means: cache too small, more cached blocks than complete ones, misaligned
    a = kvs.block_select_args(Lq=64, L=200, d_k=128, H_q=4, H_kv=1, q_pos0=136, block=64)
    cached = lib.kvs_block_select_cached
    assert cached(ctypes.byref(a), P(16), P(16), P(256), 3, 0, P(16), P(256), 1 << 24, None) == -1
    assert cached(ctypes.byref(a), P(16), P(16), P(256), 4, 4, P(16), P(256), 1 << 24, None) == -1
    assert cached(ctypes.byref(a), P(16), P(16), P(264), 4, 3, P(16), P(256), 1 << 24, None) == -1


def test_select_rejects(kvs):
    lib = kvs.library()
    P = ctypes.c_void_p

    def call(ws=P(256), nb=1 << 24, n=100000, ld=100000, **kw):
        a = kvs.select_args(**{"budget": 10, **kw})
        return lib.kvs_select(P(16), 2, n, ld, ctypes.byref(a), P(16), ws, nb, None)

    assert call(pool=kvs.RED_MAX, pool_k=6) == -1            # even pooling window
    assert call(pool=kvs.RED_SUM, pool_k=7) == -1            # SUM is not a pooling mode
    assert call(pool=kvs.RED_MAX, pool_k=2051) == -2         # halo beyond the LDS stage
    assert call(cluster_P=16, cluster_r=-1) == -1
    assert call(cluster_P=16, cluster_theta=float("nan"), cluster_r=3) == -1
    assert call(cluster_P=1000, cluster_r=100) == -2         # P + r beyond the halo
    assert call(cluster_P=16, cluster_r=3, pool=kvs.RED_MAX, pool_k=7) == -2
    assert call(budget=100001) == -1
    assert call(ld=99999) == -1
    assert call(nb=16) == -3                                  # workspace too small
    assert call(ws=P(264)) == -1                              # workspace misaligned
    assert lib.kvs_select(P(16), 2, 100, 100, None, P(16), P(256), 1 << 24, None) == -1
    assert lib.kvs_topk(P(16), 1, 100000, 100000, 10, None, 0, P(16), None, P(256), 16, None) == -3
    assert lib.kvs_select_workspace(8, 131040, 1024) == lib.kvs_topk_workspace(8, 131040, 1024)
    assert lib.kvs_select_workspace(8, 131040, 1024) > 0
    assert lib.kvs_select_workspace(8, 16384, 100) == 0      # one part: no candidates stored
    assert lib.kvs_select_workspace(8, 100, 101) == 0        # budget > n

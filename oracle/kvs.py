"""fp64 reference of the scoring-and-selection path (TEST INFRASTRUCTURE ONLY).

Every function is the plain definition written out with NumPy in float64; a
matrix product, an argsort and a cumulative sum serve as library steps.  There
is no blocking, fusion or reordering beyond what each definition states.  Only
``tests/``, the smoke check and the bench's CPU-baseline leg use this module.

Sources (web pages on the subject; cited by title and section):

* [CLAA] "CLAA: cross-layer attention aggregation ..." (pinghaoyang.com.cn blog
  post): section "Three representative token-ranking methods" (FastKV window
  score: softmax over keys, summed over the window rows and all heads; logit
  scale 1/sqrt(d_k)); section "Three design decisions" (per-layer window score,
  Eq. 6 token-wise max over the buffered layers); section "The oracle
  construction" (1-D pooling with kernel 7); section "Complete flow and cost"
  (top-k by keep rate, kept tokens keep their original positions).
* [ClusterAttn] "ClusterAttn: KV Cache Compression under Intrinsic Attention
  Clustering" (papercache.org note): section "Background and key observations",
  the feature-aggregation equations (window logits W_win, window mask M_win,
  softmax A_win^m, column sum P); section "Method details" (density-based
  clustering: block max, threshold theta, neighbourhood r, unique+topk fill;
  Table 1 theta per compression size; window concatenated afterwards).
* [CompactAttention] "CompactAttention: Accelerating Chunked Prefill with
  Block-Union KV Selection": "Core method" / "Method step details" (Q-block
  union, intra-group union, 4-head subgroups, per-group page table T_{b,g},
  kv_indptr/kv_indices); "Technical novelty" (minimality of T_{b,g}).
* [LookaheadKV] "LookaheadKV: Fast and Accurate KV Cache Eviction by Glimpsing
  into the Future without Generation": "Background: KL divergence and ListNet"
  (L1 normalisation s / ||s||_1).
* [DELTA] "DELTA: Dynamic Layer-Aware Token Attention for Efficient
  Long-Context Reasoning": "Key design 2" (token score = max over heads of the
  post-softmax attention; page score = sum over the page's tokens; recency
  pages forced); "Key design 3" (page size P = 16).

Readings where the pages are silent or garbled:
contiguous GQA grouping h -> h // G; causal visibility t <= q_pos0 + j inside the
window (the garbled ``max(W, M_win)`` read as an additive -inf mask); scores over
all L keys; GROUP_MAX sums a head's W rows before the max over heads; pooling
clipped to [0, n) (MEAN divides by the in-range count); argmax ties go to the
lowest index; top-k key (priority desc, value desc, index asc), -0 == +0, NaN
below every number; cluster centres are page argmaxes whose page max >= theta
and a token is prioritised if within r of a centre; top-p keeps a block while
the mass ranked strictly before it is < p.

Raw scores (GemFilter, Speculative Prefill, answer oracle): the queries sit at
or after the last prompt token, so nothing is masked; the scale defaults to
1/sqrt(d_k) as for the softmax scores.

Parity pins (tests/test_oracle_*.py): row-stochastic mass, identical-key closed
forms, SciPy softmax special case, GQA mapping by construction, linearity,
permutation and shift invariance, planted spans rank first; SciPy filters for
pooling; hand-built page/argmax, cluster, top-k, block-select and union cases
with known answers; brute force on tiny arrays.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

HEADS_NONE, HEADS_GROUP_SUM, HEADS_GROUP_MAX, HEADS_ALL_SUM = 0, 1, 2, 3
RED_NONE, RED_SUM, RED_MAX, RED_MEAN, RED_SUM_L1 = 0, 1, 2, 3, 4


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Scoring: masked softmax over keys, column sums over window rows and heads
# ---------------------------------------------------------------------------

def score(Q, K, *, L: int, W: int, d_k: int, H_q: int, H_kv: int, q_pos0: int,
          heads: int = HEADS_GROUP_SUM, scale: Optional[float] = None,
          per_row: bool = False) -> np.ndarray:
    """Column sums of the masked, softmax-normalised window attention.

    [ClusterAttn] feature aggregation: logits of the window queries against the
    prompt keys, masked, softmax-normalised over keys, summed over window rows.
    [CLAA] FastKV / per-layer window score: also summed over the heads of the
    group (here the G query heads sharing KV head g), or over every head of the
    layer (ALL_SUM: the per-layer score CLAA buffers, "Three design
    decisions").  [DELTA] key design 2: maximum over heads instead of the sum.

    Q: bf16 bits [H_q][W][d_k]; K: bf16 bits [H_kv][L][d_k].
    Row j of every head sits at position q_pos0 + j and sees keys t <= q_pos0 + j.
    Returns float64 [H_q][L] (NONE), [H_kv][L] (GROUP_SUM / GROUP_MAX) or
    [1][L] (ALL_SUM).
    With ``per_row`` returns the attention rows [H_q][W][L] instead.
    """
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    q = bf16_to_f64(Q).reshape(H_q, W, d_k)
    k = bf16_to_f64(K).reshape(H_kv, L, d_k)
    t = np.arange(L)
    pos = q_pos0 + np.arange(W)
    visible = t[None, :] <= pos[:, None]                 # [W][L]
    per_head = np.zeros((H_q, L), dtype=np.float64)
    rows = np.zeros((H_q, W, L), dtype=np.float64) if per_row else None
    for h in range(H_q):
        g = h // G                                        # contiguous GQA grouping
        s = scale * (q[h] @ k[g].T)                       # [W][L] logits
        s = np.where(visible, s, -np.inf)                 # additive -inf mask
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)                                 # masked entries -> 0
        a = e / e.sum(axis=1, keepdims=True)              # softmax over keys
        if per_row:
            rows[h] = a
        per_head[h] = a.sum(axis=0)                       # column sum over window rows
    if per_row:
        return rows
    if heads == HEADS_NONE:
        return per_head
    if heads == HEADS_ALL_SUM:
        return per_head.sum(axis=0, keepdims=True)
    grouped = per_head.reshape(H_kv, G, L)
    if heads == HEADS_GROUP_SUM:
        return grouped.sum(axis=1)
    if heads == HEADS_GROUP_MAX:
        return grouped.max(axis=1)
    raise ValueError("unknown heads mode")


# ---------------------------------------------------------------------------
# Raw (pre-softmax) scoring
# ---------------------------------------------------------------------------

def score_raw(Q, K, *, L: int, W: int, d_k: int, H_q: int, H_kv: int, reduce: int = RED_SUM,
              scale: Optional[float] = None) -> np.ndarray:
    """Raw attention logits of W query rows, reduced over all H_q query heads.

    [CLAA] "Three representative token-ranking methods": GemFilter scores a
    prompt token by the pre-softmax attention logit of the last prompt token's
    query, scaled by 1/sqrt(d_k) and summed over all heads (SUM with W = 1).
    Speculative Prefill takes, for each lookahead query, the maximum raw logit
    over all layers and heads (MAX here, the layers in ``aggregate_raw``); the
    answer-informed oracle ("The oracle construction") does the same with the
    queries of the generated answer (``use_softmax=False``).

    Q: bf16 bits [H_q][W][d_k]; K: bf16 bits [H_kv][L][d_k]; head h reads KV
    head h // G.  These queries come at or after the last prompt token, so every
    row sees every key and nothing is masked.
    Returns float64 [W][L]: R[j][t] = SUM or MAX over h of scale * q[h][j] . k[h//G][t].
    """
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    if reduce not in (RED_SUM, RED_MAX):
        raise ValueError("raw scores reduce over heads by SUM or MAX")
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    q = bf16_to_f64(Q).reshape(H_q, W, d_k)
    k = bf16_to_f64(K).reshape(H_kv, L, d_k)
    out = None
    for h in range(H_q):
        s = scale * (q[h] @ k[h // G].T)                  # [W][L] raw logits of head h
        if out is None:
            out = s
        elif reduce == RED_SUM:
            out = out + s
        else:
            out = np.maximum(out, s)
    return out


def aggregate_raw(layer_scores: Sequence[np.ndarray], pool_k: int = 7) -> np.ndarray:
    """Speculative Prefill / answer-oracle token scores from per-layer raw scores.

    [CLAA] "The oracle construction" and the Speculative Prefill paragraph:
    maximum over layers (each layer's [W][L] already holds the maximum over its
    heads), then the mean over the W queries, then 1-D average pooling with
    kernel ``pool_k`` (0 or 1: no pooling).  Returns float64 [L].
    """
    acc = np.asarray(layer_scores[0], dtype=np.float64).copy()
    for s in layer_scores[1:]:
        acc = np.maximum(acc, np.asarray(s, dtype=np.float64))
    y = acc.mean(axis=0, keepdims=True)
    if pool_k > 1:
        y = pool(y, RED_MEAN, pool_k)
    return y[0]


# ---------------------------------------------------------------------------
# Pooling and page aggregation
# ---------------------------------------------------------------------------

def head_reduce(x, mode: int) -> np.ndarray:
    """Reduce the rows of x [H][n] to one row: SUM, MAX or MEAN; NONE keeps x.

    [DELTA] key design 2 takes the maximum over heads before paging; the
    Speculative Prefill / answer-oracle aggregation averages over queries.
    """
    x = np.asarray(x, dtype=np.float64)
    if mode == RED_NONE:
        return x
    if mode == RED_SUM:
        return x.sum(axis=0, keepdims=True)
    if mode == RED_MAX:
        return x.max(axis=0, keepdims=True)
    if mode == RED_MEAN:
        return x.mean(axis=0, keepdims=True)
    raise ValueError("head reduce must be NONE, SUM, MAX or MEAN")


def pool(x, mode: int, k: int) -> np.ndarray:
    """1-D pooling with odd kernel k over [t - r, t + r] clipped to [0, n).

    [CLAA] the oracle construction and experimental setup: 1-D pooling with
    kernel 7 smooths token scores before ranking (average there; max pooling is
    the same window with max).  MEAN divides by the number of in-range terms.
    """
    x = np.asarray(x, dtype=np.float64)
    if mode == RED_NONE:
        return x.copy()
    if k < 1 or k % 2 == 0:
        raise ValueError("pool kernel must be odd")
    r = (k - 1) // 2
    H, n = x.shape
    if mode == RED_MAX:
        out = np.full((H, n), -np.inf)
    elif mode == RED_MEAN:
        out = np.zeros((H, n))
    else:
        raise ValueError("pool must be NONE, MAX or MEAN")
    cnt = np.zeros(n)
    for o in range(-r, r + 1):
        lo = max(0, -o)
        hi = min(n, n - o)
        if hi <= lo:
            continue
        src = x[:, lo + o:hi + o]
        if mode == RED_MAX:
            out[:, lo:hi] = np.maximum(out[:, lo:hi], src)
        else:
            out[:, lo:hi] += src
        cnt[lo:hi] += 1
    if mode == RED_MEAN:
        out = out / cnt[None, :]
    return out


def pages(x, P: int, mode: int) -> Tuple[np.ndarray, np.ndarray]:
    """Page aggregation over tokens [uP, min(uP + P, n)) and the page argmax.

    [DELTA] key design 2 (page score = sum over the page's tokens) and key
    design 3 (P = 16 tokens per page); [ClusterAttn] method details (block max
    and the block-level max index).  The argmax is the lowest index attaining
    the page maximum.
    """
    x = np.asarray(x, dtype=np.float64)
    H, n = x.shape
    n_pages = (n + P - 1) // P
    z = np.zeros((H, n_pages))
    arg = np.zeros((H, n_pages), dtype=np.int64)
    for u in range(n_pages):
        seg = x[:, u * P:min(u * P + P, n)]
        if mode == RED_SUM:
            z[:, u] = seg.sum(axis=1)
        elif mode == RED_MAX:
            z[:, u] = seg.max(axis=1)
        else:
            raise ValueError("page reduce must be SUM or MAX")
        arg[:, u] = u * P + np.argmax(seg, axis=1)       # first index of the maximum
    return z, arg


def pool_pages(S, *, head_mode: int = RED_NONE, pool_mode: int = RED_NONE, pool_k: int = 7,
               P: int = 0, page_mode: int = RED_SUM):
    """head reduce -> pool -> page, the order the library applies them in."""
    y = pool(head_reduce(S, head_mode), pool_mode, pool_k)
    if P:
        z, arg = pages(y, P, page_mode)
        return y, z, arg
    return y, None, None


# ---------------------------------------------------------------------------
# DELTA decode-time page sets
# ---------------------------------------------------------------------------

def delta_pages(Q, K, *, L: int, d_k: int, H_q: int, H_kv: int, P: int = 16, K_pages: int = 64,
                L_recent: int = 8, scale: Optional[float] = None):
    """DELTA's page set rho for one decode query of one sequence at a Delta-layer.

    [DELTA] "Key design 2": the token score is the maximum over the heads of the
    decode query's softmax attention, s_t = max_j alpha_j(t); a page's score is
    the sum of its tokens' scores; rho is the last L pages together with the
    top K - L of the remaining pages by page score.  "Key design 3": pages of
    P = 16 tokens, K = 64 pages, L = 8 recent pages.

    Q: bf16 bits [H_q][d_k], the decode token's query at position L - 1 (it sees
    every cached key).  K: bf16 bits [H_kv][L][d_k].
    Returns (rho, page_scores): rho int64 [K_pages] lists the chosen older pages
    in ascending order, then the recent pages in ascending order, then -1 for
    unused slots; page_scores float64 [ceil(L / P)].
    """
    if K_pages < L_recent or L_recent < 0:
        raise ValueError("need 0 <= L_recent <= K_pages")
    a = score(np.asarray(Q).reshape(H_q, 1, d_k), K, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv,
              q_pos0=L - 1, heads=HEADS_NONE, scale=scale)     # [H_q][L] softmax rows
    s = a.max(axis=0, keepdims=True)                          # max over heads
    z, _ = pages(s, P, RED_SUM)                               # page sums
    n_pages = z.shape[1]
    n_recent = min(L_recent, n_pages)
    n_cand = n_pages - n_recent
    keep = min(K_pages - L_recent, n_cand)
    chosen = topk(z[:, :n_cand], keep, None, n_recent)[0]     # ascending, then the recent pages
    rho = np.full(K_pages, -1, dtype=np.int64)
    rho[:len(chosen)] = chosen
    return rho, z[0]


# ---------------------------------------------------------------------------
# KV gather (compaction of the selected tokens, pages or blocks)
# ---------------------------------------------------------------------------

def gather_kv(X, *, L: int, indices, n: int, unit: int = 1, idx_ld: int = 0, indptr=None):
    """Compact copy of the selected tokens of X (bf16 bits, [H][L][d]).

    [CLAA] "Complete flow and cost": each layer keeps its KV cache for the
    indices chosen by top-k of that layer's scores, gathered from K and V.
    [CompactAttention] "Core method" contrasts this explicit copy with its
    page-table path; [DELTA] "Key design 3" reads whole pages.
    Head g's list is indices[indptr[g] : indptr[g+1]] (at most n entries) when
    indptr is given, else indices[g * idx_ld : g * idx_ld + n] (idx_ld = 0: one
    list shared by every head).  Entry e with value i selects the `unit` tokens
    [i * unit, i * unit + unit); tokens at or past L, and negative entries,
    give zero rows.  Returns uint16 [H][n * unit][d]; rows past a head's list
    are zero.
    """
    X = np.asarray(X, dtype=np.uint16)
    H, _, d = X.shape
    idx = np.asarray(indices, dtype=np.int64).reshape(-1)
    out = np.zeros((H, n * unit, d), dtype=np.uint16)
    for g in range(H):
        if indptr is not None:
            lst = idx[int(indptr[g]):int(indptr[g + 1])][:n]
        else:
            lst = idx[g * idx_ld:g * idx_ld + n]
        for e, i in enumerate(lst):
            for o in range(unit):
                t = int(i) * unit + o
                if i >= 0 and t < L:
                    out[g, e * unit + o] = X[g, t]
    return out


# ---------------------------------------------------------------------------
# Cross-layer aggregation
# ---------------------------------------------------------------------------

def aggregate_layers(layer_scores: Sequence[np.ndarray], mode: int) -> np.ndarray:
    """Combine per-layer token scores into one vector.

    Each layer's rows are summed over heads first (the FastKV / CLAA per-layer
    score sums over all heads).  SUM_L1: each layer divided by its own L1 norm
    ([LookaheadKV] s / ||s||_1), then summed over layers.  MAX: token-wise
    maximum over layers ([CLAA] Eq. 6).
    """
    per_layer = [np.asarray(s, dtype=np.float64).sum(axis=0) for s in layer_scores]
    if mode == RED_SUM_L1:
        acc = np.zeros_like(per_layer[0])
        for s in per_layer:
            acc = acc + s / np.abs(s).sum()
        return acc
    if mode == RED_MAX:
        acc = per_layer[0].copy()
        for s in per_layer[1:]:
            acc = np.maximum(acc, s)
        return acc
    raise ValueError("aggregate mode must be SUM_L1 or MAX")


# ---------------------------------------------------------------------------
# Density clustering priority ([ClusterAttn] method details)
# ---------------------------------------------------------------------------

def cluster_priority(page, page_arg, n: int, theta: float, r: int) -> np.ndarray:
    """uint8 [H][n]: 1 where a token lies within r of a cluster centre.

    Centres are the block-level max indices whose block maximum is not below
    theta; each centre gathers its neighbourhood [c - r, c + r].
    """
    page = np.asarray(page, dtype=np.float64)
    page_arg = np.asarray(page_arg)
    H = page.shape[0]
    prio = np.zeros((H, n), dtype=np.uint8)
    for h in range(H):
        for u in range(page.shape[1]):
            if page[h, u] >= theta:
                c = int(page_arg[h, u])
                prio[h, max(0, c - r):min(n, c + r + 1)] = 1
    return prio


# ---------------------------------------------------------------------------
# Top-k selection with stable ties and a forced suffix
# ---------------------------------------------------------------------------

def topk(S, budget: int, priority=None, n_forced: int = 0) -> np.ndarray:
    """Indices of the ``budget`` best tokens per row, ascending, then the suffix.

    Order: priority descending, value descending, index ascending (ties go to
    the lower index).  -0.0 equals +0.0; NaN ranks below every number.  The
    forced suffix [n, n + n_forced) is appended ([ClusterAttn] the observation
    window is kept in full; [DELTA] recency pages).  Output is sorted ascending
    so kept tokens keep their original order and positions ([CLAA] complete
    flow: original position ids).
    """
    S = np.asarray(S)
    H, n = S.shape
    if not 0 <= budget <= n:
        raise ValueError("budget must be in [0, n]")
    out = np.zeros((H, budget + n_forced), dtype=np.int64)
    for h in range(H):
        v = S[h].astype(np.float64)
        nan = np.isnan(v)
        vv = np.where(nan, 0.0, v) + 0.0                   # -0.0 + 0.0 == +0.0
        pr = np.zeros(n, dtype=np.int64) if priority is None else np.asarray(priority[h], dtype=np.int64)
        idx = np.arange(n)
        # lexsort: last key is primary.
        order = np.lexsort((idx, -vv, (~nan).astype(np.int64) * -1, -pr))
        chosen = np.sort(order[:budget])
        out[h, :budget] = chosen
        out[h, budget:] = np.arange(n, n + n_forced)
    return out


# ---------------------------------------------------------------------------
# Chunked-prefill block selection and block union ([CompactAttention])
# ---------------------------------------------------------------------------

def block_select(Qc, K, *, Lq: int, L: int, d_k: int, H_q: int, H_kv: int, q_pos0: int,
                 block: int = 64, p_mass: float = 0.9, scale: Optional[float] = None,
                 return_before: bool = False):
    """Binary block mask M [H_q][n_qb][n_kvb] from mean-pooled block logits.

    Kb[g][j] = mean of the keys of block j; Qb[h][i] = mean of the chunk rows of
    query block i.  Query block i ends at position q_pos0 + last row of the block;
    KV block j is visible when its first token is not after that position.
    Logits scale * Qb . Kb over visible blocks, softmax; blocks ordered by
    (probability desc, j asc); block j is kept while the mass ranked strictly
    before it is < p_mass (so the crossing block is kept).  With ``return_before``
    also returns that preceding mass per block (+inf where not visible).
    """
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    G = H_q // H_kv
    q = bf16_to_f64(Qc).reshape(H_q, Lq, d_k)
    k = bf16_to_f64(K).reshape(H_kv, L, d_k)
    n_qb = (Lq + block - 1) // block
    n_kvb = (L + block - 1) // block
    Kb = np.zeros((H_kv, n_kvb, d_k))
    for j in range(n_kvb):
        Kb[:, j] = k[:, j * block:min(L, j * block + block)].mean(axis=1)
    M = np.zeros((H_q, n_qb, n_kvb), dtype=np.uint8)
    mass_before = np.full((H_q, n_qb, n_kvb), np.inf)
    for h in range(H_q):
        g = h // G
        for i in range(n_qb):
            rows = q[h, i * block:min(Lq, i * block + block)]
            qb = rows.mean(axis=0)
            end_pos = q_pos0 + min(Lq, i * block + block) - 1
            vis = np.arange(n_kvb) * block <= end_pos
            b = scale * (Kb[g] @ qb)
            b = np.where(vis, b, -np.inf)
            e = np.exp(b - b.max())
            p = e / e.sum()
            order = np.lexsort((np.arange(n_kvb), -p))
            before = np.cumsum(p[order]) - p[order]          # mass ranked strictly before
            keep = (before < p_mass) & vis[order]
            M[h, i, order[keep]] = 1
            mass_before[h, i, order] = np.where(vis[order], before, np.inf)
    if return_before:
        return M, mass_before
    return M


def block_union_pagetable(M, *, H_q: int, H_kv: int, sub_group: int = 0):
    """Per-group KV page table (CSR) from a per-head 2-D block mask.

    M_bar[h][j] = OR over query blocks i of M[h][i][j]; G[s][j] = OR over the
    heads h of subgroup s (subgroups of ``sub_group`` consecutive heads inside a
    KV group); T_s = {j : G[s][j] = 1} listed ascending.  Returns kv_indptr
    [n_groups + 1] (exclusive prefix sum of |T_s|) and kv_indices.
    """
    M = np.asarray(M, dtype=np.uint8)
    G = H_q // H_kv
    sg = G if sub_group == 0 else sub_group
    if G % sg:
        raise ValueError("sub_group must divide H_q / H_kv")
    n_groups = H_q // sg
    mbar = M.max(axis=1)                                   # Q-block union
    indptr = np.zeros(n_groups + 1, dtype=np.int64)
    lists: List[np.ndarray] = []
    for s in range(n_groups):
        gm = mbar[s * sg:(s + 1) * sg].max(axis=0)        # intra-group union
        js = np.nonzero(gm)[0]
        lists.append(js)
        indptr[s + 1] = indptr[s] + len(js)
    indices = np.concatenate(lists) if lists else np.zeros(0, dtype=np.int64)
    return indptr, indices.astype(np.int64)


def token_pagetable(idx, *, P: int, n_pages: int, rows_per_group: int = 1):
    """Per-group KV page table (CSR) from token index lists.

    [CompactAttention] "Method step details": a group's page table lists, in
    ascending order, every KV page that one of its heads needs (kv_indices),
    kv_indptr being the exclusive prefix sum of the counts; "Technical
    novelty": the table is the smallest one that covers the selection.  [DELTA]
    "Key design 3": the cache is read in whole pages of P tokens.
    idx: int [H][n], the kept token positions of each row (for instance a top-k
    list with its window); group s holds rows s * rows_per_group ...
    (s + 1) * rows_per_group - 1.  Token i lies in page i // P; entries outside
    [0, n_pages * P) (such as -1 padding) name no page; repeated pages are
    listed once.  Returns (indptr int64 [n_groups + 1], indices int64).
    """
    idx = np.asarray(idx, dtype=np.int64)
    H = idx.shape[0]
    if rows_per_group < 1 or H % rows_per_group:
        raise ValueError("rows_per_group must divide the number of rows")
    n_groups = H // rows_per_group
    indptr = np.zeros(n_groups + 1, dtype=np.int64)
    out: List[int] = []
    for s in range(n_groups):
        pages = set()
        for h in range(s * rows_per_group, (s + 1) * rows_per_group):
            for i in idx[h]:
                if 0 <= i < n_pages * P:
                    pages.add(int(i) // P)
        out.extend(sorted(pages))
        indptr[s + 1] = len(out)
    return indptr, np.array(out, dtype=np.int64)

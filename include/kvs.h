/*
 * kvs.h - attention-based prompt-token importance scoring and selection on
 * AMD Instinct MI355X (gfx950).  C ABI of libkvs.so.
 *
 * Every call enqueues HIP kernels on `stream` (a hipStream_t passed as void*;
 * NULL selects the default stream) and returns without synchronizing.  All
 * tensor pointers are DEVICE pointers that the caller allocates and owns; the
 * library never allocates, frees or copies to the host, and never writes an
 * input.  Scratch memory comes from the caller through the `ws` / `ws_bytes`
 * workspace arguments, sized by the matching *_workspace() query.  Calls are
 * stateless and reentrant; calls on different streams may run concurrently as
 * long as their workspaces and outputs do not overlap.
 *
 * Errors: argument problems are detected on the host and reported BEFORE
 * anything is enqueued.  KVS_EINVAL: a null pointer, a size out of range, a
 * misaligned pointer or stride.  KVS_EUNSUPPORTED: a valid shape the
 * kernels do not cover.  KVS_EWORKSPACE: ws_bytes below the query's answer.
 * KVS_EHIP: a kernel launch failed.  Faults inside kernels surface at the
 * caller's next synchronization.  No C++ exception crosses this boundary.
 *
 * Sources (web pages on the subject, cited by title and section):
 *  [CLAA]   CLAA cross-layer attention aggregation blog post: "Three
 *           representative token-ranking methods" (FastKV window score),
 *           "Three design decisions" (per-layer window score; Eq. 6 max over
 *           buffered layers), "The oracle construction" (1-D pooling, kernel
 *           7), "Complete flow and cost" (topk by keep rate; original
 *           position ids).
 *  [ClusterAttn] "ClusterAttn: KV Cache Compression under Intrinsic Attention
 *           Clustering": "Background and key observations" (window logits,
 *           window mask, softmax, column sum P), "Method details" (density
 *           clustering; Table 1 theta; window concatenated).
 *  [CompactAttention] "CompactAttention: Accelerating Chunked Prefill with
 *           Block-Union KV Selection": "Method step details" (Q-block union,
 *           intra-group union, kv_indptr / kv_indices), "Technical novelty"
 *           (minimal page table).
 *  [LookaheadKV] "LookaheadKV: Fast and Accurate KV Cache Eviction by
 *           Glimpsing into the Future without Generation": background on KL
 *           divergence (L1 normalisation s / ||s||_1).
 *  [DELTA]  "DELTA: Dynamic Layer-Aware Token Attention for Efficient
 *           Long-Context Reasoning": key design 2 (max over heads; page sum;
 *           recency pages), key design 3 (P = 16).
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvs_status;
#define KVS_OK 0
#define KVS_EINVAL (-1)
#define KVS_EUNSUPPORTED (-2)
#define KVS_EWORKSPACE (-3)
#define KVS_EHIP (-4)
#define KVS_ESCRATCH (-5) /* kvs_score_noalloc: the call needs more than its static scratch */

/* Head reduction of the score: per query head, or over the G = H_q / H_kv
 * query heads that share a KV head. */
#define KVS_HEADS_NONE 0      /* output rows: H_q                         */
#define KVS_HEADS_GROUP_SUM 1 /* output rows: H_kv, sum over the G heads  */
#define KVS_HEADS_GROUP_MAX 2 /* output rows: H_kv, max over the G heads  */
#define KVS_HEADS_ALL_SUM 3   /* output rows: 1, sum over all H_q heads    */

/* Reductions used by pooling, paging and layer aggregation. */
#define KVS_RED_NONE 0
#define KVS_RED_SUM 1
#define KVS_RED_MAX 2
#define KVS_RED_MEAN 3
#define KVS_RED_SUM_L1 4

/* Human-readable name of a status code (static string, never NULL). */
const char* kvs_status_string(kvs_status s);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t kvs_version(void);

/* ------------------------------------------------------------------------
 * kvs_score - window-attention column scores.
 *
 * [ClusterAttn] feature aggregation and [CLAA] FastKV / per-layer window
 * score: for every query head h (KV head g = h / G, contiguous grouping) and
 * window row j at absolute position q_pos0 + j,
 *     s[h][j][t] = scale * sum_c Q[h][j][c] * K[g][t][c]     for t <= q_pos0 + j,
 *     a[h][j][t] = softmax over the visible t of s[h][j][.] (masked t -> 0),
 *     c_h[t]     = sum_j a[h][j][t],
 * and the output row is c_h (NONE), sum over the G heads of group g
 * (GROUP_SUM), the max over those heads ([DELTA] key design 2, GROUP_MAX), or
 * one row summed over every query head of the layer (ALL_SUM: the per-layer
 * score [CLAA] buffers, "Three design decisions"; the KV groups are added in
 * order g = 0, 1, ..., so a caller keeping the last n layers writes each layer
 * straight into slot l mod n of an [n][s_ld] buffer).
 * Every one of the L columns is produced, so each GROUP_SUM row sums to W*G
 * (an ALL_SUM row to W*H_q).
 * With q_pos0 >= L - 1 every row sees all L keys (lookahead / decode queries).
 *
 * Q: bf16, element [h][j][c] at Q + h*q_head_stride + j*q_row_stride + c.
 * K: bf16, element [g][t][c] at K + g*k_head_stride + t*k_tok_stride + c.
 *    KV-head-major [H_kv][L][d_k] is the default; sequence-major [L][H_kv][d_k]
 *    is k_head_stride = d_k, k_tok_stride = H_kv * d_k.
 * S: float32, element [row][t] at S + row*s_ld + t; written (accumulate = 0)
 *    or added to (accumulate = 1).
 * Strides are in elements; 0 selects the contiguous default (W*d_k, d_k,
 * L*d_k, d_k, L).  Q/K pointers and strides must be 16-byte aligned.
 * Limits: d_k in {64, 128}; W*G <= 256 after padding each head's rows to
 * 4, 8, 16 or a multiple of 32 (every W*G <= 256 with W a power of two from
 * 4 up, e.g. G = 8 with W = 32 or G = 4 with W = 64; W = 12 with G = 20 pads
 * to 320 rows and is refused); otherwise KVS_EUNSUPPORTED.
 * More than 128 padded rows are scored in two row groups (each pass reads K
 * once per group).
 * The workspace holds per-split softmax statistics (and, for GROUP_MAX over
 * two row groups, every query head's column sums, 4 * H_q * L bytes; for
 * ALL_SUM each KV group's, 4 * H_kv * L bytes) and one 8-byte flag per KV head
 * and split; its size depends only on the arguments and its contents are
 * undefined on entry.  `phase` splits the call into its
 * statistics pass and its column-sum pass (each reads K once per row group).
 * With phase 0 and at most 128 padded rows, both passes run in one launch
 * when the device holds its whole grid at once (the flags order them); the
 * result is the same bit for bit as the two phases called one after the
 * other, and bit-identical from run to run.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t L, W, d_k, H_q, H_kv;
  int32_t heads;      /* KVS_HEADS_*                                        */
  int64_t q_pos0;     /* absolute position of window row 0, >= 0           */
  int64_t q_head_stride, q_row_stride;
  int64_t k_head_stride, k_tok_stride;
  int64_t s_ld;       /* row stride of S in floats, >= L                    */
  float scale;        /* logit scale, 0 => 1/sqrt(d_k); must be >= 0       */
  int32_t accumulate; /* 0: S = score, 1: S += score                        */
  int32_t phase;      /* 0: both passes; 1: row statistics only (fills ws);
                         2: column sums only, from a ws that a phase-1 call
                         with the same arguments filled                     */
} kvs_score_args;

size_t kvs_score_workspace(const kvs_score_args* a);
kvs_status kvs_score(const kvs_score_args* a, const void* Q, const void* K, float* S,
                     void* ws, size_t ws_bytes, void* stream);

/* kvs_wait_limit - bound, in microseconds, on how long a workgroup of a
 * one-launch form (kvs_score above, kvs_delta_pages below) waits for the
 * softmax statistics of the other workgroups of its KV head or sequence;
 * 2000 by default.  A workgroup still waiting at the bound (the device shared
 * with other work that holds back part of the grid) computes the missing
 * statistics itself, so the result is unchanged and only time is lost; 0
 * sends every workgroup that finds its group incomplete down that path at
 * once (for testing it).  A negative argument only queries.  Returns the
 * previous bound.  Process-wide; calls already enqueued keep the bound they
 * were enqueued with. */
int32_t kvs_wait_limit(int32_t microseconds);

/* kvs_score_noalloc - kvs_score without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results (bit for
 * bit) and errors as kvs_score; the workspace is a static 8 MiB array that
 * the library holds on every GPU it runs on until the process ends (its
 * device address is looked up on the first call on each device).  A call
 * whose kvs_score_workspace() exceeds 8 MiB returns KVS_ESCRATCH before
 * anything is enqueued (e.g. ALL_SUM needs 4 * H_kv * L bytes beside the
 * statistics).  Allocates nothing and frees nothing.  Every call on one GPU
 * shares that GPU's array and leaves its contents behind: a phase-2 call reads
 * what the last phase-1 call on that GPU wrote, so calls that overlap in time
 * on one GPU (other streams, other threads) race and must be serialized by
 * the caller. */
kvs_status kvs_score_noalloc(const kvs_score_args* a, const void* Q, const void* K, float* S,
                             void* stream);

/* ------------------------------------------------------------------------
 * kvs_score_raw - raw (pre-softmax) attention logits reduced over all heads.
 *
 * [CLAA] "Three representative token-ranking methods": GemFilter ranks the
 * prompt tokens by the logit of the last prompt token's query, scaled by
 * 1/sqrt(d_k) and summed over all heads (reduce = KVS_RED_SUM, W = 1).
 * Speculative Prefill, and the answer-informed oracle of "The oracle
 * construction" (use_softmax=False), take for each lookahead or answer query
 * the maximum raw logit over all layers and heads, then the mean over the
 * queries, then a 1-D average pooling with kernel 7: reduce = KVS_RED_MAX
 * once per layer into the same S with accumulate = KVS_ACC_MAX (the first
 * layer KVS_ACC_WRITE), then kvs_pool_pages over the W rows with head_reduce
 * KVS_RED_MEAN and pool KVS_RED_MEAN.
 * For every query row j < W and key t < L:
 *     R[j][t] = SUM or MAX over the H_q query heads h of
 *               scale * sum_c Q[h][j][c] * K[h / G][t][c]      (G = H_q / H_kv)
 * and S[j][t] (row stride s_ld) receives R (KVS_ACC_WRITE), S + R
 * (KVS_ACC_ADD) or max(S, R) (KVS_ACC_MAX).  These queries sit at or after the
 * last prompt token (q_pos0 >= L - 1), so every row sees every key; Q and K
 * hold finite values.
 * Q, K: layouts, strides, defaults and alignment as for kvs_score; scale 0
 * selects 1/sqrt(d_k).  S: float32, 4-byte aligned.
 * Limits (else KVS_EUNSUPPORTED): d_k in {64, 128}; W <= 32; the W rows of a
 * head padded to 8, 16 or 32 rows, G times that at most 128 rows per KV
 * head, and all KV heads' padded rows (each KV head's rounded up to a
 * multiple of 32) at most 256 (d_k = 128) or 896 (d_k = 64) rows.  K is read once, no workspace is used, and the result is
 * bit-identical from run to run.
 * ---------------------------------------------------------------------- */
#define KVS_ACC_WRITE 0
#define KVS_ACC_ADD 1
#define KVS_ACC_MAX 2
typedef struct {
  int32_t L, W, d_k, H_q, H_kv;
  int32_t reduce;     /* KVS_RED_SUM or KVS_RED_MAX over all query heads    */
  int64_t q_pos0;     /* absolute position of query row 0, >= L - 1         */
  int64_t q_head_stride, q_row_stride;
  int64_t k_head_stride, k_tok_stride;
  int64_t s_ld;       /* row stride of S in floats, >= L                    */
  float scale;        /* logit scale, 0 => 1/sqrt(d_k); must be >= 0       */
  int32_t accumulate; /* KVS_ACC_WRITE, KVS_ACC_ADD or KVS_ACC_MAX          */
} kvs_raw_args;

kvs_status kvs_score_raw(const kvs_raw_args* a, const void* Q, const void* K, float* S,
                         void* stream);

/* ------------------------------------------------------------------------
 * kvs_delta_pages - DELTA decode-time page sets for a batch of sequences.
 *
 * [DELTA] "Key design 2": at a Delta-layer, for the decode query of each
 * sequence b (context length L_b, the query at position L_b - 1 sees every
 * cached key), the token score is the maximum over the H_q heads of the
 * softmax attention, s_t = max_h softmax_t(scale * Q[b][h] . K_b[h / G][t]);
 * the page score is S_u = sum of s_t over the P tokens of page u (the last page
 * may be partial); rho_b = the top K_pages - L_recent of the pages before the
 * last L_recent by S_u, in ascending order, then the last min(L_recent,
 * pages) pages in ascending order, then -1 up to K_pages entries.  Page-score
 * ties go to the lower page.  "Key design 3": P = 16, K_pages = 64,
 * L_recent = 8.
 * Q: bf16 [B][H_q][d_k], contiguous.  K: device array of B device pointers,
 * each 16-byte aligned; sequence b's keys are bf16, element [g][t][c] at
 * K[b] + g * k_head_stride +
 * t * k_tok_stride + c (k_head_stride 0 selects L_b * d_k, k_tok_stride 0
 * selects d_k).  L: device int32 [B]; each length is clamped to [0, L_max]
 * (a sequence of length 0 gets an all -1 row).  rho: int32 [B][K_pages].
 * page_scores: float32 [B][ceil(L_max / P)] receiving S_u for the pages of
 * each sequence (other entries untouched), or NULL.
 * Workspace: kvs_delta_workspace bytes, 16-byte aligned, contents undefined
 * on entry and return (the logits of every head, 4 * H_q bytes per cached
 * token, per-chunk softmax statistics, an 8-byte flag per chunk and an 8-byte
 * word per page).  With
 * H_q <= 32, when the logits of the batch fit in registers (B * L_max up to
 * about 256K tokens) and the device holds the whole grid at once, one launch
 * computes the page scores and rho without writing the logits (the flags
 * and the launch-tagged page words order its workgroups); the result is the
 * same bit for bit.
 * Limits (else KVS_EUNSUPPORTED): d_k in {64, 128}; H_q <= 128; P divides
 * 512; ceil(L_max / P) <= 16384.  K is read once; the result is
 * bit-identical from run to run.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t B;          /* sequences                                            */
  int32_t d_k, H_q, H_kv;
  int32_t P;          /* tokens per page                                      */
  int32_t K_pages;    /* pages in each rho row, >= L_recent                   */
  int32_t L_recent;   /* most recent pages always kept, >= 0                  */
  int32_t L_max;      /* bound on every context length, >= 1                  */
  int64_t k_head_stride, k_tok_stride;
  float scale;        /* logit scale, 0 => 1/sqrt(d_k); must be >= 0          */
} kvs_delta_args;

size_t kvs_delta_workspace(const kvs_delta_args* a);
kvs_status kvs_delta_pages(const kvs_delta_args* a, const void* Q, const void* const* K,
                           const int32_t* L, int32_t* rho, float* page_scores, void* ws,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_gather_kv - compact copy of the selected tokens, pages or blocks.
 *
 * [CLAA] "Complete flow and cost": each layer keeps its KV cache for the
 * indices top-k chose from that layer's scores, gathered from K and V.
 * [CompactAttention] "Core method" and its execution ablation: the explicit
 * copy of the selected blocks, next to the page-table path of
 * kvs_block_union_pagetable.  [DELTA] "Key design 3": whole pages.
 * For KV head g < H, its list is indices[indptr[g] .. indptr[g+1]) (at most n
 * entries) when indptr is given, else indices[g * idx_ld .. g * idx_ld + n)
 * (idx_ld = 0: one list shared by every head, as a CLAA layer keeps).  Entry e
 * with value i selects the unit tokens [i * unit, i * unit + unit); output row
 * e * unit + o of head g holds token i * unit + o.  Negative entries, tokens
 * at or past L, and rows past the head's list are written as zeros.
 * K, V: bf16 (any 2-byte type: bits are copied), element [g][t][c] at
 * X + g * head_stride + t * tok_stride + c (0, 0 select [H][L][d_k]).
 * K_out, V_out: [H][n * unit][d_k] contiguous.  V and V_out may be NULL.
 * Limits: d_k a multiple of 8 and at most 2048; pointers and strides 16-byte
 * aligned (else KVS_EINVAL).  The indices and indptr are device int32 arrays.
 * ---------------------------------------------------------------------- */
kvs_status kvs_gather_kv(const void* K, const void* V, int32_t H, int32_t L, int32_t d_k,
                         int64_t head_stride, int64_t tok_stride, const int32_t* indices,
                         int64_t idx_ld, const int32_t* indptr, int32_t n, int32_t unit,
                         void* K_out, void* V_out, void* stream);

/* ------------------------------------------------------------------------
 * kvs_pool_pages - head reduction, 1-D pooling, page aggregation.
 *
 * Input S float32 [H][n] with row stride ld (>= n).  In this order:
 *  1. head_reduce NONE keeps the H rows; SUM / MAX / MEAN folds them into
 *     one row ([DELTA] key design 2: max over heads; [CLAA] Speculative
 *     Prefill: mean over the lookahead queries).  H' = 1 or H rows remain;
 *     MEAN divides the float32 sum by H.
 *  2. pool NONE / MAX / MEAN over [t - r, t + r] clipped to [0, n),
 *     r = (pool_k - 1) / 2, pool_k odd; MEAN divides by the in-range count
 *     ([CLAA] 1-D pooling, kernel 7).
 *  3. if P > 0: page u covers tokens [u*P, min(u*P + P, n)); page_reduce
 *     SUM or MAX ([DELTA] page score; [ClusterAttn] block max) and page_arg =
 *     lowest index attaining the page maximum.
 * Outputs (contiguous, float32 / int32): pooled [H'][n] (may be NULL when
 * P > 0), page [H'][ceil(n/P)] and page_arg [H'][ceil(n/P)] (each may be
 * NULL).  Sums are taken left to right in float32.
 * ---------------------------------------------------------------------- */
kvs_status kvs_pool_pages(const float* S, int32_t H, int32_t n, int64_t ld,
                          int32_t head_reduce, int32_t pool, int32_t pool_k,
                          int32_t P, int32_t page_reduce,
                          float* pooled, float* page, int32_t* page_arg, void* stream);

/* ------------------------------------------------------------------------
 * kvs_topk - per-row top-`budget` selection with a forced suffix.
 *
 * [CLAA] topk(scores, keep_rate) over candidates [0, n) of each of the H rows
 * of S (row stride ld >= n).  Order: priority descending (when `priority`,
 * uint8 [H][n] contiguous, is given; nonzero = 1), value descending, index
 * ascending: ties go to the lower index.  -0.0 ranks equal to +0.0; NaN ranks
 * below every number.  The output row idx[h][0 .. budget + n_forced) lists the
 * chosen indices in ascending order (original positions preserved), followed
 * by n, n+1, ..., n + n_forced - 1 ([ClusterAttn] window appended; [DELTA]
 * recency pages).  The result is unique for a given input.
 * val, when not NULL, float32 [H][budget + n_forced] (contiguous) receives the
 * kept scores in the order of idx: val[h][e] = S[h][idx[h][e]] for e < budget
 * (a bit copy, [CLAA] topk returns the values with the indices) and NaN for
 * the forced suffix, whose positions lie outside the candidate range.
 * 0 <= budget <= n, H <= 65535.
 *
 * Workspace: kvs_topk_workspace bytes (0 when n <= 16384: rows that short
 * finish in one kernel), 16-byte aligned, owned by the caller, contents
 * undefined on entry and on return.  It holds the per-part candidates of the
 * two-stage select or, for rows whose candidates would not fit one merge
 * (more than 16384 of them: a large budget over several parts of 16384), the
 * rows' per-part histograms and counts (and ranking keys); calls that share
 * one must not overlap in time.  Those wide rows run in one launch when the
 * device holds its whole grid at once, their parts exchanging histograms
 * (kvs_wait_limit bounds their waits), else in one launch per phase; the
 * result is the same.
 * ---------------------------------------------------------------------- */
size_t kvs_topk_workspace(int32_t H, int32_t n, int32_t budget);
kvs_status kvs_topk(const float* S, int32_t H, int32_t n, int64_t ld, int32_t budget,
                    const uint8_t* priority, int32_t n_forced, int32_t* idx, float* val,
                    void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_select - pooled or cluster-prioritised top-k in one call.
 *
 * The same selection as kvs_topk (order, ties, forced suffix, ascending
 * output, workspace contract), ranked on a transform of the scores that is
 * computed on the fly (kept only in the workspace, for rows that take the
 * multi-part path):
 *  pool = KVS_RED_MAX / KVS_RED_MEAN: value = max / mean of S over
 *    [t - r, t + r] clipped to [0, n), r = (pool_k - 1) / 2 ([CLAA] oracle
 *    construction: 1-D pooling of the token scores, kernel 7, before top-k).
 *    MAX is NaN when a term is NaN; MEAN sums left to right in float32.
 *  cluster_P > 0: priority = 1 for tokens within cluster_r of the argmax
 *    (lowest index) of a page of cluster_P tokens whose maximum is
 *    >= cluster_theta; a page holding a NaN has no centre ([ClusterAttn]
 *    method details: block-max centres, threshold, gathered neighbourhood,
 *    then the best remaining tokens).  Values are the scores themselves.
 * Pooling and clustering are exclusive (KVS_EUNSUPPORTED otherwise).
 * Limits: pool_k odd, (pool_k - 1) / 2 <= KVS_SELECT_HALO_MAX;
 * cluster_P + cluster_r <= KVS_SELECT_HALO_MAX; cluster_theta not NaN.
 * ---------------------------------------------------------------------- */
#define KVS_SELECT_HALO_MAX 1024
typedef struct kvs_select_args {
  int32_t budget;        /* tokens kept per row, 0 <= budget <= n            */
  int32_t n_forced;      /* suffix n .. n + n_forced - 1 appended per row    */
  int32_t pool;          /* KVS_RED_NONE, KVS_RED_MAX or KVS_RED_MEAN        */
  int32_t pool_k;        /* odd pooling window (ignored for KVS_RED_NONE)    */
  int32_t cluster_P;     /* 0: no clustering; > 0: page size of the centres  */
  float cluster_theta;   /* centre threshold on the page maximum             */
  int32_t cluster_r;     /* gather radius around each centre, >= 0           */
} kvs_select_args;

size_t kvs_select_workspace(int32_t H, int32_t n, int32_t budget);
kvs_status kvs_select(const float* S, int32_t H, int32_t n, int64_t ld, const kvs_select_args* a,
                      int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_block_union_pagetable - per-group KV page table from a 2-D block mask.
 *
 * [CompactAttention] M uint8 [H_q][n_qb][n_kvb] (nonzero = selected).
 * Q-block union  Mb[h][j] = OR_i M[h][i][j];  intra-group union over the
 * sub_group consecutive query heads of subgroup s (inside one KV group;
 * sub_group = 0 selects G = H_q / H_kv):  Gs[s][j] = OR_h Mb[h][j].
 * T_s = { j : Gs[s][j] } ascending.  n_groups = H_q / sub_group.
 * kv_indptr int32 [n_groups + 1] = exclusive prefix sum of |T_s|;
 * kv_indices int32 [capacity >= n_groups * n_kvb] holds T_0, T_1, ... packed.
 * The table is the smallest one covering every selected block.
 * ---------------------------------------------------------------------- */
size_t kvs_block_union_workspace(int32_t H_q, int32_t H_kv, int32_t sub_group, int32_t n_kvb);
kvs_status kvs_block_union_pagetable(const uint8_t* M, int32_t H_q, int32_t H_kv, int32_t sub_group,
                                     int32_t n_qb, int32_t n_kvb, int32_t* kv_indptr,
                                     int32_t* kv_indices, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_token_pagetable - per-group KV page table from kept token positions.
 *
 * [CompactAttention] "Method step details": a paged attention kernel reads a
 * group's KV through a page table kv_indptr / kv_indices, built on the GPU;
 * "Technical novelty": the smallest table covering the selection.  [DELTA]
 * "Key design 3": whole pages of P tokens.  This turns token lists (kvs_topk
 * or kvs_select rows, window included) into such tables.
 * idx int32 [H][n] with row stride idx_ld (0 selects n): row h's kept token
 * positions, any order, duplicates allowed; entries < 0 or >= n_pages * P
 * name no page.  Group s covers rows s * rows_per_group ... (s + 1) *
 * rows_per_group - 1 (rows_per_group divides H; 1: one table per row, e.g.
 * per KV head).  T_s = { i / P : i an entry of the group } ascending;
 * kv_indptr int32 [H / rows_per_group + 1] = exclusive prefix sum of |T_s|;
 * kv_indices int32 [capacity >= (H / rows_per_group) * n_pages] holds T_0,
 * T_1, ... packed.  Workspace: kvs_token_pagetable_workspace bytes, 16-byte
 * aligned (a page mask per group and the union staging), contents undefined
 * on entry; nothing needs clearing.  Limits: n_pages <= 2^26 (else
 * KVS_EUNSUPPORTED), n_pages * P < 2^31.
 * ---------------------------------------------------------------------- */
size_t kvs_token_pagetable_workspace(int32_t H, int32_t rows_per_group, int32_t n_pages);
kvs_status kvs_token_pagetable(const int32_t* idx, int32_t H, int32_t n, int64_t idx_ld,
                               int32_t rows_per_group, int32_t P, int32_t n_pages,
                               int32_t* kv_indptr, int32_t* kv_indices, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * kvs_aggregate_layers - fold one layer's scores into a cross-layer total.
 *
 * s[t] = sum over the H rows of S[h][t] (row stride ld >= n), then
 *   SUM_L1: acc[t] (=|+=) s[t] / sum_t' |s[t']|  ([LookaheadKV] L1 norm),
 *   MAX:    acc[t] = max(acc[t], s[t])           ([CLAA] Eq. 6).
 * first_layer = 1 overwrites acc (float32 [n]) instead of combining.
 * The L1 norm is accumulated in float64 in a fixed order.
 * ---------------------------------------------------------------------- */
size_t kvs_aggregate_workspace(int32_t n);
kvs_status kvs_aggregate_layers(float* acc, const float* S, int32_t H, int32_t n, int64_t ld,
                                int32_t mode, int32_t first_layer, void* ws, size_t ws_bytes,
                                void* stream);

/* ------------------------------------------------------------------------
 * kvs_cluster_priority - density-clustering priority mask.
 *
 * [ClusterAttn] method details: centres are the block-level max indices
 * page_arg[h][u] whose block maximum page[h][u] >= theta; every token within
 * r of a centre (|t - c| <= r, t in [0, n)) gets priority[h][t] = 1, else 0.
 * page / page_arg [H][n_pages] come from kvs_pool_pages with page size P:
 * page_arg[h][u] must lie in [u*P, min(u*P + P, n)) (a centre is only looked
 * for in the pages that can hold a token within r of t).
 * ---------------------------------------------------------------------- */
kvs_status kvs_cluster_priority(const float* page, const int32_t* page_arg, int32_t H,
                                int32_t n_pages, int32_t P, int32_t n, float theta, int32_t r,
                                uint8_t* priority, void* stream);

/* ------------------------------------------------------------------------
 * kvs_block_select - block mask of a prefill chunk from mean-pooled logits.
 *
 * Chunk queries Qc bf16 [H_q][Lq][d_k] at positions q_pos0 .. q_pos0 + Lq - 1
 * against keys K bf16 [H_kv][L][d_k] (strides as in kvs_score).  Kb = mean of
 * each `block` keys, Qb = mean of each `block` chunk rows (last blocks may be
 * partial); query block i sees KV block j when j*block <= its last position.
 * Logits scale * Qb . Kb, softmax over the visible blocks, blocks ordered by
 * (probability desc, j asc); M[h][i][j] = 1 while the mass ranked strictly
 * before block j is < p_mass.  Output M uint8 [H_q][n_qb][n_kvb].
 * Stands in for the pages' learned / threshold selectors ([CompactAttention]
 * step 1) with a training-free top-p rule.  n_kvb <= 4096.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t Lq, L, d_k, H_q, H_kv, block;
  int64_t q_pos0;
  int64_t q_head_stride, q_row_stride;
  int64_t k_head_stride, k_tok_stride;
  float scale;  /* 0 => 1/sqrt(d_k) */
  float p_mass; /* in (0, 1]          */
} kvs_block_select_args;

size_t kvs_block_select_workspace(const kvs_block_select_args* a);
kvs_status kvs_block_select(const kvs_block_select_args* a, const void* Qc, const void* K,
                            uint8_t* M, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvs_block_select_cached - kvs_block_select with key-block means carried
 * from one prefill chunk to the next.
 *
 * [CompactAttention] "Core method": each chunk scores its query blocks against
 * the whole accumulated KV cache; the key blocks that earlier chunks completed
 * do not change, so their means need not be recomputed.  Kb is a caller-owned
 * float32 cache [H_kv][kb_cap][d_k] (16-byte aligned, kb_cap >= ceil(L /
 * block)); its first n_cached blocks of every KV head must hold the means of
 * those complete blocks of the same K (as an earlier call left them), and
 * n_cached <= floor(L / block).  The call writes the means of blocks
 * n_cached .. ceil(L / block) - 1 into Kb and otherwise computes exactly what
 * kvs_block_select computes (bit-identical M): a chunk reads only the keys of
 * its new blocks.  After the call, floor(L / block) blocks of Kb are complete
 * for the next chunk.  Workspace as for kvs_block_select.
 * ---------------------------------------------------------------------- */
kvs_status kvs_block_select_cached(const kvs_block_select_args* a, const void* Qc, const void* K,
                                   float* Kb, int32_t kb_cap, int32_t n_cached, uint8_t* M,
                                   void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H */

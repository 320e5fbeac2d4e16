// Internal declarations shared by the host-side API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvs.h"

namespace kvs {

constexpr size_t kWsAlign = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- score
// Rows of one KV group: the W window rows of each of the G query heads are
// padded to `head_rows` (4, 8, 16 or a multiple of 32) and the group to a
// multiple of 32 rows (`rows_pad`, at most 256); padding rows are masked out.
// The rows are processed in one or two row groups of at most 128 rows.
struct ScorePlan {
  int head_rows;
  int rows_pad;     // multiple of 32, <= 256
  int n_tiles;      // ceil(L / 32)
  int n_split;      // splits of the key range per KV head
  int tiles_per_split;
  int head_batch;   // KV heads per (pass 1, pass 2) round
  int reverse;      // pass 2 visits tiles in the reverse of pass 1's order
  int n_groups;     // row groups (1 or 2)
  int grp_row0[2];  // first padded row of each group
  int grp_rows[2];  // padded rows of each group (multiple of 32, <= 128)
  int grp_h0[2], grp_h1[2];   // query heads of each group
  size_t ws_stats;  // bytes of per-split (max, sum) pairs
  size_t ws_heads;  // bytes of per-head column sums (GROUP_MAX over two groups)
  size_t ws_flags;  // bytes of the per-(KV head, split) flags of a fused launch
  size_t ws_total;
};

struct ScoreLaunch {
  const uint16_t* Q;
  const uint16_t* K;
  float* S;
  float2* stats;  // [H_kv][rows_pad][n_split]
  float* head_rows_ws;   // [H_q][L] per-head column sums (GROUP_MAX over two row groups)
  uint64_t* flags;       // [H_kv][n_split] flags of the fused launch (see score.hip)
  int64_t qhs, qrs, khs, kts, s_ld;
  int64_t q_pos0;
  int L, W, G, H_kv, d_k, heads, accumulate, phase;
  float c;        // scale * log2(e)
};

kvs_status score_plan(const kvs_score_args* a, ScorePlan* plan);
// One-launch forms (grid.hip, grid_sync.h): the workgroups of kernel fn
// (of `threads` threads) the current device holds at once (-1: unknown), a
// fresh launch tag, and the wait bound in 100 MHz ticks; wait_limit sets that
// bound (microseconds, < 0: unchanged) and returns the previous one.
int grid_capacity(const void* fn, int threads);
uint64_t grid_epoch();
int64_t grid_wait_ticks();
int32_t wait_limit(int32_t us);
kvs_status score_run(const ScorePlan& plan, const ScoreLaunch& p, hipStream_t stream);

// Raw logits reduced over all heads (kvs_score_raw); head_rows pads each
// head's W rows as for the softmax scores.
struct RawLaunch {
  const uint16_t* Q;
  const uint16_t* K;
  float* S;
  int64_t qhs, qrs, khs, kts, s_ld;
  int L, W, G, H_kv, d_k, head_rows, reduce_max, accumulate;
  float scale;
};
kvs_status score_raw_run(const RawLaunch& p, hipStream_t stream);

// DELTA decode-time page sets for a batch of sequences (kvs_delta_pages).
struct DeltaLaunch {
  const uint16_t* Q;               // [B][H_q][d_k]
  const uint16_t* const* K;        // [B] device pointers
  const int32_t* L;                // [B] context lengths (clamped to [0, L_max])
  float* x2;                       // [B][H_q][x2_ld] logits in log2 units
  float2* cstats;                  // [B][n_chunk][H_q] per-chunk (max, sum of exp2)
  float* S;                        // [B][n_pages_max] page scores
  int32_t* rho;                    // [B][K_pages]
  uint64_t* flags;                 // [B][n_chunk] one-launch form: statistics published
  uint64_t* pwords;                // [B][n_pages_max] one-launch form: page scores tagged
                                   //   with the launch (tag << 32 | float bits)
  uint64_t epoch;                  // set by the launcher
  int64_t wait_ticks;              // set by the launcher
  int64_t khs, kts;                // khs 0: L_b * d_k
  int B, H_q, H_kv, G, d_k, P, K_pages, L_recent, L_max, n_chunk, n_pages_max;
  int chunk;                       // keys per logits workgroup, a multiple of 128
  int64_t x2_ld;                   // row stride of x2 (L_max rounded up to 32, plus 32)
  float c;                         // scale * log2(e)
};
// Keys per logits workgroup for a batch: enough workgroups for every CU,
// each streaming as long a run of keys as that allows.
int delta_chunk(int B, int L_max);
// Page scores; *selected = 1 when the same launch also wrote rho.
kvs_status delta_scores_run(const DeltaLaunch& p, hipStream_t stream, int* selected);
kvs_status delta_topk_run(const DeltaLaunch& p, hipStream_t stream);

// ---------------------------------------------------------------- others
kvs_status pool_pages_run(const float* S, int H, int n, int64_t ld, int head_reduce, int pool,
                          int pool_k, int P, int page_reduce, float* pooled, float* page,
                          int32_t* page_arg, hipStream_t stream);

kvs_status cluster_priority_run(const float* page, const int32_t* page_arg, int H, int n_pages,
                                int P, int n, float theta, int r, uint8_t* prio,
                                hipStream_t stream);

size_t aggregate_ws_bytes(int n);
kvs_status aggregate_run(float* acc, const float* S, int H, int n, int64_t ld, int mode, int first,
                         void* ws, hipStream_t stream);

// Top-k selection; the key transform is one of: none (optionally with a
// caller priority array), pooling, or the cluster priority (cluster_P > 0).
constexpr int kSelHaloMax = KVS_SELECT_HALO_MAX;
struct SelectCall {
  const float* S;
  int H, n;
  int64_t ld;
  int budget, n_forced;
  const uint8_t* priority;
  int pool, pool_k;
  int cluster_P;
  float cluster_theta;
  int cluster_r;
  int32_t* idx;
  void* ws;
  float* val;   // kvs_topk's kept scores, or null
};
size_t topk_ws_bytes(int H, int n, int budget);
kvs_status select_run(const SelectCall& c, hipStream_t stream);

// KV gather (kvs_gather_kv).
struct GatherLaunch {
  const uint16_t* K;
  const uint16_t* V;        // may be null
  uint16_t* K_out;
  uint16_t* V_out;
  const int32_t* indices;
  const int32_t* indptr;    // may be null
  int64_t idx_ld, khs, kts;
  int H, L, d_k, n, unit;
};
kvs_status gather_run(const GatherLaunch& p, hipStream_t stream);

size_t union_ws_bytes(int H_q, int H_kv, int sub_group, int n_kvb);
kvs_status union_run(const uint8_t* M, int H_q, int H_kv, int sub_group, int n_qb, int n_kvb,
                     int32_t* indptr, int32_t* indices, void* ws, hipStream_t stream);

// Per-group page tables from token lists (kvs_token_pagetable).
size_t token_pagetable_ws_bytes(int H, int rows_per_group, int n_pages);
kvs_status token_pagetable_run(const int32_t* idx, int H, int n, int64_t idx_ld,
                               int rows_per_group, int P, int n_pages, int32_t* indptr,
                               int32_t* indices, void* ws, hipStream_t stream);

struct BlockPlan {
  int n_qb, n_kvb;
  size_t ws_kb, ws_qb, ws_logit, ws_total;
};
kvs_status block_plan(const kvs_block_select_args* a, BlockPlan* plan);
// Kb null: key-block means go to the workspace.  Else Kb is a caller cache of
// kb_ld blocks per KV head whose first n_cached blocks are already valid.
kvs_status block_select_run(const kvs_block_select_args* a, const BlockPlan& plan,
                            const uint16_t* Qc, const uint16_t* K, uint8_t* M, void* ws,
                            float* Kb, int kb_ld, int n_cached, hipStream_t stream);

}  // namespace kvs

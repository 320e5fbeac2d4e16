// Chunked-prefill block selection (kvs_block_select) and the block union that
// lowers a per-head 2-D block mask to per-group KV page tables
// (kvs_block_union_pagetable).
//
// The CompactAttention page ("Method step details") takes a binary mask
// M[h][i][j] over (query block, KV block) pairs, forms the Q-block union
// OR_i M[h][i][j], then the union over the heads of each (sub)group, and hands
// the surviving KV blocks to a paged attention kernel as kv_indptr /
// kv_indices.  The page's own selectors are a learned gate and a threshold
// method; the selector here is a training-free stand-in over the same inputs:
// mean-pooled query and key blocks, softmax over the visible block logits,
// keep blocks up to 0.9 cumulative mass.
//
// The page table is built entirely on the GPU: no count travels to the host.
#include <math.h>

#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxKvb = 4096;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ block means
// out[head][blk][d] (n_blk blocks per head) = mean of rows [blk*block,
// min(L, blk*block + block)) of in[head][row][d] for blocks blk0, blk0 + 1,
// ...; rows are summed in a fixed order, so a block's mean does not depend on
// the call that computed it.  One workgroup per (block, head); a thread loads
// 8 bf16 of one row at a time.
__global__ __launch_bounds__(kThreads) void block_mean_kernel(const uint16_t* __restrict__ in,
                                                              int64_t hs, int64_t rs, int L, int d_k,
                                                              int block, int n_blk, int blk0,
                                                              float* __restrict__ out) {
  __shared__ float part[kThreads / 8][128 + 4];
  const int blk = blk0 + blockIdx.x, head = blockIdx.y;
  const int tpr = d_k / 8;                 // threads per row
  const int rows_per = kThreads / tpr;     // rows covered per step
  const int rsub = threadIdx.x / tpr, dc = (threadIdx.x % tpr) * 8;
  const int r0 = blk * block, r1 = min(L, r0 + block);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0 + rsub; r < r1; r += rows_per) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(in + (int64_t)head * hs + (int64_t)r * rs + dc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(v[e] << 16);
      acc[2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rsub][dc + e] = acc[e];
  __syncthreads();
  const float inv_cnt = 1.0f / (float)(r1 - r0);
  for (int d = threadIdx.x; d < d_k; d += kThreads) {
    float s = 0.f;
    for (int q = 0; q < rows_per; ++q) s += part[q][d];
    out[((int64_t)head * n_blk + blk) * d_k + d] = s * inv_cnt;
  }
}

// ------------------------------------------------------------------ block logits
// logit[h][i][j] = scale * Qb[h][i] . Kb[g][j] for every query block i of the
// G heads of KV group g and every key block j: a small fp32 GEMM per group on
// the matrix cores (v_mfma_f32_32x32x2_f32: fp32 products, fp32 sums).  A
// workgroup covers 64 rows (head, query block) x 64 key blocks, one 32 x 32
// block per wave.  Step m of the contraction takes dimension m from the lanes
// of the first half-wave and m + d/2 from the second, so a lane's operands
// for consecutive steps are consecutive floats of its row: 16-byte loads
// straight from global memory (L2-resident block means), no LDS.
constexpr int kLt = 64;   // tile edge
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kThreads) void block_logits_kernel(
    const float* __restrict__ Qb, const float* __restrict__ Kb, int kb_ld, int G, int n_qb,
    int n_kvb, int d_k, float scale, float* __restrict__ logit) {
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = G * n_qb;   // row r = (head g*G + r / n_qb, query block r % n_qb)
  const int r0 = blockIdx.z * kLt + 32 * (wave >> 1), j0 = blockIdx.x * kLt + 32 * (wave & 1);
  const int half = d_k / 2;
  const int ra = min(r0 + (lane & 31), rows - 1), jb = min(j0 + (lane & 31), n_kvb - 1);
  const float* qa = Qb + ((int64_t)g * rows + ra) * d_k + half * (lane >> 5);
  const float* kb = Kb + ((int64_t)g * kb_ld + jb) * d_k + half * (lane >> 5);
  f32x16_t acc = {};
  for (int m0 = 0; m0 < half; m0 += 16) {
    float4 av[4], bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[q] = *reinterpret_cast<const float4*>(qa + m0 + 4 * q);
      bv[q] = *reinterpret_cast<const float4*>(kb + m0 + 4 * q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q].x, bv[q].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q].y, bv[q].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q].z, bv[q].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q].w, bv[q].w, acc, 0, 0, 0);
    }
  }
  // accumulator i of lane l: row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
  const int j = j0 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + 8 * (i / 4) + 4 * (lane >> 5) + (i % 4);
    if (r < rows && j < n_kvb) {
      const int h = g * G + r / n_qb, qi = r % n_qb;
      logit[((int64_t)h * n_qb + qi) * n_kvb + j] = scale * acc[i];
    }
  }
}

__device__ __forceinline__ uint32_t ord_pos(float p) { return __float_as_uint(p) | 0x80000000u; }

// ------------------------------------------------------------------ top-p per (head, query block)
__global__ __launch_bounds__(kThreads) void block_topp_kernel(
    const float* __restrict__ logit, int n_qb, int n_kvb, int block, int Lq,
    int64_t q_pos0, float p_mass, uint8_t* __restrict__ M) {
  __shared__ uint64_t keys[2048];
  __shared__ float val[kMaxKvb];
  __shared__ float red[kThreads];
  const int i = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t last_row = min((int64_t)(i + 1) * block, (int64_t)Lq) - 1;
  const int64_t end_pos = q_pos0 + last_row;
  // 1. logits of the visible blocks
  const float* lr = logit + ((int64_t)h * n_qb + i) * n_kvb;
  for (int j = tid; j < n_kvb; j += kThreads)
    val[j] = (int64_t)j * block <= end_pos ? lr[j] : -__builtin_inff();
  __syncthreads();
  float mloc = -__builtin_inff();
  for (int j = tid; j < n_kvb; j += kThreads) mloc = fmaxf(mloc, val[j]);
  red[tid] = mloc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float mx = red[0];
  __syncthreads();
  // 2. softmax numerators and their sum (fixed tree order)
  float sloc = 0.f;
  for (int j = tid; j < n_kvb; j += kThreads) {
    const float e = val[j] == -__builtin_inff() ? 0.f : expf(val[j] - mx);
    val[j] = e;
    sloc += e;
  }
  red[tid] = sloc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float inv_z = 1.0f / red[0];
  __syncthreads();
  // 3. the kept blocks are a prefix of the order (probability desc, j asc): a
  // block is kept while the mass ranked strictly before it is < p_mass.  The
  // prefix ends at the block K* where the running mass first reaches p_mass;
  // K* is found by a radix select over the 44-bit key (probability bits, then
  // 4095 - j) with per-digit histograms of mass instead of counts.  Masses are
  // fixed point (2^-40 units) summed with integer atomics: exact and
  // independent of the order of the additions.
  uint64_t* hm = keys;   // 2048-bin mass histogram (the key array's first 16 KiB)
  const uint64_t need0 = (uint64_t)((double)p_mass * 1099511627776.0);   // 2^40
  uint64_t prefix = 0, need = need0;
  bool all = false;      // the whole order stays below p_mass: keep every visible block
  for (int pass = 0; pass < 4 && !all; ++pass) {
    const int shift = 33 - 11 * pass;
    const uint64_t pmask = pass == 0 ? 0ull : (~0ull << (shift + 11)) & ((1ull << 44) - 1);
    for (int b = tid; b < 2048; b += kThreads) hm[b] = 0ull;
    __syncthreads();
    for (int j = tid; j < n_kvb; j += kThreads) {
      const float p = val[j] * inv_z;
      const uint64_t key = ((uint64_t)ord_pos(p) << 12) | (uint64_t)(4095 - j);
      if ((key & pmask) == prefix)
        atomicAdd(reinterpret_cast<unsigned long long*>(&hm[(key >> shift) & 2047u]),
                  (unsigned long long)(p * 1099511627776.0f));
    }
    __syncthreads();
    // thread t owns bins [2047 - 8t - 7, 2047 - 8t]: mass above it, then its crossing bin
    uint64_t c[8], ls = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[u] = hm[2047 - 8 * tid - u];
      ls += c[u];
    }
    // exclusive prefix of the per-thread masses over the workgroup (waves, then LDS)
    const int lane = tid & 63, wave = tid >> 6;
    uint64_t inc = ls;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t v = __shfl_up(inc, off);
      if (lane >= off) inc += v;
    }
    __shared__ uint64_t wsum[kThreads / 64];
    __shared__ uint64_t sel_prefix, sel_need;
    __shared__ int found;
    if (lane == 63) wsum[wave] = inc;
    if (tid == 0) found = 0;
    __syncthreads();
    uint64_t above = inc - ls;
    for (int w = 0; w < wave; ++w) above += wsum[w];
    if (above < need && need <= above + ls) {
      uint64_t cum = above;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (cum < need && need <= cum + c[u]) {
          sel_prefix = prefix | ((uint64_t)(2047 - 8 * tid - u) << shift);
          sel_need = need - cum;
          found = 1;
        }
        cum += c[u];
      }
    }
    __syncthreads();
    if (!found) {
      all = true;   // the prefix's whole mass is below need
    } else {
      prefix = sel_prefix;
      need = sel_need;
    }
    __syncthreads();
  }
  // 4. keep the visible blocks at or above K* (every visible block when `all`)
  uint8_t* mrow = M + ((int64_t)h * n_qb + i) * n_kvb;
  for (int j = tid; j < n_kvb; j += kThreads) {
    const float p = val[j] * inv_z;
    const uint64_t key = ((uint64_t)ord_pos(p) << 12) | (uint64_t)(4095 - j);
    const bool visible = (int64_t)j * block <= end_pos;
    mrow[j] = (visible && (all || key >= prefix)) ? 1 : 0;
  }
}

// ------------------------------------------------------------------ union
// One workgroup per subgroup: OR over its heads and query blocks, then an
// ascending compaction of the set KV blocks into staging.  Thread t owns the
// 16 KV blocks [16t, 16t + 16) (n_kvb <= 4096): it reads them from every mask
// row it ORs (one 16-byte load per row when the rows are 16-byte aligned), all
// rows' loads independent of each other.
__global__ __launch_bounds__(kThreads) void union_group_kernel(const uint8_t* __restrict__ M,
                                                               int sg, int n_qb, int n_kvb,
                                                               int32_t* __restrict__ staging,
                                                               int32_t* __restrict__ counts) {
  __shared__ uint32_t wc[kThreads / 64];
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = 16 * tid;
  const int nrows = sg * n_qb;
  const uint8_t* base = M + (int64_t)s * sg * n_qb * n_kvb;
  uint32_t bits = 0;
  if (j0 < n_kvb) {
    if (n_kvb % 16 == 0 && ((uintptr_t)M & 15u) == 0) {
      u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 8
      for (int r = 0; r < nrows; ++r)
        acc |= *reinterpret_cast<const u32x4*>(base + (int64_t)r * n_kvb + j0);
#pragma unroll
      for (int e = 0; e < 16; ++e) bits |= ((acc[e / 4] >> (8 * (e % 4))) & 0xffu) ? (1u << e) : 0u;
    } else {
      for (int r = 0; r < nrows; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (j0 + e < n_kvb && base[(int64_t)r * n_kvb + j0 + e]) bits |= 1u << e;
    }
  }
  // exclusive prefix of the per-thread counts: this thread's first output slot
  uint32_t c = __popc(bits);
  uint32_t inc = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(inc, off);
    if (lane >= off) inc += u;
  }
  if (lane == 63) wc[wave] = inc;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    before += w < wave ? wc[w] : 0u;
    total += wc[w];
  }
  uint32_t pos = before + inc - c;
  int32_t* st = staging + (int64_t)s * n_kvb;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if ((bits >> e) & 1u) st[pos++] = j0 + e;
  if (tid == 0) counts[s] = (int32_t)total;
}

__global__ __launch_bounds__(kThreads) void union_pack_kernel(const int32_t* __restrict__ staging,
                                                              const int32_t* __restrict__ counts,
                                                              int n_groups, int n_kvb,
                                                              int32_t* __restrict__ indptr,
                                                              int32_t* __restrict__ indices) {
  int off = 0;
  for (int s = 0; s < n_groups; ++s) {
    const int c = counts[s];
    if (threadIdx.x == 0) indptr[s] = off;
    for (int x = threadIdx.x; x < c; x += kThreads) indices[off + x] = staging[(int64_t)s * n_kvb + x];
    off += c;
  }
  if (threadIdx.x == 0) indptr[n_groups] = off;
}

}  // namespace

kvs_status block_plan(const kvs_block_select_args* a, BlockPlan* pl) {
  pl->n_qb = (a->Lq + a->block - 1) / a->block;
  pl->n_kvb = (a->L + a->block - 1) / a->block;
  if (pl->n_kvb > kMaxKvb) return KVS_EUNSUPPORTED;
  pl->ws_kb = align_up((size_t)a->H_kv * pl->n_kvb * a->d_k * sizeof(float), kWsAlign);
  pl->ws_qb = align_up((size_t)a->H_q * pl->n_qb * a->d_k * sizeof(float), kWsAlign);
  pl->ws_logit = align_up((size_t)a->H_q * pl->n_qb * pl->n_kvb * sizeof(float), kWsAlign);
  pl->ws_total = pl->ws_kb + pl->ws_qb + pl->ws_logit;
  return KVS_OK;
}

kvs_status block_select_run(const kvs_block_select_args* a, const BlockPlan& pl,
                            const uint16_t* Qc, const uint16_t* K, uint8_t* M, void* ws,
                            float* Kb, int kb_ld, int n_cached, hipStream_t stream) {
  if (!Kb) {   // no cache: every key block's mean goes to the workspace
    Kb = static_cast<float*>(ws);
    kb_ld = pl.n_kvb;
    n_cached = 0;
  }
  float* Qb = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.ws_kb);
  float* logit = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.ws_kb + pl.ws_qb);
  const float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->d_k);
  if (pl.n_kvb > n_cached)
    hipLaunchKernelGGL(block_mean_kernel, dim3(pl.n_kvb - n_cached, a->H_kv), dim3(kThreads), 0,
                       stream, K, a->k_head_stride, a->k_tok_stride, a->L, a->d_k, a->block, kb_ld,
                       n_cached, Kb);
  hipLaunchKernelGGL(block_mean_kernel, dim3(pl.n_qb, a->H_q), dim3(kThreads), 0, stream, Qc,
                     a->q_head_stride, a->q_row_stride, a->Lq, a->d_k, a->block, pl.n_qb, 0, Qb);
  const int G = a->H_q / a->H_kv;
  hipLaunchKernelGGL(block_logits_kernel,
                     dim3((pl.n_kvb + kLt - 1) / kLt, a->H_kv, (G * pl.n_qb + kLt - 1) / kLt),
                     dim3(kThreads), 0, stream, Qb, Kb, kb_ld, G, pl.n_qb, pl.n_kvb, a->d_k, scale,
                     logit);
  hipLaunchKernelGGL(block_topp_kernel, dim3(pl.n_qb, a->H_q), dim3(kThreads), 0, stream, logit,
                     pl.n_qb, pl.n_kvb, a->block, a->Lq, a->q_pos0, a->p_mass, M);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

size_t union_ws_bytes(int H_q, int H_kv, int sub_group, int n_kvb) {
  const int G = H_q / H_kv;
  const int sg = sub_group == 0 ? G : sub_group;
  const int n_groups = H_q / sg;
  return align_up((size_t)n_groups * n_kvb * sizeof(int32_t), kWsAlign) +
         align_up((size_t)n_groups * sizeof(int32_t), kWsAlign);
}

kvs_status union_run(const uint8_t* M, int H_q, int H_kv, int sub_group, int n_qb, int n_kvb,
                     int32_t* indptr, int32_t* indices, void* ws, hipStream_t stream) {
  const int G = H_q / H_kv;
  const int sg = sub_group == 0 ? G : sub_group;
  const int n_groups = H_q / sg;
  int32_t* staging = static_cast<int32_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(
      static_cast<char*>(ws) + align_up((size_t)n_groups * n_kvb * sizeof(int32_t), kWsAlign));
  hipLaunchKernelGGL(union_group_kernel, dim3(n_groups), dim3(kThreads), 0, stream, M, sg, n_qb,
                     n_kvb, staging, counts);
  hipLaunchKernelGGL(union_pack_kernel, dim3(1), dim3(kThreads), 0, stream, staging, counts,
                     n_groups, n_kvb, indptr, indices);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

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

__device__ __forceinline__ uint32_t ord_pos(float p) { return __float_as_uint(p) | 0x80000000u; }

// ------------------------------------------------------------------ top-p per (head, query block)
__global__ __launch_bounds__(kThreads) void block_topp_kernel(
    const float* __restrict__ Qb, const float* __restrict__ Kb, int kb_ld, int G, int n_qb,
    int n_kvb, int sort_n, int d_k, int block, int Lq, int64_t q_pos0, float scale, float p_mass,
    uint8_t* __restrict__ M) {
  __shared__ uint64_t keys[kMaxKvb];
  __shared__ float val[kMaxKvb];
  __shared__ float qv[128];
  __shared__ float red[kThreads];
  const int i = blockIdx.x, h = blockIdx.y, g = h / G;
  const int tid = threadIdx.x;
  for (int d = tid; d < d_k; d += kThreads) qv[d] = Qb[((int64_t)h * n_qb + i) * d_k + d];
  __syncthreads();
  const int64_t last_row = min((int64_t)(i + 1) * block, (int64_t)Lq) - 1;
  const int64_t end_pos = q_pos0 + last_row;
  const float* kg = Kb + (int64_t)g * kb_ld * d_k;
  // 1. logits of visible blocks
  float mloc = -__builtin_inff();
  for (int j = tid; j < n_kvb; j += kThreads) {
    float v = -__builtin_inff();
    if ((int64_t)j * block <= end_pos) {
      const float* kr = kg + (int64_t)j * d_k;
      float s = 0.f;
      for (int d = 0; d < d_k; ++d) s = fmaf(qv[d], kr[d], s);
      v = scale * s;
    }
    val[j] = v;
    mloc = fmaxf(mloc, v);
  }
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
  // 3. sort keys: probability desc, then j asc (bit-inverted j in the low word)
  for (int j = tid; j < sort_n; j += kThreads) {
    uint64_t k = 0ull;  // padding sorts last
    if (j < n_kvb) {
      const float p = val[j] * inv_z;
      k = ((uint64_t)ord_pos(p) << 32) | (uint64_t)(~(uint32_t)j);
    }
    keys[j] = k;
  }
  __syncthreads();
  for (int size = 2; size <= sort_n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < sort_n; x += kThreads) {
        const int y = x ^ stride;
        if (y > x) {
          const bool desc = (x & size) == 0;
          const uint64_t a = keys[x], b = keys[y];
          if (desc ? (a < b) : (a > b)) {
            keys[x] = b;
            keys[y] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // 4. exclusive prefix of the sorted probabilities: contiguous chunk per thread
  const int per = sort_n / kThreads > 0 ? sort_n / kThreads : 1;
  const int lo = tid * per;
  float csum = 0.f;
  for (int s = lo; s < lo + per && s < sort_n; ++s)
    csum += __uint_as_float((uint32_t)(keys[s] >> 32) & 0x7fffffffu);
  red[tid] = csum;
  __syncthreads();
  float before = 0.f;
  for (int t = 0; t < tid; ++t) before += red[t];
  uint8_t* mrow = M + ((int64_t)h * n_qb + i) * n_kvb;
  for (int s = lo; s < lo + per && s < sort_n; ++s) {
    const uint64_t k = keys[s];
    const uint32_t j = ~(uint32_t)k;
    const float p = __uint_as_float((uint32_t)(k >> 32) & 0x7fffffffu);
    if (k != 0ull && j < (uint32_t)n_kvb) {
      const bool visible = (int64_t)j * block <= end_pos;
      mrow[j] = (visible && before < p_mass) ? 1 : 0;
    }
    before += p;
  }
}

// ------------------------------------------------------------------ union
// One workgroup per subgroup: OR over its heads and query blocks, then an
// ascending compaction of the set KV blocks into staging.
__global__ __launch_bounds__(kThreads) void union_group_kernel(const uint8_t* __restrict__ M,
                                                               int sg, int n_qb, int n_kvb,
                                                               int32_t* __restrict__ staging,
                                                               int32_t* __restrict__ counts) {
  __shared__ uint32_t wc[kThreads / 64];
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint32_t run = 0;
  for (int base = 0; base < n_kvb; base += kThreads) {
    const int j = base + tid;
    bool on = false;
    if (j < n_kvb) {
      for (int h = s * sg; h < (s + 1) * sg && !on; ++h)
        for (int i = 0; i < n_qb; ++i)
          if (M[((int64_t)h * n_qb + i) * n_kvb + j]) {
            on = true;
            break;
          }
    }
    const uint64_t m = __ballot(on);
    if (lane == 0) wc[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, tile = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      before += w < wave ? wc[w] : 0u;
      tile += wc[w];
    }
    if (on) staging[(int64_t)s * n_kvb + run + before + __popcll(m & lt_mask)] = j;
    run += tile;
    __syncthreads();
  }
  if (tid == 0) counts[s] = (int32_t)run;
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
  int s = 1;
  while (s < pl->n_kvb) s <<= 1;
  pl->sort_n = s;
  pl->ws_kb = align_up((size_t)a->H_kv * pl->n_kvb * a->d_k * sizeof(float), kWsAlign);
  pl->ws_qb = align_up((size_t)a->H_q * pl->n_qb * a->d_k * sizeof(float), kWsAlign);
  pl->ws_total = pl->ws_kb + pl->ws_qb;
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
  const float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->d_k);
  if (pl.n_kvb > n_cached)
    hipLaunchKernelGGL(block_mean_kernel, dim3(pl.n_kvb - n_cached, a->H_kv), dim3(kThreads), 0,
                       stream, K, a->k_head_stride, a->k_tok_stride, a->L, a->d_k, a->block, kb_ld,
                       n_cached, Kb);
  hipLaunchKernelGGL(block_mean_kernel, dim3(pl.n_qb, a->H_q), dim3(kThreads), 0, stream, Qc,
                     a->q_head_stride, a->q_row_stride, a->Lq, a->d_k, a->block, pl.n_qb, 0, Qb);
  hipLaunchKernelGGL(block_topp_kernel, dim3(pl.n_qb, a->H_q), dim3(kThreads), 0, stream, Qb, Kb,
                     kb_ld, a->H_q / a->H_kv, pl.n_qb, pl.n_kvb, pl.sort_n, a->d_k, a->block, a->Lq,
                     a->q_pos0, scale, a->p_mass, M);
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

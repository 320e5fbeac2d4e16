// Post-processing of token scores on gfx950: head reduction, 1-D pooling and
// page aggregation (kvs_pool_pages), density-clustering priority
// (kvs_cluster_priority) and cross-layer aggregation (kvs_aggregate_layers).
//
// These steps move a few bytes per token, so they are bound by HBM / L2
// bandwidth: each workgroup stages a chunk of the head-reduced row plus the
// pooling halo in LDS once, then pools and pages from LDS.  Every sum runs
// left to right in float32 so the result does not depend on the launch shape.
#include <math.h>

#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kChunk = 2048;   // most tokens per workgroup (the LDS stage)
constexpr int kChunkTarget = 512;   // tokens per workgroup when pages allow: many workgroups
constexpr int kThreads = 256;
constexpr int kMaxHalo = 64;   // pool_k <= 129
constexpr float kNegInf = -__builtin_inff();

// Row h' of the head-reduced input at token t (caller guarantees 0 <= t < n).
// The heads are loaded kHeadBatch at a time, all loads of a batch in flight
// together, and combined in head order.
constexpr int kHeadBatch = 16;
__device__ __forceinline__ float reduced(const float* S, int H, int64_t ld, int head_reduce,
                                         int row, int t) {
  if (head_reduce == KVS_RED_NONE) return S[(int64_t)row * ld + t];
  float v = 0.f;
  for (int h0 = 0; h0 < H; h0 += kHeadBatch) {
    float x[kHeadBatch];
#pragma unroll
    for (int k = 0; k < kHeadBatch; ++k)
      x[k] = h0 + k < H ? S[(int64_t)(h0 + k) * ld + t] : 0.f;
#pragma unroll
    for (int k = 0; k < kHeadBatch; ++k) {
      if (h0 + k >= H) break;
      v = h0 + k == 0 ? x[k] : head_reduce == KVS_RED_MAX ? fmaxf(v, x[k]) : v + x[k];
    }
  }
  return head_reduce == KVS_RED_MEAN ? v / (float)H : v;
}

__global__ __launch_bounds__(kThreads) void pool_pages_kernel(
    const float* __restrict__ S, int H, int n, int64_t ld, int head_reduce, int pool, int pool_k,
    int P, int page_reduce, int chunk, float* __restrict__ pooled, float* __restrict__ page,
    int32_t* __restrict__ page_arg) {
  __shared__ float xs[kChunk + 2 * kMaxHalo];
  __shared__ float ys[kChunk];
  const int row = blockIdx.y;
  const int c0 = blockIdx.x * chunk;
  const int c1 = min(c0 + chunk, n);
  const int r = pool == KVS_RED_NONE ? 0 : (pool_k - 1) / 2;
  // 1. head-reduced values for [c0 - r, c1 + r) clipped to [0, n)
  for (int i = threadIdx.x; i < (c1 - c0) + 2 * r; i += kThreads) {
    const int t = c0 - r + i;
    xs[i] = (t >= 0 && t < n) ? reduced(S, H, ld, head_reduce, row, t) : 0.f;
  }
  __syncthreads();
  // 2. pooling over the clipped window, left to right
  for (int i = threadIdx.x; i < c1 - c0; i += kThreads) {
    const int t = c0 + i;
    float y;
    if (pool == KVS_RED_NONE) {
      y = xs[i];
    } else {
      const int lo = max(t - r, 0), hi = min(t + r, n - 1);
      if (pool == KVS_RED_MAX) {
        y = kNegInf;
        for (int u = lo; u <= hi; ++u) y = fmaxf(y, xs[u - c0 + r]);
      } else {
        float s = 0.f;
        for (int u = lo; u <= hi; ++u) s += xs[u - c0 + r];
        y = s / (float)(hi - lo + 1);
      }
    }
    ys[i] = y;
    if (pooled) pooled[(int64_t)row * n + t] = y;
  }
  if (P <= 0) return;
  __syncthreads();
  // 3. pages: chunk boundaries are multiples of P
  const int n_pages = (n + P - 1) / P;
  const int u0 = c0 / P;
  const int u1 = (c1 + P - 1) / P;
  for (int u = u0 + threadIdx.x; u < u1; u += kThreads) {
    const int a = u * P, e = min(a + P, n);
    float best = ys[a - c0];
    int arg = a;
    float acc = best;
    for (int t = a + 1; t < e; ++t) {
      const float y = ys[t - c0];
      if (y > best) {
        best = y;
        arg = t;
      }
      acc = page_reduce == KVS_RED_SUM ? acc + y : acc;
    }
    const float z = page_reduce == KVS_RED_SUM ? acc : best;
    if (page) page[(int64_t)row * n_pages + u] = z;
    if (page_arg) page_arg[(int64_t)row * n_pages + u] = arg;
  }
}

__global__ __launch_bounds__(kThreads) void cluster_kernel(const float* __restrict__ page,
                                                           const int32_t* __restrict__ page_arg,
                                                           int n_pages, int P, int n, float theta,
                                                           int r, uint8_t* __restrict__ prio) {
  const int row = blockIdx.y;
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= n) return;
  int ua = (t - r) / P;
  if (t - r < 0) ua = 0;
  int ub = (t + r) / P;
  if (ub > n_pages - 1) ub = n_pages - 1;
  uint8_t hit = 0;
  for (int u = ua; u <= ub; ++u) {
    const float z = page[(int64_t)row * n_pages + u];
    const int cc = page_arg[(int64_t)row * n_pages + u];
    const int d = t - cc;
    if (z >= theta && d <= r && d >= -r) hit = 1;
  }
  prio[(int64_t)row * n + t] = hit;
}

constexpr int kAggThreads = 256;   // one token per thread
constexpr int kAggBatch = 8;       // head rows loaded together

// Sum over the H rows of token t, left to right in float32; the rows are
// loaded kAggBatch at a time so their latencies overlap.
__device__ __forceinline__ float head_sum(const float* S, int H, int64_t ld, int t) {
  float v = 0.f;
  for (int h0 = 0; h0 < H; h0 += kAggBatch) {
    float x[kAggBatch];
#pragma unroll
    for (int i = 0; i < kAggBatch; ++i) x[i] = h0 + i < H ? S[(int64_t)(h0 + i) * ld + t] : 0.f;
#pragma unroll
    for (int i = 0; i < kAggBatch; ++i)
      if (h0 + i < H) v = h0 + i == 0 ? x[i] : v + x[i];
  }
  return v;
}

// Partial L1 norms, one float64 per workgroup (a fixed-order tree over its
// tokens).
__global__ __launch_bounds__(kAggThreads) void agg_norm_kernel(const float* __restrict__ S, int H,
                                                               int n, int64_t ld,
                                                               double* __restrict__ part) {
  __shared__ double red[kAggThreads];
  const int t = blockIdx.x * kAggThreads + threadIdx.x;
  red[threadIdx.x] = t < n ? fabs((double)head_sum(S, H, ld, t)) : 0.0;
  __syncthreads();
  for (int w = kAggThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// acc (=|+=|max) the head sum of token t, SUM_L1 scaled by 1 / (sum of the
// partial norms).  The first wave adds the partials: lane l the partials
// l, l + 64, ... in order, then the lanes in a fixed tree, so every workgroup
// and every call gets the same norm.
__global__ __launch_bounds__(kAggThreads) void agg_apply_kernel(
    float* __restrict__ acc, const float* __restrict__ S, int H, int n, int64_t ld, int mode,
    int first, const double* __restrict__ part, int n_part) {
  __shared__ float inv_norm_s;
  const int t = blockIdx.x * kAggThreads + threadIdx.x;
  const float s = t < n ? head_sum(S, H, ld, t) : 0.f;
  float inv_norm = 0.f;
  if (mode == KVS_RED_SUM_L1) {
    if (threadIdx.x < 64) {
      double norm = 0.0;
      for (int i = threadIdx.x; i < n_part; i += 64) norm += part[i];
#pragma unroll
      for (int d = 32; d > 0; d >>= 1) norm += __shfl_xor(norm, d);
      if (threadIdx.x == 0) inv_norm_s = (float)(1.0 / norm);
    }
    __syncthreads();
    inv_norm = inv_norm_s;
  }
  if (t >= n) return;
  if (mode == KVS_RED_SUM_L1) {
    const float v = s * inv_norm;
    acc[t] = first ? v : acc[t] + v;
  } else {
    acc[t] = first ? s : fmaxf(acc[t], s);
  }
}

}  // namespace

kvs_status pool_pages_run(const float* S, int H, int n, int64_t ld, int head_reduce, int pool,
                          int pool_k, int P, int page_reduce, float* pooled, float* page,
                          int32_t* page_arg, hipStream_t stream) {
  const int rows = head_reduce == KVS_RED_NONE ? H : 1;
  // page-aligned chunks of about kChunkTarget tokens (a whole page when pages are longer)
  int chunk = kChunkTarget;
  if (P > 0) chunk = P <= kChunkTarget ? kChunkTarget / P * P : P;
  if (chunk <= 0 || chunk > kChunk) return KVS_EUNSUPPORTED;
  dim3 grid((n + chunk - 1) / chunk, rows);
  hipLaunchKernelGGL(pool_pages_kernel, grid, dim3(kThreads), 0, stream, S, H, n, ld, head_reduce,
                     pool, pool_k, P, page_reduce, chunk, pooled, page, page_arg);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

kvs_status cluster_priority_run(const float* page, const int32_t* page_arg, int H, int n_pages,
                                int P, int n, float theta, int r, uint8_t* prio,
                                hipStream_t stream) {
  dim3 grid((n + kThreads - 1) / kThreads, H);
  hipLaunchKernelGGL(cluster_kernel, grid, dim3(kThreads), 0, stream, page, page_arg, n_pages, P, n,
                     theta, r, prio);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

size_t aggregate_ws_bytes(int n) {
  const size_t blocks = ((size_t)n + kAggThreads - 1) / kAggThreads;
  return align_up(blocks * sizeof(double), kWsAlign);
}

kvs_status aggregate_run(float* acc, const float* S, int H, int n, int64_t ld, int mode, int first,
                         void* ws, hipStream_t stream) {
  const int blocks = (n + kAggThreads - 1) / kAggThreads;
  double* part = static_cast<double*>(ws);
  if (mode == KVS_RED_SUM_L1)
    hipLaunchKernelGGL(agg_norm_kernel, dim3(blocks), dim3(kAggThreads), 0, stream, S, H, n, ld, part);
  hipLaunchKernelGGL(agg_apply_kernel, dim3(blocks), dim3(kAggThreads), 0, stream, acc, S, H, n, ld,
                     mode, first, part, blocks);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

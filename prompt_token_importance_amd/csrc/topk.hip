// Top-k selection with stable ties and a forced suffix (kvs_topk).
//
// The CLAA page selects topk(scores, keep_rate) and keeps the chosen tokens at
// their original positions ("Complete flow and cost"); the ClusterAttn page
// ranks clustered tokens first and fills with the best remaining ones, then
// appends the observation window ("Method details").  Order: priority desc,
// value desc, index asc; the output lists the chosen indices ascending.
//
// One 1024-thread workgroup per row:
//  1. Radix select over the 33-bit key (priority bit, order-preserving map of
//     the float32 value): three histogram passes of 12, 11 and 10 bits in LDS
//     find the exact key K* of the budget-th element and how many elements
//     equal to K* must be taken.
//  2. Stable compaction in index order: tiles of 1024 consecutive elements,
//     wave ballots give each element its rank among the K*-equal elements and
//     its output slot, so ties go to the lower index and the output is sorted.
// Everything is integer work on the keys: the result is exact and unique.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Order-preserving map of a float32 to uint32: -0 equals +0, NaN is lowest.
__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t full_key(const float* row, const uint8_t* prow, int i) {
  const uint64_t pr = (prow && prow[i]) ? 1ull : 0ull;
  return (pr << 32) | ord_key(row[i]);
}

// Digit of pass p: bits [32:21], [20:10], [9:0] of the 33-bit key.
__device__ __forceinline__ uint32_t digit(uint64_t k, int p) {
  return p == 0 ? (uint32_t)(k >> 21) & 0xFFFu : p == 1 ? (uint32_t)(k >> 10) & 0x7FFu
                                                        : (uint32_t)k & 0x3FFu;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ S, int n,
                                                        int64_t ld, int budget,
                                                        const uint8_t* __restrict__ prio,
                                                        int n_forced, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t scan[kThreads];
  __shared__ uint32_t wcnt[2][kWaves];
  __shared__ uint64_t s_prefix;
  __shared__ uint32_t s_need;

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* x = S + (int64_t)row * ld;
  const uint8_t* pr = prio ? prio + (int64_t)row * n : nullptr;
  int32_t* out = idx + (int64_t)row * (budget + n_forced);

  for (int i = tid; i < n_forced; i += kThreads) out[budget + i] = n + i;
  if (budget == 0) return;

  // ---------------------------------------------------------------- select
  uint64_t prefix = 0;   // bits of K* fixed so far (in place)
  uint64_t pmask = 0;    // which bits of the key are fixed
  uint32_t need = (uint32_t)budget;
  const int bits[3] = {12, 11, 10};
  const int shift[3] = {21, 10, 0};
  for (int p = 0; p < 3; ++p) {
    const int nb = 1 << bits[p];
    for (int b = tid; b < nb; b += kThreads) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint64_t k = full_key(x, pr, i);
      if ((k & pmask) == prefix) atomicAdd(&hist[digit(k, p)], 1u);
    }
    __syncthreads();
    // each thread owns nb / kThreads consecutive bins; suffix sums from the top
    const int per = nb / kThreads;  // 4, 2 or 1
    uint32_t ls = 0;
    for (int b = 0; b < per; ++b) ls += hist[tid * per + b];
    scan[kThreads - 1 - tid] = ls;   // reversed: position 0 = highest bins
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const uint32_t v = tid >= off ? scan[tid - off] : 0u;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    // inclusive scan over reversed order; bins above this thread's range:
    const int rt = kThreads - 1 - tid;
    const uint32_t above = rt > 0 ? scan[rt - 1] : 0u;
    if (above < need && need <= above + ls) {
      uint32_t cum = above;
      for (int b = per - 1; b >= 0; --b) {
        const int bin = tid * per + b;
        const uint32_t h = hist[bin];
        if (cum + h >= need) {
          s_prefix = prefix | ((uint64_t)bin << shift[p]);
          s_need = need - cum;
          break;
        }
        cum += h;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    pmask |= (uint64_t)(nb - 1) << shift[p];
    __syncthreads();
  }
  const uint64_t kstar = prefix;    // exact key of the budget-th element
  const uint32_t need_eq = need;    // K*-equal elements to take, lowest indices first

  // ---------------------------------------------------------------- compact
  uint32_t run_eq = 0, run_sel = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    bool gt = false, eq = false;
    if (i < n) {
      const uint64_t k = full_key(x, pr, i);
      gt = k > kstar;
      eq = k == kstar;
    }
    const uint64_t m_eq = __ballot(eq);
    if (lane == 0) wcnt[0][wave] = (uint32_t)__popcll(m_eq);
    __syncthreads();
    uint32_t eq_before = 0, eq_tile = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = wcnt[0][w];
      eq_before += w < wave ? c : 0u;
      eq_tile += c;
    }
    const uint32_t eq_rank = run_eq + eq_before + (uint32_t)__popcll(m_eq & lt_mask);
    const bool sel = gt || (eq && eq_rank < need_eq);
    const uint64_t m_sel = __ballot(sel);
    if (lane == 0) wcnt[1][wave] = (uint32_t)__popcll(m_sel);
    __syncthreads();
    uint32_t sel_before = 0, sel_tile = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = wcnt[1][w];
      sel_before += w < wave ? c : 0u;
      sel_tile += c;
    }
    if (sel) out[run_sel + sel_before + (uint32_t)__popcll(m_sel & lt_mask)] = i;
    run_eq += eq_tile;
    run_sel += sel_tile;
    __syncthreads();
  }
}

}  // namespace

size_t topk_ws_bytes(int, int, int) { return 0; }

kvs_status topk_run(const float* S, int H, int n, int64_t ld, int budget, const uint8_t* prio,
                    int n_forced, int32_t* idx, void*, hipStream_t stream) {
  if (H == 0) return KVS_OK;
  hipLaunchKernelGGL(topk_kernel, dim3(H), dim3(kThreads), 0, stream, S, n, ld, budget, prio,
                     n_forced, idx);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

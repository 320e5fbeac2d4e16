// Top-k selection with stable ties and a forced suffix (kvs_topk).
//
// The CLAA page selects topk(scores, keep_rate) and keeps the chosen tokens at
// their original positions ("Complete flow and cost"); the ClusterAttn page
// ranks clustered tokens first and fills with the best remaining ones, then
// appends the observation window ("Method details").  Order: priority desc,
// value desc, index asc; the output lists the chosen indices ascending.
//
// Every row is split into chunks of kChunk elements, one 256-thread workgroup
// per (chunk, row), so a launch covers the whole GPU even for 8 rows:
//  1. Radix select over the 33-bit key (priority bit, order-preserving map of
//     the float32 value) in three passes of 12, 11 and 10 bits.  A pass builds
//     a per-workgroup LDS histogram of the digit among the elements matching
//     the prefix found so far and adds it to the row's histogram in the
//     workspace with integer atomics (exact, order-free).  The next kernel's
//     workgroups each scan the finished histograms to fix the digits of the
//     threshold key K* and how many K*-equal elements are needed: kernel
//     boundaries order the passes, so no device-wide fence is needed.
//  2. A count pass records, per chunk, the elements above K* and equal to K*.
//  3. The output pass gives each chunk its offset from the counts of the
//     chunks before it; a thread owns kEpt consecutive elements, and two
//     workgroup prefix sums (K*-equal elements, then chosen elements) give
//     every element its rank and output slot in index order: ties go to the
//     lower index and the output is ascending.
// Everything is integer work on the keys: the result is exact and unique.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kEpt = 16;                       // elements per thread per chunk
constexpr int kChunk = kThreads * kEpt;        // 4096
constexpr int kBins0 = 4096, kBins1 = 2048, kBins2 = 1024;
constexpr int kShift[3] = {21, 10, 0};

// Per-row state in the workspace.
struct RowState {
  uint64_t prefix;   // fixed high bits of K*
  uint32_t need;     // elements still to take at or below the prefix
  uint32_t unused;
};

struct Ws {
  RowState* state;   // [H]
  uint32_t* hist;    // [H][kBins0 + kBins1 + kBins2]
  uint32_t* counts;  // [H][n_chunks][2]  (above K*, equal to K*)
};

__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN below every number
  if (b == 0x80000000u) b = 0u;                     // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float v, uint8_t pr) {
  return ((uint64_t)(pr ? 1u : 0u) << 32) | ord_key(v);
}

__device__ __forceinline__ uint32_t pass_bins(int p) {
  return p == 0 ? kBins0 : p == 1 ? kBins1 : kBins2;
}
__device__ __forceinline__ uint32_t pass_offset(int p) {
  return p == 0 ? 0 : p == 1 ? kBins0 : kBins0 + kBins1;
}
__device__ __forceinline__ uint64_t pass_mask(int p) {  // bits fixed before pass p
  return p == 0 ? 0ull : p == 1 ? (0xFFFull << 21) : (0x7FFFFFull << 10);  // bits 21..32, 10..32
}

// Loads this thread's kEpt keys of the chunk; invalid slots get valid = false.
__device__ __forceinline__ void load_keys(const float* x, const uint8_t* pr, int n, int c0,
                                          uint64_t (&k)[kEpt], uint32_t& valid) {
  float v[kEpt];
  uint8_t q[kEpt];
  valid = 0;
#pragma unroll
  for (int e = 0; e < kEpt; ++e) {
    const int i = c0 + (int)threadIdx.x * kEpt + e;
    const bool ok = i < n;
    v[e] = ok ? x[i] : 0.f;
    q[e] = (ok && pr) ? pr[i] : (uint8_t)0;
    valid |= ok ? (1u << e) : 0u;
  }
#pragma unroll
  for (int e = 0; e < kEpt; ++e) k[e] = make_key(v[e], q[e]);
}

__global__ __launch_bounds__(kThreads) void topk_zero_kernel(Ws ws, int H, int n_chunks) {
  const int total = H * (kBins0 + kBins1 + kBins2);
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads)
    ws.hist[i] = 0u;
  if (blockIdx.x == 0)
    for (int h = threadIdx.x; h < H; h += kThreads) ws.state[h] = RowState{0ull, 0u, 0u};
  (void)n_chunks;
}

// Picks the digit of pass p from the row histogram of that pass (complete
// because the pass ran in an earlier kernel): suffix scan from the top bin to
// the bin holding the need-th candidate.  Every workgroup of a row computes
// the same answer.  Returns the updated (prefix, need).
__device__ void pick_digit(const uint32_t* __restrict__ gh, int p, uint64_t prefix, uint32_t need,
                           uint32_t* h, uint32_t* scan, uint64_t* s_prefix, uint32_t* s_need) {
  const uint32_t nb = pass_bins(p);
  const uint32_t per = nb / kThreads;   // 16, 8 or 4 bins per thread
  uint32_t vals[16];
#pragma unroll
  for (uint32_t b = 0; b < 16; ++b) vals[b] = b < per ? gh[threadIdx.x * per + b] : 0u;
  uint32_t ls = 0;
#pragma unroll
  for (uint32_t b = 0; b < 16; ++b) {
    if (b < per) h[threadIdx.x * per + b] = vals[b];
    ls += vals[b];
  }
  scan[kThreads - 1 - threadIdx.x] = ls;  // position 0 = highest bins
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint32_t v = (int)threadIdx.x >= off ? scan[threadIdx.x - off] : 0u;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  const int rt = kThreads - 1 - threadIdx.x;
  const uint32_t above = rt > 0 ? scan[rt - 1] : 0u;
  if (above < need && need <= above + ls) {
    uint32_t cum = above;
    for (int b = (int)per - 1; b >= 0; --b) {
      const uint32_t bin = threadIdx.x * per + b;
      const uint32_t c = h[bin];
      if (cum + c >= need) {
        *s_prefix = prefix | ((uint64_t)bin << kShift[p]);
        *s_need = need - cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// Threshold key K* and the number of K*-equal elements to take, from the
// histograms of passes 0 .. upto-1.
__device__ void replay_digits(const Ws& ws, int row, int budget, int upto, uint32_t* h,
                              uint32_t* scan, uint64_t* s_prefix, uint32_t* s_need) {
  if (threadIdx.x == 0) {
    *s_prefix = 0ull;
    *s_need = (uint32_t)budget;
  }
  __syncthreads();
  const uint32_t* gh = ws.hist + (size_t)row * (kBins0 + kBins1 + kBins2);
  for (int p = 0; p < upto; ++p) {
    const uint64_t prefix = *s_prefix;
    const uint32_t need = *s_need;
    __syncthreads();
    pick_digit(gh + pass_offset(p), p, prefix, need, h, scan, s_prefix, s_need);
  }
}

// Radix pass p: per-workgroup LDS histogram of digit p among the elements
// matching the prefix fixed by passes 0 .. p-1, added into the row histogram
// with integer atomics (exact).
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ S, int n,
                                                             int64_t ld,
                                                             const uint8_t* __restrict__ prio,
                                                             int budget, int pass, Ws ws) {
  __shared__ uint32_t h[kBins0];
  __shared__ uint32_t scan[kThreads];
  __shared__ uint64_t s_prefix;
  __shared__ uint32_t s_need;
  const int row = blockIdx.y;
  const int c0 = blockIdx.x * kChunk;
  const float* x = S + (int64_t)row * ld;
  const uint8_t* pr = prio ? prio + (int64_t)row * n : nullptr;
  uint64_t k[kEpt];
  uint32_t valid;
  load_keys(x, pr, n, c0, k, valid);
  replay_digits(ws, row, budget, pass, h, scan, &s_prefix, &s_need);
  const uint64_t prefix = s_prefix;
  const uint32_t nb = pass_bins(pass);
  const int shift = kShift[pass];
  const uint64_t pmask = pass_mask(pass);
  for (uint32_t b = threadIdx.x; b < nb; b += kThreads) h[b] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if (((valid >> e) & 1u) && (k[e] & pmask) == prefix)
      atomicAdd(&h[(uint32_t)(k[e] >> shift) & (nb - 1)], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)row * (kBins0 + kBins1 + kBins2) + pass_offset(pass);
  for (uint32_t b = threadIdx.x; b < nb; b += kThreads)
    if (h[b]) atomicAdd(&gh[b], h[b]);
}

__device__ __forceinline__ void block_counts(uint32_t a, uint32_t b, uint32_t* red,
                                             uint32_t& ta, uint32_t& tb) {
  // sums of a and b over the workgroup (fixed order)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_down(a, off);
    b += __shfl_down(b, off);
  }
  if (lane == 0) {
    red[2 * wave] = a;
    red[2 * wave + 1] = b;
  }
  __syncthreads();
  ta = tb = 0;
  for (int w = 0; w < kWaves; ++w) {
    ta += red[2 * w];
    tb += red[2 * w + 1];
  }
}

__global__ __launch_bounds__(kThreads) void topk_count_kernel(const float* __restrict__ S, int n,
                                                              int64_t ld,
                                                              const uint8_t* __restrict__ prio,
                                                              int budget, Ws ws) {
  __shared__ uint32_t red[2 * kWaves];
  const int row = blockIdx.y;
  const int c0 = blockIdx.x * kChunk;
  const float* x = S + (int64_t)row * ld;
  const uint8_t* pr = prio ? prio + (int64_t)row * n : nullptr;
  __shared__ uint32_t h[kBins0];
  __shared__ uint32_t scan[kThreads];
  __shared__ uint64_t s_prefix;
  __shared__ uint32_t s_need;
  uint64_t k[kEpt];
  uint32_t valid;
  load_keys(x, pr, n, c0, k, valid);
  replay_digits(ws, row, budget, 3, h, scan, &s_prefix, &s_need);
  const uint64_t kstar = s_prefix;
  if (blockIdx.x == 0 && threadIdx.x == 0) ws.state[row] = RowState{s_prefix, s_need, 0u};
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if ((valid >> e) & 1u) {
      gt += k[e] > kstar;
      eq += k[e] == kstar;
    }
  uint32_t tg, te;
  block_counts(gt, eq, red, tg, te);
  if (threadIdx.x == 0) {
    uint32_t* c = ws.counts + ((size_t)row * gridDim.x + blockIdx.x) * 2;
    c[0] = tg;
    c[1] = te;
  }
}

// Exclusive prefix sum of one value per thread over the workgroup.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(inc, off);
    if (lane >= off) inc += u;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before += w < wave ? wtot[w] : 0u;
  __syncthreads();
  return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void topk_out_kernel(const float* __restrict__ S, int n,
                                                            int64_t ld,
                                                            const uint8_t* __restrict__ prio,
                                                            int budget, int n_forced, Ws ws,
                                                            int32_t* __restrict__ idx) {
  __shared__ uint32_t wtot[kWaves];
  __shared__ uint32_t s_base[2];
  const int row = blockIdx.y;
  const int chunk = blockIdx.x;
  const int c0 = chunk * kChunk;
  int32_t* out = idx + (int64_t)row * (budget + n_forced);
  if (chunk == 0)
    for (int i = threadIdx.x; i < n_forced; i += kThreads) out[budget + i] = n + i;
  if (budget == 0) return;
  const float* x = S + (int64_t)row * ld;
  const uint8_t* pr = prio ? prio + (int64_t)row * n : nullptr;
  const RowState st = ws.state[row];
  const uint64_t kstar = st.prefix;
  const uint32_t need_eq = st.need;
  if (threadIdx.x == 0) {
    // offsets from the chunks before this one
    const uint32_t* c = ws.counts + (size_t)row * gridDim.x * 2;
    uint32_t eq_before = 0, sel_before = 0;
    for (int j = 0; j < chunk; ++j) {
      const uint32_t g = c[2 * j], e = c[2 * j + 1];
      const uint32_t take = eq_before >= need_eq ? 0u : min(e, need_eq - eq_before);
      sel_before += g + take;
      eq_before += e;
    }
    s_base[0] = eq_before;
    s_base[1] = sel_before;
  }
  uint64_t k[kEpt];
  uint32_t valid;
  load_keys(x, pr, n, c0, k, valid);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kEpt; ++e) {
    const bool ok = (valid >> e) & 1u;
    gt |= (ok && k[e] > kstar) ? (1u << e) : 0u;
    eq |= (ok && k[e] == kstar) ? (1u << e) : 0u;
  }
  // rank of this thread's first K*-equal element among the row's K*-equal elements
  uint32_t run_eq = block_excl_scan((uint32_t)__popc(eq), wtot) + s_base[0];
  uint32_t sel = gt;
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if ((eq >> e) & 1u) {
      if (run_eq < need_eq) sel |= 1u << e;
      ++run_eq;
    }
  uint32_t pos = block_excl_scan((uint32_t)__popc(sel), wtot) + s_base[1];
  const int i0 = c0 + (int)threadIdx.x * kEpt;
#pragma unroll
  for (int e = 0; e < kEpt; ++e)
    if ((sel >> e) & 1u) out[pos++] = i0 + e;
}

size_t ws_state_bytes(int H) { return align_up((size_t)H * sizeof(RowState), kWsAlign); }
size_t ws_hist_bytes(int H) {
  return align_up((size_t)H * (kBins0 + kBins1 + kBins2) * sizeof(uint32_t), kWsAlign);
}
int n_chunks_of(int n) { return (n + kChunk - 1) / kChunk; }

}  // namespace

size_t topk_ws_bytes(int H, int n, int) {
  return ws_state_bytes(H) + ws_hist_bytes(H) +
         align_up((size_t)H * n_chunks_of(n) * 2 * sizeof(uint32_t), kWsAlign);
}

kvs_status topk_run(const float* S, int H, int n, int64_t ld, int budget, const uint8_t* prio,
                    int n_forced, int32_t* idx, void* wsp, hipStream_t stream) {
  if (H == 0) return KVS_OK;
  char* base = static_cast<char*>(wsp);
  Ws ws;
  ws.state = reinterpret_cast<RowState*>(base);
  ws.hist = reinterpret_cast<uint32_t*>(base + ws_state_bytes(H));
  ws.counts = reinterpret_cast<uint32_t*>(base + ws_state_bytes(H) + ws_hist_bytes(H));
  const int nc = n_chunks_of(n);
  const dim3 grid(nc, H);
  if (budget > 0) {
    hipLaunchKernelGGL(topk_zero_kernel, dim3(min(64, H * 4)), dim3(kThreads), 0, stream, ws, H, nc);
    for (int p = 0; p < 3; ++p)
      hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, S, n, ld, prio, budget,
                         p, ws);
    hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kThreads), 0, stream, S, n, ld, prio, budget,
                       ws);
  }
  hipLaunchKernelGGL(topk_out_kernel, grid, dim3(kThreads), 0, stream, S, n, ld, prio, budget,
                     n_forced, ws, idx);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

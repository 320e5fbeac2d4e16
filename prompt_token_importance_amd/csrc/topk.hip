// Top-k selection with stable ties and a forced suffix (kvs_topk, kvs_select).
//
// The CLAA page selects topk(scores, keep_rate) and keeps the chosen tokens at
// their original positions ("Complete flow and cost"), after a 1-D pooling of
// the scores ("Oracle construction"); the ClusterAttn page ranks the tokens
// gathered around block-max centres first and fills with the best remaining
// ones, then appends the observation window ("Method details").  Order:
// priority desc, value desc, index asc; the chosen indices come out ascending.
//
// The ranking key is 33 bits: the priority bit above an order-preserving map
// of the float32 value.  Selection runs inside single 1024-thread workgroups,
// so no workgroup ever waits for another and no device-wide hand-off is paid:
//  stage 1  a row is cut into parts of kCap = 16384 elements, one workgroup
//           per (part, row).  The workgroup computes the keys of its part in
//           registers (16 per thread; the optional pooling or cluster
//           transform reads a 48-score register window per thread, or
//           LDS-staged scores for wide windows), finds its local top-`budget` by a three-digit radix
//           select (12, 11, 10 bits) with LDS histograms, and writes the
//           chosen (key, index) pairs in index order.  Every element of the
//           global top-`budget` is in its part's local top-`budget`, because
//           fewer than `budget` elements of that part precede it.
//  stage 2  one workgroup per row runs the same radix select over the
//           candidates of all parts (in registers when they fit in kCap,
//           else re-read tile by tile) and writes the chosen indices.
// Each radix pass has its own LDS histogram; one wave fixes the digit.
// Rows of at most kCap elements finish in stage 1.  Ties at the threshold key
// K* go to the lower index: after K* and the number `need` of K*-equal
// elements to take are fixed, a workgroup prefix sum ranks the K*-equal
// elements in index order, and a second one gives every chosen element its
// output slot, so the output is ascending and unique.
#include <math.h>

#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kT = 1024;                    // threads per workgroup
constexpr int kW = kT / 64;                 // waves per workgroup
constexpr int kKpt = 16;                    // keys per thread
constexpr int kCap = kT * kKpt;             // keys per workgroup tile (16384)
constexpr int kStage = kCap + 2 * kSelHaloMax;   // staged scores of a part and its halo
constexpr uint64_t kIdxMask = 0x7FFFFFFFull;

enum Transform { kPlain = 0, kPool = 1, kCluster = 2 };

constexpr int kHistWords = 4096 + 2048 + 1024;   // one histogram per radix pass

template <int T>
struct LdsWords {
  static constexpr int value = T == kPlain ? kHistWords : T == kPool ? kStage : 2 * kStage + 8;
};

struct Params {
  const float* S;
  int64_t ld;
  int n;
  const uint8_t* prio;   // kPlain: optional uint8 [H][n]
  int pool_max;          // kPool: 1 = MAX, 0 = MEAN
  int pool_r;            // kPool: half window
  int P;                 // kCluster: page size
  float theta;           // kCluster: centre threshold
  int r;                 // kCluster: gather radius
  int budget, n_forced;
  int vec;               // S rows 16-byte aligned: vector loads
  int parts;             // stage-1 parts per row
  int stride;            // candidate slots per part: min(budget, kCap)
  int64_t cand_ld;       // candidate slots per row (multiple of kCap)
  uint64_t* cand;        // [H][cand_ld] (key << 31 | index)
  uint32_t* wide;        // wide path: per-(row, part) histograms and counts
  int32_t* idx;
};

struct Shared {
  uint32_t w[kW];
  uint64_t prefix;
  uint32_t need;
  uint32_t all_eq;   // the last digit's bin is taken whole: every K*-equal key is chosen
};

__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN below every number
  if (b == 0x80000000u) b = 0u;                     // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float v, bool pr) {
  return ((uint64_t)(pr ? 1u : 0u) << 32) | ord_key(v);
}

// Exclusive prefix sum of one value per thread over the workgroup, and the total.
__device__ __forceinline__ uint32_t scan_excl(uint32_t v, Shared& sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(inc, off);
    if (lane >= off) inc += u;
  }
  if (lane == 63) sh.w[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const uint32_t x = sh.w[w];
    before += w < wave ? x : 0u;
    total += x;
  }
  __syncthreads();
  return before + inc - v;
}

__device__ __forceinline__ int pass_bins(int p) { return p == 0 ? 4096 : p == 1 ? 2048 : 1024; }
__device__ __forceinline__ int pass_shift(int p) { return p == 0 ? 21 : p == 1 ? 10 : 0; }
__device__ __forceinline__ int pass_offset(int p) { return p == 0 ? 0 : p == 1 ? 4096 : 6144; }
__device__ __forceinline__ uint64_t pass_mask(int p) {  // key bits fixed before pass p
  return p == 0 ? 0ull : p == 1 ? (0xFFFull << 21) : (0x7FFFFFull << 10);
}

// Adds this thread's matching keys to the LDS histogram of pass p.
__device__ __forceinline__ void hist_add(uint32_t* hist, int p, uint64_t prefix,
                                         const uint64_t (&k)[kKpt], uint32_t valid) {
  const int shift = pass_shift(p);
  const uint32_t bmask = (uint32_t)pass_bins(p) - 1u;
  const uint64_t pmask = pass_mask(p);
#pragma unroll
  for (int e = 0; e < kKpt; ++e)
    if (((valid >> e) & 1u) && (k[e] & pmask) == prefix)
      atomicAdd(&hist[(uint32_t)(k[e] >> shift) & bmask], 1u);
}

// Fixes the digit of pass p from its complete histogram: the bin holding the
// need-th candidate counted from the top.  Thread t owns the bins of rank
// [t * per, (t + 1) * per) from the top; a workgroup prefix sum of the
// per-thread counts finds the owner.  Leaves (prefix, need, all_eq) in sh.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int p, uint64_t prefix,
                                           uint32_t need, Shared& sh) {
  const int nb = pass_bins(p), per = nb / kT;   // 4, 2 or 1 bins per thread
  const int top = nb - (int)threadIdx.x * per;  // one past this thread's highest bin
  uint32_t c[4];
  uint32_t ls = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    c[b] = b < per ? hist[top - 1 - b] : 0u;
    ls += c[b];
  }
  uint32_t total;
  const uint32_t above = scan_excl(ls, sh, total);
  if (above < need && need <= above + ls) {
    uint32_t cum = above;
    bool done = false;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < per && !done) {
        if (cum + c[b] >= need) {
          sh.prefix = prefix | ((uint64_t)(top - 1 - b) << pass_shift(p));
          sh.need = need - cum;
          sh.all_eq = need - cum == c[b];
          done = true;
        } else {
          cum += c[b];
        }
      }
    }
  }
  __syncthreads();
}

// Radix select over keys held in registers: the threshold key K* and the
// number of K*-equal elements to take so that exactly `budget` are chosen.
// `hist` holds kHistWords words: the three pass histograms, cleared together.
__device__ __forceinline__ void radix_regs(const uint64_t (&k)[kKpt], uint32_t valid,
                                           uint32_t budget, uint32_t* hist, Shared& sh,
                                           uint64_t& kstar, uint32_t& need_eq) {
  for (int b = threadIdx.x; b < kHistWords; b += kT) hist[b] = 0u;
  __syncthreads();
  uint64_t prefix = 0;
  uint32_t need = budget;
  for (int p = 0; p < 3; ++p) {
    uint32_t* h = hist + pass_offset(p);
    hist_add(h, p, prefix, k, valid);
    __syncthreads();
    pick_digit(h, p, prefix, need, sh);
    prefix = sh.prefix;
    need = sh.need;
  }
  kstar = prefix;
  need_eq = need;
}

// Chosen elements of this thread (bit e), ranked in element order: all keys
// above K*, then K*-equal keys while the running rank is below need_eq.
// `eq_base` counts the K*-equal elements of earlier tiles.
__device__ __forceinline__ uint32_t choose(const uint64_t (&k)[kKpt], uint32_t valid,
                                           uint64_t kstar, uint32_t need_eq, uint32_t eq_base,
                                           Shared& sh, uint32_t& eq_total) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool ok = (valid >> e) & 1u;
    gt |= (ok && k[e] > kstar) ? (1u << e) : 0u;
    eq |= (ok && k[e] == kstar) ? (1u << e) : 0u;
  }
  if (sh.all_eq) {
    eq_total = 0;   // not needed: every K*-equal element is chosen
    return gt | eq;
  }
  uint32_t rank = scan_excl((uint32_t)__popc(eq), sh, eq_total) + eq_base;
  uint32_t sel = gt;
#pragma unroll
  for (int e = 0; e < kKpt; ++e)
    if ((eq >> e) & 1u) {
      if (rank < need_eq) sel |= 1u << e;
      ++rank;
    }
  return sel;
}

// Stages the scores [w0, w1) of a row in LDS (coalesced) and synchronizes.
__device__ __forceinline__ void stage(const float* x, int w0, int w1, float* xs) {
#pragma unroll 6
  for (int i = threadIdx.x; i < w1 - w0; i += kT) xs[i] = x[w0 + i];
  __syncthreads();
}

constexpr int kWin = 16;   // halo of the register window on each side

// Scores x[i0 - 16 .. i0 + 32) of a row into registers (w[j] = x[i0 - 16 + j])
// with 16-byte loads.  Requires n % 4 == 0 and 16-byte aligned rows; a float4
// that lies outside [0, n) is read from a clamped in-range position instead,
// and the caller masks every position outside [0, n).
__device__ __forceinline__ void load_window(const Params& s, const float* x, int i0,
                                            float (&w)[kKpt + 2 * kWin]) {
  const float4* p4 = reinterpret_cast<const float4*>(x);
  const int q0 = (i0 - kWin) / 4, qmax = s.n / 4 - 1;
#pragma unroll
  for (int q = 0; q < (kKpt + 2 * kWin) / 4; ++q) {
    const float4 f = p4[min(max(q0 + q, 0), qmax)];
    w[4 * q] = f.x;
    w[4 * q + 1] = f.y;
    w[4 * q + 2] = f.z;
    w[4 * q + 3] = f.w;
  }
}

// Pooling from the register window: element e's terms are w[e + 16 + o],
// |o| <= r <= kWin, clipped to [0, n) and taken left to right.  Terms outside
// [0, n) are replaced once by the identity of the reduction (-inf / +0, which
// leaves a left-to-right float32 sum unchanged) and NaNs are tracked in a bit
// mask, so the inner loop is a plain max or add.  R is r when known at
// compile time, else kWin with a mask on |o|.
template <int R, bool MAX>
__device__ __forceinline__ void pool_regs(const Params& s, int i0, float (&w)[kKpt + 2 * kWin],
                                          uint64_t (&k)[kKpt]) {
  const int r = R < kWin ? R : s.pool_r;
  uint64_t nanm = 0;
#pragma unroll
  for (int j = 0; j < kKpt + 2 * kWin; ++j) {
    const int pos = i0 - kWin + j;
    const bool in = pos >= 0 && pos < s.n;
    nanm |= (uint64_t)(in && w[j] != w[j]) << j;
    w[j] = in ? w[j] : (MAX ? -__builtin_inff() : 0.f);
  }
  const uint64_t span = (2ull << (2 * r)) - 1ull;   // 2r + 1 ones
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const int t = i0 + e;
    float y = MAX ? -__builtin_inff() : 0.f;
#pragma unroll
    for (int o = -R; o <= R; ++o) {
      const float z = w[e + kWin + o];
      const bool use = R < kWin || (o >= -r && o <= r);
      if (MAX)
        y = use ? fmaxf(y, z) : y;
      else
        y = use ? y + z : y;
    }
    if (MAX) {
      if ((nanm >> (e + kWin - r)) & span) y = __builtin_nanf("");
    } else {
      const int lo = max(t - r, 0), hi = min(t + r, s.n - 1);
      y = y / (float)(hi - lo + 1);
    }
    k[e] = make_key(t < s.n ? y : 0.f, false);
  }
}

// Cluster priority with pages of 16 tokens and radius r <= kWin from the
// register window: i0 is page-aligned, so the centres that can reach this
// thread's tokens lie in the previous, own and next pages.
__device__ __forceinline__ void cluster_regs(const Params& s, int i0,
                                             const float (&w)[kKpt + 2 * kWin],
                                             uint64_t (&k)[kKpt]) {
  int cen[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    const int a0 = i0 + 16 * (g - 1);
    float best = w[16 * g];
    int arg = a0;
    bool nan = best != best;
#pragma unroll
    for (int j = 1; j < 16; ++j) {
      const float z = w[16 * g + j];
      const bool in = a0 + j < s.n;
      nan |= in && z != z;
      if (in && z > best) {
        best = z;
        arg = a0 + j;
      }
    }
    const bool page = a0 >= 0 && a0 < s.n;
    cen[g] = (page && !nan && best >= s.theta) ? arg : -1;
  }
  const int r = s.r;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const int t = i0 + e;
    bool pr = false;
#pragma unroll
    for (int g = 0; g < 3; ++g) pr |= cen[g] >= 0 && t - cen[g] <= r && cen[g] - t <= r;
    k[e] = make_key(t < s.n ? w[e + kWin] : 0.f, pr);
  }
}

// Keys of this thread's elements i0 + e (i0 = p0 + 16 * tid) of the part
// [p0, p1); bit e of `valid` tells whether i0 + e < p1.  Leaves `smem` free.
template <int T>
__device__ __forceinline__ void part_keys(const Params& s, int row, int p0, int p1, uint32_t* smem,
                                          uint64_t (&k)[kKpt], uint32_t& valid) {
  const float* x = s.S + (int64_t)row * s.ld;
  const int i0 = p0 + (int)threadIdx.x * kKpt;
  valid = 0;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) valid |= (i0 + e < p1) ? (1u << e) : 0u;
  if constexpr (T == kPlain) {
    float v[kKpt];
    if (s.vec && i0 + kKpt <= p1) {
      const float4* p4 = reinterpret_cast<const float4*>(x + i0);
#pragma unroll
      for (int q = 0; q < kKpt / 4; ++q) {
        const float4 f = p4[q];
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
    } else {
      // clamped (always in-bounds) loads without branches; masked by `valid`
#pragma unroll
      for (int e = 0; e < kKpt; ++e) v[e] = x[min(i0 + e, s.n - 1)];
    }
    if (s.prio) {
      const uint8_t* pr = s.prio + (int64_t)row * s.n;
      uint8_t q[kKpt];
#pragma unroll
      for (int e = 0; e < kKpt; ++e) q[e] = pr[min(i0 + e, s.n - 1)];
#pragma unroll
      for (int e = 0; e < kKpt; ++e) k[e] = make_key(v[e], q[e] != 0);
    } else {
#pragma unroll
      for (int e = 0; e < kKpt; ++e) k[e] = make_key(v[e], false);
    }
  } else if constexpr (T == kPool) {
    // pooled value over [t - r, t + r] clipped to [0, n): max (NaN if any term
    // is NaN) or the left-to-right float32 mean of the in-range terms
    if (s.pool_r <= kWin && s.vec && s.n % 4 == 0) {
      float w[kKpt + 2 * kWin];
      load_window(s, x, i0, w);
      if (s.pool_r == 3)
        s.pool_max ? pool_regs<3, true>(s, i0, w, k) : pool_regs<3, false>(s, i0, w, k);
      else
        s.pool_max ? pool_regs<kWin, true>(s, i0, w, k) : pool_regs<kWin, false>(s, i0, w, k);
      return;
    }
    float* xs = reinterpret_cast<float*>(smem);
    const int rp = s.pool_r;
    const int w0 = max(p0 - rp, 0), w1 = min(p1 + rp, s.n);
    stage(x, w0, w1, xs);
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const int t = i0 + e;
      float y = 0.f;
      if (t < p1) {
        const int lo = max(t - rp, 0), hi = min(t + rp, s.n - 1);
        if (s.pool_max) {
          float m = -__builtin_inff();
          bool nan = false;
          for (int u = lo; u <= hi; ++u) {
            const float z = xs[u - w0];
            nan |= z != z;
            m = fmaxf(m, z);
          }
          y = nan ? __builtin_nanf("") : m;
        } else {
          float acc = 0.f;
          for (int u = lo; u <= hi; ++u) acc += xs[u - w0];
          y = acc / (float)(hi - lo + 1);
        }
      }
      k[e] = make_key(y, false);
    }
    __syncthreads();
  } else {
    // cluster priority: a token is gathered when it lies within r of the
    // argmax (lowest index) of a page of P tokens whose maximum is >= theta;
    // a page holding a NaN has no centre.  Pages [qa, qb] hold every centre
    // that can reach the part.
    if (s.P == 16 && s.r <= kWin && s.vec && s.n % 4 == 0) {
      float w[kKpt + 2 * kWin];
      load_window(s, x, i0, w);
      cluster_regs(s, i0, w, k);
      return;
    }
    const int P = s.P, r = s.r;
    const int qa = max(p0 - r, 0) / P;
    const int qb = min(p1 - 1 + r, s.n - 1) / P;
    const int w0 = qa * P, w1 = min((qb + 1) * P, s.n);
    float* xs = reinterpret_cast<float*>(smem);
    int* cen = reinterpret_cast<int*>(smem + kStage);
    stage(x, w0, w1, xs);
    for (int j = threadIdx.x; j <= qb - qa; j += kT) {
      const int a0 = (qa + j) * P, a1 = min(a0 + P, s.n);
      float best = xs[a0 - w0];
      int arg = a0;
      bool nan = best != best;
      for (int t = a0 + 1; t < a1; ++t) {
        const float z = xs[t - w0];
        nan |= z != z;
        if (z > best) {
          best = z;
          arg = t;
        }
      }
      cen[j] = (!nan && best >= s.theta) ? arg : -1;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const int t = i0 + e;
      bool pr = false;
      float v = 0.f;
      if (t < p1) {
        v = xs[t - w0];
        const int ua = max(t - r, 0) / P, ub = min(t + r, s.n - 1) / P;
        for (int u = ua; u <= ub; ++u) {
          const int cc = cen[u - qa];
          pr |= cc >= 0 && t - cc <= r && cc - t <= r;
        }
      }
      k[e] = make_key(v, pr);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void write_forced(const Params& s, int32_t* out) {
  for (int i = threadIdx.x; i < s.n_forced; i += kT) out[s.budget + i] = s.n + i;
}

// Stage 1: local top-`budget` of one part.  With a single part per row this is
// the final answer (indices), else the chosen (key, index) candidates.
template <int T>
__global__ __launch_bounds__(kT) void topk_part_kernel(Params s) {
  __shared__ uint32_t smem[LdsWords<T>::value];
  __shared__ Shared sh;
  const int row = blockIdx.y, part = blockIdx.x;
  const int p0 = part * kCap, p1 = min(p0 + kCap, s.n);
  const int m = p1 - p0;
  uint64_t k[kKpt];
  uint32_t valid;
  part_keys<T>(s, row, p0, p1, smem, k, valid);
  const uint32_t keep = (uint32_t)min(s.budget, m);
  uint32_t sel, tot;
  if (keep == (uint32_t)m) {
    sel = valid;
  } else {
    uint64_t kstar;
    uint32_t need_eq;
    radix_regs(k, valid, keep, smem, sh, kstar, need_eq);
    sel = choose(k, valid, kstar, need_eq, 0u, sh, tot);
  }
  uint32_t pos = scan_excl((uint32_t)__popc(sel), sh, tot);
  const int i0 = p0 + (int)threadIdx.x * kKpt;
  if (s.parts == 1) {
    int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if ((sel >> e) & 1u) out[pos++] = i0 + e;
    write_forced(s, out);
  } else {
    uint64_t* c = s.cand + (int64_t)row * s.cand_ld + (int64_t)part * s.stride;
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if ((sel >> e) & 1u) c[pos++] = (k[e] << 31) | (uint64_t)(uint32_t)(i0 + e);
  }
}

// Candidate keys of tile [t0, t0 + kCap) of a row: slot i belongs to part
// i / stride and holds a candidate when i % stride < that part's count.
__device__ __forceinline__ void cand_keys(const Params& s, const uint64_t* c, int64_t t0,
                                          uint64_t (&k)[kKpt], uint32_t (&ix)[kKpt],
                                          uint32_t& valid) {
  const int64_t i0 = t0 + (int64_t)threadIdx.x * kKpt;
  const uint4* p4 = reinterpret_cast<const uint4*>(c + i0);
  valid = 0;
#pragma unroll
  for (int q = 0; q < kKpt / 2; ++q) {
    const uint4 v = p4[q];
    const uint64_t a = ((uint64_t)v.y << 32) | v.x, b = ((uint64_t)v.w << 32) | v.z;
    k[2 * q] = a >> 31;
    k[2 * q + 1] = b >> 31;
    ix[2 * q] = (uint32_t)(a & kIdxMask);
    ix[2 * q + 1] = (uint32_t)(b & kIdxMask);
  }
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const int64_t i = i0 + e;
    const int part = (int)(i / s.stride);
    const int slot = (int)(i - (int64_t)part * s.stride);
    const int m = part < s.parts ? min(kCap, s.n - part * kCap) : 0;
    valid |= slot < min(s.budget, m) ? (1u << e) : 0u;
  }
}

// Stage 2: the final selection among the candidates of all parts of a row.
__global__ __launch_bounds__(kT) void topk_merge_kernel(Params s) {
  __shared__ uint32_t hist[kHistWords];
  __shared__ Shared sh;
  const int row = blockIdx.x;
  const uint64_t* c = s.cand + (int64_t)row * s.cand_ld;
  int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
  const int64_t count = (int64_t)s.parts * s.stride;
  uint64_t k[kKpt];
  uint32_t ix[kKpt];
  uint32_t valid;
  uint32_t tot;
  if (count <= kCap) {
    cand_keys(s, c, 0, k, ix, valid);
    uint64_t kstar;
    uint32_t need_eq;
    radix_regs(k, valid, (uint32_t)s.budget, hist, sh, kstar, need_eq);
    const uint32_t sel = choose(k, valid, kstar, need_eq, 0u, sh, tot);
    uint32_t pos = scan_excl((uint32_t)__popc(sel), sh, tot);
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if ((sel >> e) & 1u) out[pos++] = (int32_t)ix[e];
  } else {
    // more candidates than registers hold: every pass re-reads them by tiles
    for (int b = threadIdx.x; b < kHistWords; b += kT) hist[b] = 0u;
    __syncthreads();
    uint64_t prefix = 0;
    uint32_t need = (uint32_t)s.budget;
    for (int p = 0; p < 3; ++p) {
      uint32_t* h = hist + pass_offset(p);
      for (int64_t t0 = 0; t0 < count; t0 += kCap) {
        cand_keys(s, c, t0, k, ix, valid);
        hist_add(h, p, prefix, k, valid);
      }
      __syncthreads();
      pick_digit(h, p, prefix, need, sh);
      prefix = sh.prefix;
      need = sh.need;
    }
    uint32_t eq_base = 0, sel_base = 0;
    for (int64_t t0 = 0; t0 < count; t0 += kCap) {
      cand_keys(s, c, t0, k, ix, valid);
      uint32_t eq_tot;
      const uint32_t sel = choose(k, valid, prefix, need, eq_base, sh, eq_tot);
      uint32_t pos = scan_excl((uint32_t)__popc(sel), sh, tot) + sel_base;
#pragma unroll
      for (int e = 0; e < kKpt; ++e)
        if ((sel >> e) & 1u) out[pos++] = (int32_t)ix[e];
      eq_base += eq_tot;
      sel_base += tot;
    }
  }
  write_forced(s, out);
}

// ------------------------------------------------------------------ wide rows
// Rows whose candidates would not fit one workgroup (parts * min(budget,
// kCap) > kCap, e.g. a 20% keep rate of a 128K-token row) run the radix
// select across all parts of the row instead: five launches, each one
// workgroup per (part, row), with no workgroup ever waiting for another.
// Every launch recomputes its part's keys.  Launch P (0 < P <= 3) first fixes
// digit P-1 from the sum over parts of that pass's per-part histograms and
// the state (prefix, need) the previous launch left; every workgroup of the
// row reaches the same digit, and part 0 records the new state for the next
// launch.  Launches 0-2 then write their part's histogram of pass P; launch 3,
// which has fixed K* and the number of K*-equal elements to take, writes the
// part's counts of keys above and equal to K*.  Launch 4 gives each part its
// output offset and its share of the K*-equal elements (in part order, so
// ties still go to the lower index) and writes the chosen indices.
constexpr int kWideMaxParts = 16;
constexpr int kCnt = 4096 + 2048 + 1024;       // per part: the three histograms, then (gt, eq)
constexpr int kState = kCnt + 2;               // part 0 only: state after pass p at kState + 4p
constexpr int kWideWords = kState + 12;        // per (row, part)

__device__ __forceinline__ uint32_t* wide_of(const Params& s, int row, int part) {
  return s.wide + ((int64_t)row * s.parts + part) * kWideWords;
}

// The digit of pass p from the per-part histograms of the row, given the
// prefix and need before it.  Leaves (prefix, need, all_eq) in sh.
__device__ __forceinline__ void wide_pick(const Params& s, int row, int p, uint64_t prefix,
                                          uint32_t need, uint32_t* hist, Shared& sh) {
  const int nb = pass_bins(p);
  for (int b = threadIdx.x; b < nb; b += kT) {
    uint32_t c[kWideMaxParts];
#pragma unroll
    for (int q = 0; q < kWideMaxParts; ++q)
      c[q] = q < s.parts ? wide_of(s, row, q)[pass_offset(p) + b] : 0u;
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < kWideMaxParts; ++q) v += c[q];
    hist[b] = v;
  }
  __syncthreads();
  pick_digit(hist, p, prefix, need, sh);
}

template <int T, int STAGE>
__global__ __launch_bounds__(kT) void topk_wide_kernel(Params s) {
  __shared__ uint32_t smem[LdsWords<T>::value];
  __shared__ Shared sh;
  const int row = blockIdx.y, part = blockIdx.x;
  const int p0 = part * kCap, p1 = min(p0 + kCap, s.n);
  uint64_t k[kKpt];
  uint32_t valid;
  part_keys<T>(s, row, p0, p1, smem, k, valid);
  uint32_t* mine = wide_of(s, row, part);
  uint32_t* state = wide_of(s, row, 0) + kState;
  // the state before this launch's digit, then the digit itself
  uint64_t prefix = 0;
  uint32_t need = (uint32_t)s.budget;
  if constexpr (STAGE >= 2) {
    const uint32_t* st = state + 4 * (STAGE - 2);
    prefix = ((uint64_t)st[1] << 32) | st[0];
    need = st[2];
    if constexpr (STAGE == 4) {
      if (threadIdx.x == 0) sh.all_eq = st[3];
      __syncthreads();
    }
  }
  if constexpr (STAGE >= 1 && STAGE <= 3) {
    wide_pick(s, row, STAGE - 1, prefix, need, smem, sh);
    prefix = sh.prefix;
    need = sh.need;
    if (part == 0 && threadIdx.x == 0) {
      uint32_t* st = state + 4 * (STAGE - 1);
      st[0] = (uint32_t)prefix;
      st[1] = (uint32_t)(prefix >> 32);
      st[2] = need;
      st[3] = sh.all_eq;
    }
  }
  if constexpr (STAGE < 3) {
    uint32_t* h = smem;
    for (int b = threadIdx.x; b < pass_bins(STAGE); b += kT) h[b] = 0u;
    __syncthreads();
    hist_add(h, STAGE, prefix, k, valid);
    __syncthreads();
    for (int b = threadIdx.x; b < pass_bins(STAGE); b += kT) mine[pass_offset(STAGE) + b] = h[b];
  } else if constexpr (STAGE == 3) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const bool ok = (valid >> e) & 1u;
      gt += (ok && k[e] > prefix) ? 1u : 0u;
      eq += (ok && k[e] == prefix) ? 1u : 0u;
    }
    uint32_t tot_gt, tot_eq;
    scan_excl(gt, sh, tot_gt);
    scan_excl(eq, sh, tot_eq);
    if (threadIdx.x == 0) {
      mine[kCnt] = tot_gt;
      mine[kCnt + 1] = tot_eq;
    }
  } else {
    // offset of this part's output and its share of the K*-equal elements
    uint32_t gt_before = 0, eq_before = 0;
    for (int q = 0; q < part; ++q) {
      gt_before += wide_of(s, row, q)[kCnt];
      eq_before += wide_of(s, row, q)[kCnt + 1];
    }
    const uint32_t my_eq = mine[kCnt + 1];
    const uint32_t take_eq = need > eq_before ? min(need - eq_before, my_eq) : 0u;
    const uint32_t base = gt_before + min(eq_before, need);
    uint32_t sel_eq, tot;
    const uint32_t sel = choose(k, valid, prefix, take_eq, 0u, sh, sel_eq);
    uint32_t pos = scan_excl((uint32_t)__popc(sel), sh, tot) + base;
    int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
    const int i0 = p0 + (int)threadIdx.x * kKpt;
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if ((sel >> e) & 1u) {
        if (pos < (uint32_t)s.budget) out[pos] = i0 + e;   // the counts make pos < budget
        ++pos;
      }
    if (part == 0) write_forced(s, out);
  }
}

// ------------------------------------------------------------------ DELTA page sets
// One workgroup per sequence: rho = the top K - L older pages by page score
// (ascending), then the last min(L, pages) pages, then -1.  [DELTA] key design
// 2; pages per sequence <= kCap.
__global__ __launch_bounds__(kT) void topk_delta_kernel(DeltaLaunch p) {
  __shared__ uint32_t hist[kHistWords];
  __shared__ Shared sh;
  const int b = blockIdx.x;
  const int Lb = min(max(p.L[b], 0), p.L_max);
  const int n_pages = (Lb + p.P - 1) / p.P;
  const int n_recent = min(p.L_recent, n_pages);
  const int n_cand = n_pages - n_recent;
  const int keep = min(p.K_pages - p.L_recent, n_cand);
  const float* Sb = p.S + (int64_t)b * p.n_pages_max;
  int32_t* out = p.rho + (int64_t)b * p.K_pages;
  const int i0 = (int)threadIdx.x * kKpt;
  uint64_t k[kKpt];
  uint32_t valid = 0;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool in = i0 + e < n_cand;
    valid |= in ? (1u << e) : 0u;
    k[e] = make_key(in ? Sb[i0 + e] : 0.f, false);
  }
  uint32_t sel, tot;
  if (keep >= n_cand) {
    sel = valid;
  } else if (keep == 0) {
    sel = 0;
  } else {
    uint64_t kstar;
    uint32_t need_eq;
    radix_regs(k, valid, (uint32_t)keep, hist, sh, kstar, need_eq);
    sel = choose(k, valid, kstar, need_eq, 0u, sh, tot);
  }
  uint32_t pos = scan_excl((uint32_t)__popc(sel), sh, tot);
#pragma unroll
  for (int e = 0; e < kKpt; ++e)
    if ((sel >> e) & 1u) out[pos++] = i0 + e;
  for (int i = threadIdx.x; i < p.K_pages - keep; i += kT)
    out[keep + i] = i < n_recent ? n_cand + i : -1;
}

// budget == 0: only the forced suffix.
__global__ __launch_bounds__(256) void topk_forced_kernel(int n, int n_forced,
                                                          int32_t* __restrict__ idx) {
  int32_t* out = idx + (int64_t)blockIdx.y * n_forced;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_forced; i += gridDim.x * 256)
    out[i] = n + i;
}

int parts_of(int n) { return (n + kCap - 1) / kCap; }
int stride_of(int budget) { return budget < kCap ? budget : kCap; }
int64_t cand_ld_of(int n, int budget) {
  const int64_t slots = (int64_t)parts_of(n) * stride_of(budget);
  return (slots + kCap - 1) / kCap * kCap;
}

template <int T>
void launch(const Params& s, int H, hipStream_t stream) {
  hipLaunchKernelGGL(topk_part_kernel<T>, dim3(s.parts, H), dim3(kT), 0, stream, s);
  if (s.parts > 1) hipLaunchKernelGGL(topk_merge_kernel, dim3(H), dim3(kT), 0, stream, s);
}

bool wide_path(int n, int budget) {
  const int parts = parts_of(n);
  return parts > 1 && parts <= kWideMaxParts && (int64_t)parts * stride_of(budget) > kCap;
}

template <int T>
void launch_wide(const Params& s, int H, hipStream_t stream) {
  const dim3 grid(s.parts, H);
  hipLaunchKernelGGL((topk_wide_kernel<T, 0>), grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL((topk_wide_kernel<T, 1>), grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL((topk_wide_kernel<T, 2>), grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL((topk_wide_kernel<T, 3>), grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL((topk_wide_kernel<T, 4>), grid, dim3(kT), 0, stream, s);
}

}  // namespace

size_t topk_ws_bytes(int H, int n, int budget) {
  if (budget <= 0 || parts_of(n) == 1) return 0;
  if (wide_path(n, budget))
    return align_up((size_t)H * parts_of(n) * kWideWords * sizeof(uint32_t), kWsAlign);
  return align_up((size_t)H * cand_ld_of(n, budget) * sizeof(uint64_t), kWsAlign);
}

kvs_status delta_topk_run(const DeltaLaunch& p, hipStream_t stream) {
  if (p.n_pages_max > kCap) return KVS_EUNSUPPORTED;
  hipLaunchKernelGGL(topk_delta_kernel, dim3(p.B), dim3(kT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

kvs_status select_run(const SelectCall& c, hipStream_t stream) {
  if (c.H == 0) return KVS_OK;
  if (c.budget == 0) {
    if (c.n_forced > 0)
      hipLaunchKernelGGL(topk_forced_kernel, dim3((c.n_forced + 255) / 256, c.H), dim3(256), 0,
                         stream, c.n, c.n_forced, c.idx);
    return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
  }
  Params s;
  s.S = c.S;
  s.ld = c.ld;
  s.n = c.n;
  s.prio = c.priority;
  s.pool_max = c.pool == KVS_RED_MAX;
  s.pool_r = c.pool == KVS_RED_NONE ? 0 : (c.pool_k - 1) / 2;
  s.P = c.cluster_P;
  s.theta = c.cluster_theta;
  s.r = c.cluster_r;
  s.budget = c.budget;
  s.n_forced = c.n_forced;
  s.vec = ((uintptr_t)c.S % 16 == 0) && (c.ld % 4 == 0);
  s.parts = parts_of(c.n);
  s.stride = stride_of(c.budget);
  s.cand_ld = cand_ld_of(c.n, c.budget);
  s.cand = static_cast<uint64_t*>(c.ws);
  s.wide = static_cast<uint32_t*>(c.ws);
  s.idx = c.idx;
  const bool wide = wide_path(c.n, c.budget);
  if (c.cluster_P > 0)
    wide ? launch_wide<kCluster>(s, c.H, stream) : launch<kCluster>(s, c.H, stream);
  else if (c.pool != KVS_RED_NONE)
    wide ? launch_wide<kPool>(s, c.H, stream) : launch<kPool>(s, c.H, stream);
  else
    wide ? launch_wide<kPlain>(s, c.H, stream) : launch<kPlain>(s, c.H, stream);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

// Top-k selection with stable ties and a forced suffix (kvs_topk, kvs_select).
//
// The CLAA page selects topk(scores, keep_rate) and keeps the chosen tokens at
// their original positions ("Complete flow and cost"), after a 1-D pooling of
// the scores ("Oracle construction"); the ClusterAttn page ranks the tokens
// gathered around block-max centres first and fills with the best remaining
// ones, then appends the observation window ("Method details").  Order:
// priority desc, value desc, index asc; the chosen indices come out ascending.
//
// An element's rank is decided by its class (1 = priority) and then by an
// order-preserving 32-bit map of its float32 value.  Selection runs inside
// single workgroups, so no workgroup ever waits for another:
//  stage 1  a row is cut into parts (4096 or 8192 elements for 256- or
//           512-thread workgroups when the candidates of all parts fit one
//           merge, else 16384 for 1024 threads), one workgroup per (part,
//           row).  The workgroup
//           computes its keys in registers (16 per thread; the pooling or
//           cluster transform is applied here and never stored), finds its
//           local top-`budget` and writes the chosen (key, index) pairs in
//           index order.  Every element of the global top-`budget` is in its
//           part's local top-`budget`, because fewer than `budget` elements of
//           that part precede it.
//  stage 2  one 1024-thread workgroup per row runs the same selection over the
//           candidates of all parts and writes the chosen indices.
// Both stages run the in-register selection of select_ops.h.
#include <math.h>

#include <type_traits>

#include "grid_sync.h"
#include "kvs_internal.h"
#include "select_ops.h"
#include "wave_ops.h"

namespace kvs {
namespace {

constexpr int kCap = kT * kKpt;             // keys of a 1024-thread workgroup (16384)
constexpr int kSmallT = 512;                // threads of a stage-1 workgroup on small parts
constexpr int kSmallCap = kSmallT * kKpt;   // 8192
constexpr int kTinyT = 256;                 // ... and on the smallest parts
constexpr int kTinyCap = kTinyT * kKpt;     // 4096
constexpr uint32_t kIdxMask = 0x7FFFFFFFu;

enum Transform { kPlain = 0, kPool = 1, kCluster = 2 };

template <int NT>
constexpr int stage_words() { return NT * kKpt + 2 * kSelHaloMax; }   // a part and its halo

template <int T, int NT>
struct LdsWords {
  static constexpr int staged = T == kPlain ? 0
                                : T == kPool ? stage_words<NT>()
                                             : 2 * stage_words<NT>() + 8;
  static constexpr int value = staged > kSelWords ? staged : kSelWords;
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
  int part;              // elements per stage-1 part (threads of its workgroup * kKpt)
  int parts;             // stage-1 parts per row
  int stride;            // candidate slots per part: min(budget, part)
  int64_t cand_ld;       // candidate slots per row (multiple of kCap)
  uint64_t* cand;        // [H][cand_ld] (priority << 63 | value << 31 | index)
  uint32_t* wide;        // wide path: per-(row, part) histograms and counts
  int32_t* idx;
};

// ------------------------------------------------------------------ keys
template <int NT>
__device__ __forceinline__ void stage(const float* x, int w0, int w1, float* xs) {
#pragma unroll 6
  for (int i = threadIdx.x; i < w1 - w0; i += NT) xs[i] = x[w0 + i];
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

// The 16 scores x[a0 .. a0 + 16) (a0 >= 0, a multiple of 4) with clamped
// 16-byte loads, under the same conditions as load_window.
__device__ __forceinline__ void load_page(const Params& s, const float* x, int a0, float (&v)[16]) {
  const float4* p4 = reinterpret_cast<const float4*>(x);
  const int q0 = a0 / 4, qmax = s.n / 4 - 1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 f = p4[min(q0 + q, qmax)];
    v[4 * q] = f.x;
    v[4 * q + 1] = f.y;
    v[4 * q + 2] = f.z;
    v[4 * q + 3] = f.w;
  }
}

// Pooling from the register window: element e's terms are w[e + 16 + d],
// |d| <= r <= kWin, clipped to [0, n) and taken left to right.  Terms outside
// [0, n) are replaced once by the identity of the reduction (-inf / +0, which
// leaves a left-to-right float32 sum unchanged) and NaNs are tracked in a bit
// mask, so the inner loop is a plain max or add.  R is r when known at
// compile time, else kWin with a mask on |d|.
template <int R, bool MAX>
__device__ __forceinline__ void pool_regs(const Params& s, int i0, float (&w)[kKpt + 2 * kWin],
                                          uint32_t (&o)[kKpt]) {
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
    for (int d = -R; d <= R; ++d) {
      const float z = w[e + kWin + d];
      const bool use = R < kWin || (d >= -r && d <= r);
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
    o[e] = ord_key(t < s.n ? y : 0.f);
  }
}

// Centre of the page of 16 tokens starting at a0: the argmax (lowest index)
// over its in-range tokens when the page exists, holds no NaN and its maximum
// is >= theta; else -1.
__device__ __forceinline__ int page_centre(const Params& s, const float (&v)[16], int a0) {
  float best = v[0];
  int arg = a0;
  bool nan = best != best;
#pragma unroll
  for (int j = 1; j < 16; ++j) {
    const float z = v[j];
    const bool in = a0 + j < s.n;
    nan |= in && z != z;
    if (in && z > best) {
      best = z;
      arg = a0 + j;
    }
  }
  const bool page = a0 >= 0 && a0 < s.n;
  return (page && !nan && best >= s.theta) ? arg : -1;
}

// Cluster priority with pages of 16 tokens and radius r <= 16: a thread's 16
// keys are exactly one page (i0 is page-aligned), and the centres that can
// reach them are those of its own page and of the pages on either side.
// Every thread finds its own page's centre; the neighbours' come from LDS,
// with the pages just outside the part found by the first and last threads.
template <int NT>
__device__ __forceinline__ void cluster_page_keys(const Params& s, const float* x, int i0, int p0,
                                                  int* cen, uint32_t (&o)[kKpt], uint32_t& pb) {
  const bool first = threadIdx.x == 0, last = threadIdx.x == NT - 1;
  const int ea = first ? p0 - 16 : p0 + NT * kKpt;   // the page outside the part
  const bool extra = (first && p0 > 0) || (last && ea < s.n);
  float v[16], u[16];
  load_page(s, x, i0, v);
  if (extra) load_page(s, x, ea, u);
  cen[threadIdx.x + 1] = page_centre(s, v, i0);
  if (first || last) cen[first ? 0 : NT + 1] = extra ? page_centre(s, u, ea) : -1;
  __syncthreads();
  // centre c gathers the tokens [c - r, c + r]: over this thread's 16 tokens,
  // the bits [lo, hi1) with lo = c - r - i0 and hi1 = c + r + 1 - i0 clamped
  // to [0, 16]
  const int cc[3] = {cen[threadIdx.x], cen[threadIdx.x + 1], cen[threadIdx.x + 2]};
  const int r = s.r;
  pb = 0;
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    const int lo = min(max(cc[g] - r - i0, 0), kKpt);
    const int hi1 = min(max(cc[g] + r + 1 - i0, 0), kKpt);
    const uint32_t span = hi1 > lo ? (1u << hi1) - (1u << lo) : 0u;
    pb |= cc[g] >= 0 ? span : 0u;
  }
#pragma unroll
  for (int e = 0; e < kKpt; ++e) o[e] = ord_key(i0 + e < s.n ? v[e] : 0.f);
}

// Keys of this thread's elements i0 + e (i0 = p0 + 16 * tid) of the part
// [p0, p1): value bits o[e], priority bit e of pb, and bit e of `valid` when
// i0 + e < p1.  Leaves `smem` free.  FAST takes the register-window forms of
// the pooling and cluster transforms where they apply; without it the scores
// are staged in LDS (the same keys, fewer registers).
template <int T, int NT, bool FAST = true>
__device__ __forceinline__ void part_keys(const Params& s, int row, int p0, int p1, uint32_t* smem,
                                          int* cen, uint32_t (&o)[kKpt], uint32_t& pb,
                                          uint32_t& valid) {
  const float* x = s.S + (int64_t)row * s.ld;
  const int i0 = p0 + (int)threadIdx.x * kKpt;
  valid = 0;
  pb = 0;
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
#pragma unroll
      for (int e = 0; e < kKpt; ++e) pb |= pr[min(i0 + e, s.n - 1)] != 0 ? (1u << e) : 0u;
    }
#pragma unroll
    for (int e = 0; e < kKpt; ++e) o[e] = ord_key(v[e]);
  } else if constexpr (T == kPool) {
    // pooled value over [t - r, t + r] clipped to [0, n): max (NaN if any term
    // is NaN) or the left-to-right float32 mean of the in-range terms
    if (FAST && s.pool_r <= kWin && s.vec && s.n % 4 == 0) {
      float w[kKpt + 2 * kWin];
      load_window(s, x, i0, w);
      if (s.pool_r == 3)
        s.pool_max ? pool_regs<3, true>(s, i0, w, o) : pool_regs<3, false>(s, i0, w, o);
      else
        s.pool_max ? pool_regs<kWin, true>(s, i0, w, o) : pool_regs<kWin, false>(s, i0, w, o);
      return;
    }
    float* xs = reinterpret_cast<float*>(smem);
    const int rp = s.pool_r;
    const int w0 = max(p0 - rp, 0), w1 = min(p1 + rp, s.n);
    stage<NT>(x, w0, w1, xs);
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
      o[e] = ord_key(y);
    }
    __syncthreads();
  } else {
    // cluster priority: a token is gathered when it lies within r of the
    // argmax (lowest index) of a page of P tokens whose maximum is >= theta;
    // a page holding a NaN has no centre.  Pages [qa, qb] hold every centre
    // that can reach the part.
    if (FAST && s.P == 16 && s.r <= kWin && s.vec && s.n % 4 == 0) {
      cluster_page_keys<NT>(s, x, i0, p0, cen, o, pb);
      return;
    }
    const int P = s.P, r = s.r;
    const int qa = max(p0 - r, 0) / P;
    const int qb = min(p1 - 1 + r, s.n - 1) / P;
    const int w0 = qa * P, w1 = min((qb + 1) * P, s.n);
    float* xs = reinterpret_cast<float*>(smem);
    int* pc = reinterpret_cast<int*>(smem + stage_words<NT>());
    stage<NT>(x, w0, w1, xs);
    for (int j = threadIdx.x; j <= qb - qa; j += NT) {
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
      pc[j] = (!nan && best >= s.theta) ? arg : -1;
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
          const int c = pc[u - qa];
          pr |= c >= 0 && t - c <= r && c - t <= r;
        }
      }
      pb |= pr ? (1u << e) : 0u;
      o[e] = ord_key(v);
    }
    __syncthreads();
  }
}

template <int NT>
__device__ __forceinline__ void write_forced(const Params& s, int32_t* out) {
  for (int i = threadIdx.x; i < s.n_forced; i += NT) out[s.budget + i] = s.n + i;
}

// Candidate slot i of a row is stored at cand_at(i): within each tile of kCap
// slots, slot 16t + e (key e of merge thread t) sits at (e / 2) * 2 * kT +
// 2t + e % 2, so every 16-byte load of the merge is coalesced across a wave.
__device__ __forceinline__ int64_t cand_at(int64_t i) {
  const int64_t tile = i & ~(int64_t)(kCap - 1);
  const int u = (int)(i & (kCap - 1)), t = u >> 4, e = u & 15;
  return tile + (e >> 1) * (2 * kT) + 2 * t + (e & 1);
}

// ------------------------------------------------------------------ stage 1
// Local top-`budget` of one part.  With a single part per row this is the
// final answer (indices), else the chosen (key, index) candidates.  Workgroup
// i takes part i / H of row i % H: workgroups are dealt to the XCDs in turn,
// so with H a multiple of 8 every part of a row runs on the XCD that then
// runs the row's merge workgroup, and the candidates stay in its L2.
template <int T, int NT>
__global__ __launch_bounds__(NT) void topk_part_kernel(Params s, int H) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[LdsWords<T, NT>::value];
  __shared__ int cen[T == kCluster ? NT + 2 : 1];
  __shared__ Shared sh;
  const int row = (int)(blockIdx.x % (unsigned)H), part = (int)(blockIdx.x / (unsigned)H);
  const int p0 = part * s.part, p1 = min(p0 + s.part, s.n);
  const int m = p1 - p0;
  uint32_t o[kKpt], pb, valid;
  part_keys<T, NT>(s, row, p0, p1, smem, cen, o, pb, valid);
  const uint32_t keep = (uint32_t)min(s.budget, m);
  int ph = 0;
  Kstar ks{0u, 0u, 0u};
  uint32_t gt = valid, eq = 0u;
  if (keep != (uint32_t)m) {
    ks = select_regs<NT>(o, pb, valid, keep, smem, sh, ph);
    classify(o, pb, valid, ks, gt, eq);
  }
  uint32_t pos, rank, tg, te;
  place<NT>(gt, eq, ks.need_eq, 0u, 0u, sh, ph, pos, rank, tg, te);
  const int i0 = p0 + (int)threadIdx.x * kKpt;
  if (s.parts == 1) {
    int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const bool q = (eq >> e) & 1u;
      if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) out[pos++] = i0 + e;
      rank += q;
    }
    write_forced<NT>(s, out);
  } else {
    uint64_t* c = s.cand + (int64_t)row * s.cand_ld;
    const int64_t slot0 = (int64_t)part * s.stride;
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const bool q = (eq >> e) & 1u;
      if (((gt >> e) & 1u) || (q && rank < ks.need_eq))
        c[cand_at(slot0 + pos++)] = ((uint64_t)((pb >> e) & 1u) << 63) | ((uint64_t)o[e] << 31) |
                                    (uint64_t)(uint32_t)(i0 + e);
      rank += q;
    }
  }
}

// ------------------------------------------------------------------ stage 2
// Candidates of part q of a row: min(budget, elements of the part).
__device__ __forceinline__ uint32_t part_count(const Params& s, uint32_t q) {
  if (q >= (uint32_t)s.parts) return 0u;
  const int64_t m = min((int64_t)s.part, (int64_t)s.n - (int64_t)q * s.part);
  return (uint32_t)min((int64_t)s.budget, m);
}

// Candidate keys of tile [t0, t0 + kCap) of a row (count slots in all), this
// thread's slots t0 + 16 * tid + e: slot j belongs to part j / stride and
// holds a candidate when j % stride < that part's count.
__device__ __forceinline__ void cand_keys(const Params& s, const uint64_t* c, int64_t t0,
                                          int64_t count, uint32_t (&o)[kKpt], uint32_t& pb,
                                          uint32_t (&ix)[kKpt], uint32_t& valid) {
  const int64_t i0 = t0 + (int64_t)threadIdx.x * kKpt;
  valid = 0;
  pb = 0;
  if (i0 >= count) {
#pragma unroll
    for (int e = 0; e < kKpt; ++e) o[e] = ix[e] = 0u;
    return;
  }
  const uint4* p4 = reinterpret_cast<const uint4*>(c + t0 + 2 * threadIdx.x);
#pragma unroll
  for (int q = 0; q < kKpt / 2; ++q) {
    const uint4 v = p4[q * kT];
    o[2 * q] = (v.y << 1) | (v.x >> 31);
    o[2 * q + 1] = (v.w << 1) | (v.z >> 31);
    pb |= (v.y >> 31) << (2 * q);
    pb |= (v.w >> 31) << (2 * q + 1);
    ix[2 * q] = v.x & kIdxMask;
    ix[2 * q + 1] = v.z & kIdxMask;
  }
  // one division per thread; the slots then step through at most two parts
  // (stride >= 16) or one part at a time
  const uint32_t stride = (uint32_t)s.stride, j0 = (uint32_t)i0;
  uint32_t q = j0 / stride, slot = j0 - q * stride;
  if (stride >= (uint32_t)kKpt) {
    const uint32_t c0 = part_count(s, q), c1 = part_count(s, q + 1u), b = stride - slot;
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const uint32_t u = (uint32_t)e;
      valid |= (u < b ? slot + u < c0 : u - b < c1) ? (1u << e) : 0u;
    }
  } else {
    uint32_t cq = part_count(s, q);
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      valid |= slot < cq ? (1u << e) : 0u;
      if (++slot == stride) {
        slot = 0;
        cq = part_count(s, ++q);
      }
    }
  }
}

// The final selection among the candidates of all parts of a row, by NT
// threads: as many as hold the candidates in registers (every wave runs
// every phase, filled or not, and each barrier waits for the slowest), or kT
// with the candidates re-read by tiles when they are more.
template <int NT>
__global__ __launch_bounds__(NT) void topk_merge_kernel(Params s) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kSelWords];
  __shared__ Shared sh;
  const int row = blockIdx.x;
  const uint64_t* c = s.cand + (int64_t)row * s.cand_ld;
  int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
  const int64_t count = (int64_t)s.parts * s.stride;
  uint32_t o[kKpt], ix[kKpt], pb, valid;
  int ph = 0;
  uint32_t gt, eq, pos, rank, tg, te;
  if (count <= (int64_t)NT * kKpt) {
    cand_keys(s, c, 0, count, o, pb, ix, valid);
    const Kstar ks = select_regs<NT>(o, pb, valid, (uint32_t)s.budget, hist, sh, ph);
    classify(o, pb, valid, ks, gt, eq);
    place<NT>(gt, eq, ks.need_eq, 0u, 0u, sh, ph, pos, rank, tg, te);
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const bool q = (eq >> e) & 1u;
      if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) out[pos++] = (int32_t)ix[e];
      rank += q;
    }
  } else if constexpr (NT == kT) {
    // more candidates than registers hold: every pass re-reads them by tiles
    for (int b = threadIdx.x; b < kHistWords; b += kT) hist[b] = 0u;
    uint32_t acc[5] = {0u, ~0u, 0u, ~0u, 0u};
    for (int64_t t0 = 0; t0 < count; t0 += kCap) {
      cand_keys(s, c, t0, count, o, pb, ix, valid);
      uint32_t st[5];
      class_stats<kT>(o, pb, valid, sh, st);
      acc[0] += st[0];
      acc[1] = min(acc[1], st[1]);
      acc[2] = max(acc[2], st[2]);
      acc[3] = min(acc[3], st[3]);
      acc[4] = max(acc[4], st[4]);
      __syncthreads();   // sh.r is written again by the next tile
    }
    SelectStart a = select_start(acc, (uint32_t)s.budget);
#pragma unroll 1
    for (int p = 0; p < 3 && a.hi > 0; ++p) {
      const int w = min(a.hi, pass_width(p));
      uint32_t* h = hist + pass_offset(p);
      for (int64_t t0 = 0; t0 < count; t0 += kCap) {
        cand_keys(s, c, t0, count, o, pb, ix, valid);
        hist_add(h, o, valid & (a.cls ? pb : ~pb), a.prefix, a.hi, w, p == 0);
      }
      __syncthreads();
      pick_digit(h, 1 << w, a.need, sh);
      a.hi -= w;
      a.prefix |= sh.digit << a.hi;
      a.need = sh.need;
      if (a.need == sh.cnt) break;   // the bin is taken whole: K* stops at it
    }
    const Kstar ks{a.cls, a.prefix, a.need};
    uint32_t gt_base = 0, eq_base = 0;
    for (int64_t t0 = 0; t0 < count; t0 += kCap) {
      cand_keys(s, c, t0, count, o, pb, ix, valid);
      classify(o, pb, valid, ks, gt, eq);
      place<kT>(gt, eq, ks.need_eq, gt_base, eq_base, sh, ph, pos, rank, tg, te);
#pragma unroll
      for (int e = 0; e < kKpt; ++e) {
        const bool q = (eq >> e) & 1u;
        if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) out[pos++] = (int32_t)ix[e];
        rank += q;
      }
      gt_base += tg;
      eq_base += te;
    }
  }
  write_forced<NT>(s, out);
}

// ------------------------------------------------------------------ wide rows
// Rows whose candidates would not fit one workgroup (parts * min(budget,
// kCap) > kCap, e.g. a 20% keep rate of a 128K-token row) run the selection
// across all parts of the row instead: six launches, each one workgroup per
// (part, row) of kCap elements, with no workgroup ever waiting for another.
//  launch 0  computes the part's keys (the transform runs once), stores them
//            and the part's class statistics;
//  launch 1  combines every part's statistics into the row's (the class of
//            K*, the budget left in it, the value bits still open: the same
//            start as the in-register selection), and part 0 records that
//            state; every part then writes its histogram of the first digit;
//  launch 2, 3  fix the previous digit from the sum over parts of that
//            digit's per-part histograms, record the new state (part 0) and
//            write the next digit's histogram;
//  launch 4  fixes the last digit, which settles K* and the number of
//            K*-equal elements to take, and writes the part's counts of keys
//            above and equal to K*;
//  launch 5  gives each part its output offset and its share of the K*-equal
//            elements (in part order, so ties still go to the lower index)
//            and writes the chosen indices.
// Every workgroup of a row reaches the same digits.  Workspace: per (row,
// part) statistics, counts and three histograms; per row four states and the
// stored keys (value bits and priority bits).
constexpr int kWideMaxParts = 16;
constexpr int kWStat = 8;                         // per part: class stats (5), counts (2), pad
constexpr int kPartWords = kWStat + kHistWords;   // then the three digit histograms
constexpr int kRowState = 16;                     // per row: four states of (cls, prefix, need, hi)

__device__ __forceinline__ uint32_t* wide_part(const Params& s, int row, int part) {
  return s.wide + ((int64_t)row * s.parts + part) * kPartWords;
}
__device__ __forceinline__ uint32_t* wide_state(const Params& s, int row) {
  return s.wide + (int64_t)gridDim.y * s.parts * kPartWords + (int64_t)row * kRowState;
}
__device__ __forceinline__ uint32_t* wide_keys(const Params& s, int row) {
  return s.wide + (int64_t)gridDim.y * (s.parts * kPartWords + kRowState) +
         (int64_t)row * s.parts * kCap;
}
__device__ __forceinline__ uint16_t* wide_prio(const Params& s, int row) {
  uint32_t* end = s.wide + (int64_t)gridDim.y * (s.parts * kPartWords + kRowState + s.parts * kCap);
  return reinterpret_cast<uint16_t*>(end) + (int64_t)row * s.parts * kT;
}

template <int T>
__global__ __launch_bounds__(kT) void topk_wide_keys_kernel(Params s) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[LdsWords<T, kT>::value];
  __shared__ int cen[T == kCluster ? kT + 2 : 1];
  __shared__ Shared sh;
  const int row = blockIdx.y, part = blockIdx.x;
  const int p0 = part * kCap, p1 = min(p0 + kCap, s.n);
  uint32_t o[kKpt], pb, valid;
  part_keys<T, kT>(s, row, p0, p1, smem, cen, o, pb, valid);
  const int i0 = p0 + (int)threadIdx.x * kKpt;
  uint4* k4 = reinterpret_cast<uint4*>(wide_keys(s, row) + i0);
#pragma unroll
  for (int q = 0; q < kKpt / 4; ++q) k4[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  wide_prio(s, row)[i0 / kKpt] = (uint16_t)(pb & valid);
  uint32_t st[5];
  class_stats<kT>(o, pb, valid, sh, st);
  if (threadIdx.x == 0) {
    uint32_t* w = wide_part(s, row, part);
#pragma unroll
    for (int j = 0; j < 5; ++j) w[j] = st[j];
  }
}

// The sum over parts of the per-part histograms of pass p (nb bins) into
// LDS, then the digit holding the need-th key.  Leaves (digit, need) in sh.
__device__ __forceinline__ void wide_pick(const Params& s, int row, int p, int nb, uint32_t need,
                                          uint32_t* hist, Shared& sh) {
  for (int b = threadIdx.x; b < nb; b += kT) {
    uint32_t c[kWideMaxParts];
#pragma unroll
    for (int q = 0; q < kWideMaxParts; ++q)
      c[q] = q < s.parts ? wide_part(s, row, q)[kWStat + pass_offset(p) + b] : 0u;
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < kWideMaxParts; ++q) v += c[q];
    hist[b] = v;
  }
  __syncthreads();
  pick_digit(hist, nb, need, sh);
}

template <int STAGE>
__global__ __launch_bounds__(kT) void topk_wide_kernel(Params s) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[kHistWords];
  __shared__ Shared sh;
  const int row = blockIdx.y, part = blockIdx.x;
  const int p0 = part * kCap, p1 = min(p0 + kCap, s.n);
  const int i0 = p0 + (int)threadIdx.x * kKpt;
  // the stored keys
  uint32_t o[kKpt], valid = 0;
  const uint4* k4 = reinterpret_cast<const uint4*>(wide_keys(s, row) + i0);
#pragma unroll
  for (int q = 0; q < kKpt / 4; ++q) {
    const uint4 v = k4[q];
    o[4 * q] = v.x;
    o[4 * q + 1] = v.y;
    o[4 * q + 2] = v.z;
    o[4 * q + 3] = v.w;
  }
  const uint32_t pb = wide_prio(s, row)[i0 / kKpt];
#pragma unroll
  for (int e = 0; e < kKpt; ++e) valid |= (i0 + e < p1) ? (1u << e) : 0u;
  uint32_t* state = wide_state(s, row);
  SelectStart a;
  if constexpr (STAGE == 1) {
    uint32_t st[5] = {0u, ~0u, 0u, ~0u, 0u};
    for (int q = 0; q < s.parts; ++q) {
      const uint32_t* w = wide_part(s, row, q);
      st[0] += w[0];
      st[1] = min(st[1], w[1]);
      st[2] = max(st[2], w[2]);
      st[3] = min(st[3], w[3]);
      st[4] = max(st[4], w[4]);
    }
    a = select_start(st, (uint32_t)s.budget);
  } else {
    const uint32_t* st = state + 4 * (STAGE - 2);
    a.cls = st[0];
    a.prefix = st[1];
    a.need = st[2];
    a.hi = (int)st[3];
    if (STAGE <= 4 && a.hi > 0) {
      const int w = min(a.hi, pass_width(STAGE - 2));
      wide_pick(s, row, STAGE - 2, 1 << w, a.need, smem, sh);
      a.hi -= w;
      a.prefix |= sh.digit << a.hi;
      a.need = sh.need;
    }
  }
  if (STAGE <= 4 && part == 0 && threadIdx.x == 0) {
    uint32_t* st = state + 4 * (STAGE - 1);
    st[0] = a.cls;
    st[1] = a.prefix;
    st[2] = a.need;
    st[3] = (uint32_t)a.hi;
  }
  if constexpr (STAGE <= 3) {
    if (a.hi > 0) {
      const int p = STAGE - 1;
      const int w = min(a.hi, pass_width(p));
      const int nb = 1 << w;
      uint32_t* h = smem;
      __syncthreads();   // the pick's LDS sums are read
      for (int b = threadIdx.x; b < nb; b += kT) h[b] = 0u;
      __syncthreads();
      hist_add(h, o, valid & (a.cls ? pb : ~pb), a.prefix, a.hi, w, STAGE == 1);
      __syncthreads();
      uint32_t* mine = wide_part(s, row, part) + kWStat + pass_offset(p);
      for (int b = threadIdx.x; b < nb; b += kT) mine[b] = h[b];
    }
  } else {
    const Kstar ks{a.cls, a.prefix, a.need};
    uint32_t gt, eq;
    classify(o, pb, valid, ks, gt, eq);
    int ph = 0;
    uint32_t* mine = wide_part(s, row, part);
    if constexpr (STAGE == 4) {
      uint32_t total;
      block_scan<kT>(((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(eq), sh, ph, total);
      if (threadIdx.x == 0) {
        mine[5] = total >> 16;
        mine[6] = total & 0xFFFFu;
      }
    } else {
      // offset of this part's output and its share of the K*-equal elements
      uint32_t gt_before = 0, eq_before = 0;
      for (int q = 0; q < part; ++q) {
        gt_before += wide_part(s, row, q)[5];
        eq_before += wide_part(s, row, q)[6];
      }
      uint32_t pos, rank, tg, te;
      place<kT>(gt, eq, ks.need_eq, gt_before, eq_before, sh, ph, pos, rank, tg, te);
      int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
#pragma unroll
      for (int e = 0; e < kKpt; ++e) {
        const bool q = (eq >> e) & 1u;
        if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) {
          if (pos < (uint32_t)s.budget) out[pos] = i0 + e;   // the counts make pos < budget
          ++pos;
        }
        rank += q;
      }
      if (part == 0) write_forced<kT>(s, out);
    }
  }
}

// ------------------------------------------------------------------ one launch
// Wide rows (2 to kWideMaxParts parts of kCap elements) run the whole
// selection in one launch when the grid fits on the device at once: the phases
// (class statistics, up to three digit histograms, the counts of keys above
// and equal to K*) become exchanges between the parts of a row, with every
// part's keys in registers from first to last.  An exchanged value travels as
// 16-bit fields of 64-bit words whose upper 48 bits carry the launch's tag, a
// value no earlier launch of the process used (grid_sync.h): a part stores
// its words with device-scope stores and reads the others' with device-scope
// loads until every tag matches, one memory round trip when the parts keep
// pace, and no word needs clearing between launches.  A part whose words are
// still missing when a reader's bound runs out is computed by the reader from
// the scores (its keys, then that phase's integers, identical to the owner's).
constexpr int kGridStat = 9;                      // count, then 4 x (hi, lo) of min/max
constexpr int kGridCnt = kGridStat;               // gt, eq
constexpr int kGridHist = 16;                     // the digit histograms start here
constexpr int kGridWords = kGridHist + 1024 + 2048 + 2048;   // per (row, part)
constexpr int kGridPhases = 5;                    // statistics, three digit passes, counts
constexpr int kGridCopies = 4;                    // LDS copies of a digit histogram
static_assert(kGridCopies * 2048 <= kSelWords, "the histogram copies fit a selection's LDS");

// Digit widths of the one-launch passes (10 + 11 + 11 = 32 bits in three
// passes, the widest first pass one bin per thread) and their histogram
// offsets.
__device__ __forceinline__ constexpr int grid_pass_width(int p) { return p == 0 ? 10 : 11; }
__device__ __forceinline__ constexpr int grid_pass_offset(int p) {
  return p == 0 ? 0 : p == 1 ? 1024 : 3072;
}

struct GridArgs {
  Params s;
  uint64_t* words;   // [H][parts][kGridWords]
  uint64_t tag;      // the launch's tag in the upper 48 bits
  int64_t wait_ticks;
};

template <int T>
__global__ __launch_bounds__(kT) void topk_grid_kernel(GridArgs g) {
  __shared__ __attribute__((aligned(16))) uint32_t smem[LdsWords<T, kT>::value];
  __shared__ int cen[T == kCluster ? kT + 2 : 1];
  __shared__ Shared sh;
  __shared__ uint32_t missing;   // parts whose words a reader gave up waiting for
  const Params& s = g.s;
  const int row = blockIdx.y, part = blockIdx.x;
  const uint64_t tag = g.tag;
  uint64_t* rw = g.words + (int64_t)row * s.parts * kGridWords;
  const auto word = [&](int q, int i) { return rw + (int64_t)q * kGridWords + i; };
  const auto put16 = [&](int q, int i, uint32_t v) {
    __hip_atomic_store(word(q, i), tag | (v & 0xFFFFu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  uint32_t o[kKpt], pb, valid;
  // keys of part q; in the late-part path (inside the phase loop) through
  // LDS staging, which needs fewer registers than the register windows
  const auto keys_of = [&](int q, auto fast) {
    // q opaque: the addresses are computed at each call rather than kept
    // live from the first to the last
    asm volatile("" : "+s"(q));
    const int q0 = q * kCap, q1 = min(q0 + kCap, s.n);
    part_keys<T, kT, decltype(fast)::value>(s, row, q0, q1, smem, cen, o, pb, valid);
  };
  keys_of(part, std::true_type{});
  SelectStart a{0u, 0u, 0u, 0};
  bool whole = false;   // a digit pass found its bin taken whole: K* stops there
  int ph_scan = 0;
  // Phase ph's words of part q, from the keys in o / pb / valid.
  const auto put = [&](int ph, int q) {
    if (ph == 0) {
      uint32_t st[5];
      class_stats<kT>(o, pb, valid, sh, st);
      const int j = threadIdx.x;
      if (j < kGridStat) {
        const uint32_t v = j == 0 ? st[0] : j <= 2 ? st[1] : j <= 4 ? st[2] : j <= 6 ? st[3] : st[4];
        put16(q, j, j == 0 ? v : (j & 1) ? v >> 16 : v);
      }
      __syncthreads();   // sh.r is written again by the next use
    } else if (ph <= 3) {
      const int p = ph - 1;
      const int w = min(a.hi, grid_pass_width(p));
      const int nb = 1 << w;
      // kGridCopies copies of the histogram, one per group of waves: keys
      // that crowd into a few bins then queue on kGridCopies times fewer
      // atomics each
      __syncthreads();   // smem is free (key staging, the last sums)
      for (int b = threadIdx.x; b < kGridCopies * nb; b += kT) smem[b] = 0u;
      __syncthreads();
      // the wide rows' scores are pooled or smoothed more often than not
      hist_add_runs(smem + ((threadIdx.x >> 6) % kGridCopies) * nb, o,
                    valid & (a.cls ? pb : ~pb), a.prefix, a.hi, w, p == 0);
      __syncthreads();
      for (int b = threadIdx.x; b < nb; b += kT) {
        uint32_t v = 0;
#pragma unroll
        for (int c = 0; c < kGridCopies; ++c) v += smem[c * nb + b];
        put16(q, kGridHist + grid_pass_offset(p) + b, v);
      }
    } else {
      uint32_t gt, eq, total;
      classify(o, pb, valid, Kstar{a.cls, a.prefix, a.need}, gt, eq);
      block_scan<kT>(((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(eq), sh, ph_scan, total);
      if (threadIdx.x == 0) {
        put16(q, kGridCnt, total >> 16);
        put16(q, kGridCnt + 1, total & 0xFFFFu);
      }
    }
  };
  // Reads this thread's words of phase ph into LDS: ph 0, word t of the
  // row's statistics (9 per part); ph 1-3, the sum over the parts of bin t;
  // ph 4, word t of the counts of the parts before this one.  Each load is
  // repeated until its tag matches or the bound runs out; parts then still
  // missing are marked in `missing`.
  const auto gather = [&](int ph) {
    const int t = threadIdx.x;
    const int64_t t0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    uint32_t miss = 0;
    if (ph == 0 || ph == 4) {
      const bool mine = ph == 0 ? t < kGridStat * s.parts : t < 2 * part;
      const int q = ph == 0 ? t / kGridStat : t / 2;
      const int i = ph == 0 ? t % kGridStat : kGridCnt + t % 2;
      if (mine) {
        for (;;) {
          const uint64_t x = __hip_atomic_load(word(q, i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((x >> 16) == (tag >> 16)) {
            smem[t] = (uint32_t)(x & 0xFFFFu);
            break;
          }
          if ((int64_t)__builtin_amdgcn_s_memrealtime() - t0 >= g.wait_ticks) {
            miss = 1u << q;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    } else {
      const int p = ph - 1;
      const int nb = 1 << min(a.hi, grid_pass_width(p));
      constexpr int QB = kWideMaxParts / 2;   // parts read at once
      for (int b = t; b < nb; b += kT) {
        uint32_t need = (1u << s.parts) - 1u;   // parts whose bin is not in yet
        uint32_t v = 0;
        for (;;) {
          for (int q0 = 0; q0 < s.parts; q0 += QB) {
            // QB parts' words at once: clamped addresses, no branch
            uint64_t x[QB];
#pragma unroll
            for (int k = 0; k < QB; ++k)
              x[k] = __hip_atomic_load(word(min(q0 + k, s.parts - 1), kGridHist + grid_pass_offset(p) + b),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int k = 0; k < QB; ++k) {
              const int q = q0 + k;
              if (((need >> q) & 1u) && (x[k] >> 16) == (tag >> 16)) {
                v += (uint32_t)(x[k] & 0xFFFFu);
                need &= ~(1u << q);
              }
            }
          }
          if (!need) break;
          if ((int64_t)__builtin_amdgcn_s_memrealtime() - t0 >= g.wait_ticks) {
            miss |= need;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        smem[b] = v;
      }
    }
    if (miss) atomicOr(&missing, miss);
  };
#pragma unroll 1
  for (int ph = 0; ph < kGridPhases; ++ph) {
    if (ph >= 1 && ph <= 3 && (a.hi == 0 || whole)) continue;   // K* settled (alike in every part)
    put(ph, part);
    // read the row's words; a part still missing at the bound is computed
    // here, in this part's key registers, whose own keys are computed again
    // afterwards (the transform is deterministic), and the words read again
    for (int round = 0;; ++round) {
      __syncthreads();   // smem is free; `missing` is read by nobody
      if (threadIdx.x == 0) missing = 0u;
      __syncthreads();
      gather(ph);
      __syncthreads();
      const uint32_t m = __builtin_amdgcn_readfirstlane(missing);
      if (!m || round == 1) break;   // after a round of computing, every word is in
      for (int q = 0; q < s.parts; ++q) {
        if (!((m >> q) & 1u)) continue;
        keys_of(q, std::false_type{});
        put(ph, q);
      }
      keys_of(part, std::false_type{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the words computed here are stored
      __syncthreads();
    }
    if (ph == 0) {
      uint32_t st[5] = {0u, ~0u, 0u, ~0u, 0u};
      for (int q = 0; q < s.parts; ++q) {
        const uint32_t* w = smem + kGridStat * q;
        st[0] += w[0];
        st[1] = min(st[1], (w[1] << 16) | w[2]);
        st[2] = max(st[2], (w[3] << 16) | w[4]);
        st[3] = min(st[3], (w[5] << 16) | w[6]);
        st[4] = max(st[4], (w[7] << 16) | w[8]);
      }
      a = select_start(st, (uint32_t)s.budget);
    } else if (ph <= 3) {
      // the digit from the summed histogram
      const int p = ph - 1;
      const int w = min(a.hi, grid_pass_width(p));
      pick_digit(smem, 1 << w, a.need, sh);
      a.hi -= w;
      a.prefix |= sh.digit << a.hi;
      a.need = sh.need;
      whole = a.need == sh.cnt;
    }
  }
  // this part's output offset and its share of the K*-equal keys
  const Kstar ks{a.cls, a.prefix, a.need};
  uint32_t gt_before = 0, eq_before = 0;
  for (int q = 0; q < part; ++q) {
    gt_before += smem[2 * q];
    eq_before += smem[2 * q + 1];
  }
  uint32_t gt, eq;
  classify(o, pb, valid, ks, gt, eq);
  uint32_t pos, rank, tg, te;
  place<kT>(gt, eq, ks.need_eq, gt_before, eq_before, sh, ph_scan, pos, rank, tg, te);
  const int i0 = part * kCap + (int)threadIdx.x * kKpt;
  int32_t* out = s.idx + (int64_t)row * (s.budget + s.n_forced);
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool q = (eq >> e) & 1u;
    if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) {
      if (pos < (uint32_t)s.budget) out[pos] = i0 + e;   // the counts make pos < budget
      ++pos;
    }
    rank += q;
  }
  if (part == 0) write_forced<kT>(s, out);
}

// ------------------------------------------------------------------ DELTA page sets
// One workgroup per sequence (one wave when the pages fit 16 per lane): rho =
// the top K - L older pages by page score (ascending), then the last min(L,
// pages) pages, then -1.  [DELTA] key design 2; pages per sequence <= kCap.
template <int NT>
__global__ __launch_bounds__(NT) void topk_delta_kernel(DeltaLaunch p) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kSelWords];
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
  uint32_t o[kKpt], valid = 0;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool in = i0 + e < n_cand;
    valid |= in ? (1u << e) : 0u;
    o[e] = ord_key(in ? Sb[i0 + e] : 0.f);
  }
  int ph = 0;
  Kstar ks{0u, 0u, 0u};
  uint32_t gt = valid, eq = 0u;
  if (keep == 0) {
    gt = 0u;
  } else if (keep < n_cand) {
    ks = select_regs<NT>(o, 0u, valid, (uint32_t)keep, hist, sh, ph);
    classify(o, 0u, valid, ks, gt, eq);
  }
  uint32_t pos, rank, tg, te;
  place<NT>(gt, eq, ks.need_eq, 0u, 0u, sh, ph, pos, rank, tg, te);
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool q = (eq >> e) & 1u;
    if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) out[pos++] = i0 + e;
    rank += q;
  }
  for (int i = threadIdx.x; i < p.K_pages - keep; i += NT)
    out[keep + i] = i < n_recent ? n_cand + i : -1;
}

// budget == 0: only the forced suffix.
__global__ __launch_bounds__(256) void topk_forced_kernel(int n, int n_forced,
                                                          int32_t* __restrict__ idx) {
  int32_t* out = idx + (int64_t)blockIdx.y * n_forced;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_forced; i += gridDim.x * 256)
    out[i] = n + i;
}

// kvs_topk's kept scores: val[h][e] = S[h][idx[h][e]] for the budget chosen
// entries (a bit copy), NaN for the forced suffix.
__global__ __launch_bounds__(256) void topk_values_kernel(const float* __restrict__ S, int64_t ld,
                                                          const int32_t* __restrict__ idx,
                                                          int budget, int n_forced,
                                                          float* __restrict__ val) {
  const int w = budget + n_forced;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= w) return;
  const int64_t o = (int64_t)blockIdx.y * w + e;
  val[o] = e < budget ? S[(int64_t)blockIdx.y * ld + idx[o]] : __builtin_nanf("");
}

// ------------------------------------------------------------------ host
int ceil_div(int a, int b) { return (a + b - 1) / b; }

bool wide_path(int n, int budget) {
  const int parts = ceil_div(n, kCap);
  const int stride = budget < kCap ? budget : kCap;
  return parts > 1 && parts <= kWideMaxParts && (int64_t)parts * stride > kCap;
}

// Elements per stage-1 part: the smallest of 4 096, 8 192 and 16 384 (more
// workgroups, each with fewer keys) whose parts' candidates all still fit one
// merge workgroup.
int part_of(int n, int budget) {
  if (n <= kCap || wide_path(n, budget)) return kCap;
  for (const int part : {kTinyCap, kSmallCap}) {
    const int stride = budget < part ? budget : part;
    if ((int64_t)ceil_div(n, part) * stride <= kCap) return part;
  }
  return kCap;
}

int64_t cand_ld_of(int n, int budget) {
  const int part = part_of(n, budget);
  const int stride = budget < part ? budget : part;
  const int64_t slots = (int64_t)ceil_div(n, part) * stride;
  return (slots + kCap - 1) / kCap * kCap;
}

template <int T>
void launch(const Params& s, int H, hipStream_t stream) {
  const unsigned grid = (unsigned)s.parts * (unsigned)H;
  // a single part gets only the threads its elements fill (as the merge below)
  const bool one = s.parts == 1;
  if (s.part == kTinyCap || (one && s.n <= kTinyCap))
    hipLaunchKernelGGL((topk_part_kernel<T, kTinyT>), dim3(grid), dim3(kTinyT), 0, stream, s, H);
  else if (s.part == kSmallCap || (one && s.n <= kSmallCap))
    hipLaunchKernelGGL((topk_part_kernel<T, kSmallT>), dim3(grid), dim3(kSmallT), 0, stream, s, H);
  else
    hipLaunchKernelGGL((topk_part_kernel<T, kT>), dim3(grid), dim3(kT), 0, stream, s, H);
  if (s.parts > 1) {
    const int64_t count = (int64_t)s.parts * s.stride;
    if (count <= kTinyCap)
      hipLaunchKernelGGL(topk_merge_kernel<kTinyT>, dim3(H), dim3(kTinyT), 0, stream, s);
    else if (count <= kSmallCap)
      hipLaunchKernelGGL(topk_merge_kernel<kSmallT>, dim3(H), dim3(kSmallT), 0, stream, s);
    else
      hipLaunchKernelGGL(topk_merge_kernel<kT>, dim3(H), dim3(kT), 0, stream, s);
  }
}

// The one-launch form for rows of 2 to kWideMaxParts parts of kCap elements;
// false (nothing launched) when the grid does not fit on the device at once.
template <int T>
bool launch_grid(const Params& s0, int H, void* ws, hipStream_t stream) {
  GridArgs g;
  g.s = s0;
  g.s.part = kCap;
  g.s.parts = ceil_div(s0.n, kCap);
  if (g.s.parts < 2 || g.s.parts > kWideMaxParts) return false;
  const void* fn = reinterpret_cast<const void*>(&topk_grid_kernel<T>);
  if ((int64_t)g.s.parts * H > (int64_t)grid_capacity(fn, kT)) return false;
  g.words = static_cast<uint64_t*>(ws);
  g.tag = grid_epoch() << 16;
  g.wait_ticks = grid_wait_ticks();
  hipLaunchKernelGGL((topk_grid_kernel<T>), dim3(g.s.parts, H), dim3(kT), 0, stream, g);
  return true;
}

template <int T>
void launch_wide(const Params& s, int H, hipStream_t stream) {
  const dim3 grid(s.parts, H);
  hipLaunchKernelGGL(topk_wide_keys_kernel<T>, grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL(topk_wide_kernel<1>, grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL(topk_wide_kernel<2>, grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL(topk_wide_kernel<3>, grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL(topk_wide_kernel<4>, grid, dim3(kT), 0, stream, s);
  hipLaunchKernelGGL(topk_wide_kernel<5>, grid, dim3(kT), 0, stream, s);
}

}  // namespace

size_t topk_ws_bytes(int H, int n, int budget) {
  if (budget <= 0 || n <= kCap) return 0;
  const size_t parts = (size_t)ceil_div(n, kCap);
  // the one-launch form of wide rows: tagged words per (row, part)
  const size_t grid =
      wide_path(n, budget) ? (size_t)H * parts * kGridWords * sizeof(uint64_t) : 0;
  size_t other;
  if (wide_path(n, budget)) {
    const size_t words = parts * kPartWords + kRowState + parts * kCap + parts * kT / 2;
    other = (size_t)H * words * sizeof(uint32_t);
  } else {
    other = (size_t)H * cand_ld_of(n, budget) * sizeof(uint64_t);
  }
  return align_up(grid > other ? grid : other, kWsAlign);
}

kvs_status delta_topk_run(const DeltaLaunch& p, hipStream_t stream) {
  if (p.n_pages_max > kCap) return KVS_EUNSUPPORTED;
  // one wave per sequence while its pages fit 16 per lane: no barrier waits on other waves
  if (p.n_pages_max <= 64 * kKpt)
    hipLaunchKernelGGL(topk_delta_kernel<64>, dim3(p.B), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(topk_delta_kernel<kT>, dim3(p.B), dim3(kT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

namespace {
kvs_status select_indices(const SelectCall& c, hipStream_t stream);
}

kvs_status select_run(const SelectCall& c, hipStream_t stream) {
  if (c.H == 0) return KVS_OK;
  const kvs_status st = select_indices(c, stream);
  if (st != KVS_OK || !c.val || c.budget + c.n_forced == 0) return st;
  hipLaunchKernelGGL(topk_values_kernel, dim3(ceil_div(c.budget + c.n_forced, 256), c.H), dim3(256),
                     0, stream, c.S, c.ld, c.idx, c.budget, c.n_forced, c.val);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

namespace {
kvs_status select_indices(const SelectCall& c, hipStream_t stream) {
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
  s.part = part_of(c.n, c.budget);
  s.parts = ceil_div(c.n, s.part);
  s.stride = c.budget < s.part ? c.budget : s.part;
  s.cand_ld = cand_ld_of(c.n, c.budget);
  s.cand = static_cast<uint64_t*>(c.ws);
  s.wide = static_cast<uint32_t*>(c.ws);
  s.idx = c.idx;
  const bool wide = wide_path(c.n, c.budget);
  if (!wide && (int64_t)s.parts * c.H > 0x7FFFFFFF) return KVS_EUNSUPPORTED;
  // Rows selected across all their parts: one launch when the grid fits the
  // device.  (Its exchanges cost about what a launch boundary does, 4-5 us
  // each, so rows whose candidates fit one merge keep the two launches of
  // local candidates and merge: one boundary against five exchanges.)
  if (wide) {
    const bool one = c.cluster_P > 0    ? launch_grid<kCluster>(s, c.H, c.ws, stream)
                     : c.pool != KVS_RED_NONE ? launch_grid<kPool>(s, c.H, c.ws, stream)
                                              : launch_grid<kPlain>(s, c.H, c.ws, stream);
    if (one) return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
  }
  if (c.cluster_P > 0)
    wide ? launch_wide<kCluster>(s, c.H, stream) : launch<kCluster>(s, c.H, stream);
  else if (c.pool != KVS_RED_NONE)
    wide ? launch_wide<kPool>(s, c.H, stream) : launch<kPool>(s, c.H, stream);
  else
    wide ? launch_wide<kPlain>(s, c.H, stream) : launch<kPlain>(s, c.H, stream);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}
}  // namespace

}  // namespace kvs

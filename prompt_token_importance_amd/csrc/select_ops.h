// In-register radix selection of one workgroup (shared by the top-k kernels
// and the one-launch DELTA kernel).
//
// A workgroup of NT threads holds kKpt keys per thread: an order-preserving
// 32-bit map of each float value and a class bit (1 = priority).  The
// threshold key K* of a top-`budget` selection is found by first counting the
// priority keys (which fixes the class of K*), then reducing the minimum and
// maximum value of that class: their common leading bits are shared by the
// whole class, so the radix digits (12, 11 and 10 bits, one LDS histogram
// each) cover only the bits below them; clustered values then spread over
// the histogram instead of piling into a few bins, and a narrow class needs
// fewer passes.  Ties at K* go to the lower index:
// one workgroup prefix sum of the per-thread counts of keys above and equal
// to K* gives every chosen element its output slot, so the output is
// ascending and unique.
#pragma once

#include <stdint.h>

#include "kvs_internal.h"
#include "wave_ops.h"

namespace kvs {
namespace {

constexpr int kT = 1024;                    // threads of a merge or single-part workgroup
constexpr int kWMax = kT / 64;              // waves per workgroup, at most
constexpr int kKpt = 16;                    // keys per thread

constexpr int kHistWords = 4096 + 2048 + 1024;   // one histogram per radix pass
constexpr int kList = 4096;                       // keys left after the first pass, at most
constexpr int kSelWords = kHistWords + kList;     // LDS words of a selection
constexpr uint32_t kFinish = 32;                  // lists this short are finished by one wave
__device__ __forceinline__ constexpr int pass_width(int p) { return p == 0 ? 12 : p == 1 ? 11 : 10; }
__device__ __forceinline__ constexpr int pass_offset(int p) { return p == 0 ? 0 : p == 1 ? 4096 : 6144; }

struct Shared {
  uint32_t w[2][kWMax];   // block scans: per-wave totals, the two buffers used in turn
  uint32_t r[5][kWMax];   // class statistics: per-wave partial results
  uint32_t digit, need;   // result of a digit pick: the bin and the need within it,
  uint32_t cnt;           // and the bin's count
  uint32_t list_n;        // keys compacted into the list
  uint32_t kval, need_eq; // K* found from the list
};

// The threshold of a selection: K* = (cls, value).  Every element of a higher
// class, or of class cls with a larger value, is chosen, and so are the first
// need_eq elements (in index order) of class cls with value K*.value.
struct Kstar {
  uint32_t cls, value, need_eq;
};

__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN below every number
  if (b == 0x80000000u) b = 0u;                     // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ------------------------------------------------------------------ wave and block scans
// Exclusive prefix sum of one value per thread over the workgroup, and the
// total.  The per-wave totals alternate between two LDS buffers (`ph`), so one
// barrier suffices: a buffer is written again only two scans later, after
// every thread has passed the barrier of the scan in between.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, Shared& sh, int& ph, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_scan<OpAdd>(v, 0u);
  uint32_t* w = sh.w[ph];
  ph ^= 1;
  if (lane == 63) w[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t x = w[i];
    before += i < wave ? x : 0u;
    tot += x;
  }
  total = tot;
  return before + inc - v;
}

// ------------------------------------------------------------------ radix select
// Fixes the digit of a pass from its complete histogram h of nb bins (a power
// of two, at most 4096): the bin holding the need-th matching key counted
// from the top.  Wave 0 alone: lane l owns the bins of rank [l * per,
// (l + 1) * per) from the top; a wave prefix sum finds the owner lane, whose
// bins are then spread over the lanes for a second one.  Leaves (digit, need
// within the bin, the bin's count) in sh and synchronises the workgroup.
__device__ __forceinline__ void pick_digit(const uint32_t* h, int nb, uint32_t need, Shared& sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = nb >= 64 ? nb >> 6 : 1;
    const int top = nb - lane * per;   // one past the lane's highest bin
    uint32_t ls = 0;
    if (per >= 4) {
      const uint4* h4 = reinterpret_cast<const uint4*>(h + (top - per));
      for (int k = 0; k < (per >> 2); ++k) {
        const uint4 v = h4[k];
        ls += v.x + v.y + v.z + v.w;
      }
    } else {
      for (int b = 0; b < per; ++b)
        if (top - 1 - b >= 0) ls += h[top - 1 - b];
    }
    const uint32_t inc = wave_scan<OpAdd>(ls, 0u);
    const uint64_t own = __ballot(inc - ls < need && need <= inc);
    const int L = (int)__builtin_ctzll(own);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(inc - ls), L);
    const int topL = nb - L * per;
    const uint32_t c = (lane < per && topL - 1 - lane >= 0) ? h[topL - 1 - lane] : 0u;
    const uint32_t inc2 = above + wave_scan<OpAdd>(c, 0u);
    const uint64_t hit = __ballot(lane < per && inc2 - c < need && need <= inc2);
    if (lane == (int)__builtin_ctzll(hit)) {
      sh.digit = (uint32_t)(topL - 1 - lane);
      sh.need = need - (inc2 - c);
      sh.cnt = c;
    }
  }
  __syncthreads();
}

// K* among the c <= 64 keys of list: the need-th largest, and how many of the
// keys equal to it are taken.  Wave 0 alone: lane l counts the keys above and
// at least its own.  Leaves (kval, need_eq) in sh and synchronises.
__device__ __forceinline__ void finish_list(const uint32_t* list, uint32_t c, uint32_t need,
                                            Shared& sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const bool ok = (uint32_t)lane < c;
    const uint32_t x = ok ? list[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < c; ++j) {
      const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)j);
      gt += y > x ? 1u : 0u;
      ge += y >= x ? 1u : 0u;
    }
    const uint64_t hit = __ballot(ok && gt < need && need <= ge);
    if (lane == (int)__builtin_ctzll(hit)) {
      sh.kval = x;
      sh.need_eq = need - gt;
    }
  }
  __syncthreads();
}

// Class statistics of this thread's keys (the number of priority keys and the
// (min, max) value of each class), block-reduced into out.
template <int NT>
__device__ __forceinline__ void class_stats(const uint32_t (&o)[kKpt], uint32_t pb, uint32_t valid,
                                            Shared& sh, uint32_t (&out)[5]) {
  constexpr int NW = NT / 64;
  uint32_t v[5] = {(uint32_t)__popc(pb & valid), ~0u, 0u, ~0u, 0u};
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool ok = (valid >> e) & 1u, p = (pb >> e) & 1u;
    const uint32_t x = o[e];
    v[1] = (ok && !p && x < v[1]) ? x : v[1];
    v[2] = (ok && !p && x > v[2]) ? x : v[2];
    v[3] = (ok && p && x < v[3]) ? x : v[3];
    v[4] = (ok && p && x > v[4]) ? x : v[4];
  }
  v[0] = wave_scan<OpAdd>(v[0], 0u);
  v[1] = wave_scan<OpMin>(v[1], ~0u);
  v[2] = wave_scan<OpMax>(v[2], 0u);
  v[3] = wave_scan<OpMin>(v[3], ~0u);
  v[4] = wave_scan<OpMax>(v[4], 0u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < 5; ++j) sh.r[j][wave] = v[j];
  }
  __syncthreads();
  out[0] = 0u;
  out[1] = ~0u;
  out[2] = 0u;
  out[3] = ~0u;
  out[4] = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    out[0] += sh.r[0][i];
    out[1] = min(out[1], sh.r[1][i]);
    out[2] = max(out[2], sh.r[2][i]);
    out[3] = min(out[3], sh.r[3][i]);
    out[4] = max(out[4], sh.r[4][i]);
  }
}

// Class of K*, the budget left within it, and the value bits still to be
// decided: the class's values all share the leading bits of its (min, max).
struct SelectStart {
  uint32_t cls, need, prefix;
  int hi;   // number of low value bits not yet fixed
};

__device__ __forceinline__ SelectStart select_start(const uint32_t (&st)[5], uint32_t budget) {
  SelectStart a;
  a.cls = st[0] >= budget ? 1u : 0u;
  a.need = a.cls ? budget : budget - st[0];
  const uint32_t mn = a.cls ? st[3] : st[1], mx = a.cls ? st[4] : st[2];
  a.hi = mn == mx ? 0 : 32 - __clz(mn ^ mx);
  a.prefix = a.hi == 32 ? 0u : (mn >> a.hi) << a.hi;
  return a;
}

// Adds the keys of mask cm whose bits above `hi` equal the prefix (all of
// them on the first pass) to the histogram of the digit of bits [hi - w, hi).
__device__ __forceinline__ void hist_add(uint32_t* h, const uint32_t (&o)[kKpt], uint32_t cm,
                                         uint32_t prefix, int hi, int w, bool first) {
  const int shift = hi - w;
  const uint32_t dm = (1u << w) - 1u;
#pragma unroll
  for (int e = 0; e < kKpt; ++e)
    if (((cm >> e) & 1u) && (first || ((o[e] ^ prefix) >> hi) == 0u))
      atomicAdd(&h[(o[e] >> shift) & dm], 1u);
}

// hist_add with one atomic per run of equal digits among a thread's keys
// (consecutive elements): pooled or smoothed scores put neighbours in the
// same few bins, where one atomic per key would queue on the same address.
// It costs more than it saves on unsmoothed scores.
__device__ __forceinline__ void hist_add_runs(uint32_t* h, const uint32_t (&o)[kKpt], uint32_t cm,
                                              uint32_t prefix, int hi, int w, bool first) {
  const int shift = hi - w;
  const uint32_t dm = (1u << w) - 1u;
  uint32_t cur = 0, cnt = 0;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    if (((cm >> e) & 1u) && (first || ((o[e] ^ prefix) >> hi) == 0u)) {
      const uint32_t d = (o[e] >> shift) & dm;
      if (cnt && d != cur) {
        atomicAdd(&h[cur], cnt);
        cnt = 0;
      }
      cur = d;
      ++cnt;
    }
  }
  if (cnt) atomicAdd(&h[cur], cnt);
}

// Radix select over keys held in registers.  `hist` holds kSelWords words:
// the three pass histograms, then the list.  After the first pass only the
// class keys of the chosen bin can hold K*; when they fit the list they are
// compacted into it, and the later passes read the list instead of every key.
// Once a pass finds that every key of its chosen bin is taken (the need within
// the bin equals the bin's count), K* stops at that bin: the value returned
// keeps the bits fixed so far and zeros below, so every key of the bin is at
// least K* (above it, or equal with all of them taken) and every key of a
// lower bin below it.  The chosen set is the same.
template <int NT>
__device__ __forceinline__ Kstar select_regs(const uint32_t (&o)[kKpt], uint32_t pb,
                                             uint32_t valid, uint32_t budget, uint32_t* hist,
                                             Shared& sh, int& ph) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int b = threadIdx.x; b < kHistWords / 4; b += NT) h4[b] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) sh.list_n = 0u;
  uint32_t st[5];
  class_stats<NT>(o, pb, valid, sh, st);   // its barrier also orders the clear
  SelectStart a = select_start(st, budget);
  if (a.hi == 0) return {a.cls, a.prefix, a.need};
  const uint32_t cm = valid & (a.cls ? pb : ~pb);
  int w = min(a.hi, pass_width(0));
  hist_add(hist, o, cm, a.prefix, a.hi, w, true);
  __syncthreads();
  pick_digit(hist, 1 << w, a.need, sh);
  a.hi -= w;
  a.prefix |= sh.digit << a.hi;
  a.need = sh.need;
  const uint32_t c0 = sh.cnt;
  if (a.hi == 0 || a.need == c0) return {a.cls, a.prefix, a.need};
  if (c0 <= (uint32_t)kList) {
    uint32_t* list = hist + kHistWords;
    uint32_t mm = 0;
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      mm |= (((cm >> e) & 1u) && (o[e] >> a.hi) == (a.prefix >> a.hi)) ? (1u << e) : 0u;
    const uint32_t cnt = (uint32_t)__popc(mm);
    const uint32_t inc = wave_scan<OpAdd>(cnt, 0u);
    const uint32_t wtot = __builtin_amdgcn_readlane(inc, 63);
    uint32_t base = 0;
    if ((threadIdx.x & 63) == 0 && wtot) base = atomicAdd(&sh.list_n, wtot);
    uint32_t at = __builtin_amdgcn_readlane(base, 0) + inc - cnt;
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if ((mm >> e) & 1u) list[at++] = o[e];
    __syncthreads();
    if (c0 <= kFinish) {
      finish_list(list, c0, a.need, sh);
      return {a.cls, sh.kval, sh.need_eq};
    }
#pragma unroll 1
    for (int p = 1; p < 3 && a.hi > 0; ++p) {
      w = min(a.hi, pass_width(p));
      uint32_t* h = hist + pass_offset(p);
      const int shift = a.hi - w;
      const uint32_t dm = (1u << w) - 1u;
      for (uint32_t i = threadIdx.x; i < c0; i += NT) {
        const uint32_t x = list[i];
        if (((x ^ a.prefix) >> a.hi) == 0u) atomicAdd(&h[(x >> shift) & dm], 1u);
      }
      __syncthreads();
      pick_digit(h, 1 << w, a.need, sh);
      a.hi -= w;
      a.prefix |= sh.digit << a.hi;
      a.need = sh.need;
      if (a.need == sh.cnt) break;
    }
  } else {
#pragma unroll 1
    for (int p = 1; p < 3 && a.hi > 0; ++p) {
      w = min(a.hi, pass_width(p));
      uint32_t* h = hist + pass_offset(p);
      hist_add(h, o, cm, a.prefix, a.hi, w, false);
      __syncthreads();
      pick_digit(h, 1 << w, a.need, sh);
      a.hi -= w;
      a.prefix |= sh.digit << a.hi;
      a.need = sh.need;
      if (a.need == sh.cnt) break;
    }
  }
  return {a.cls, a.prefix, a.need};
}

// ------------------------------------------------------------------ one wave
// The same selection by one wave alone (64 lanes of kKpt keys, all of one
// class; no barrier, so the other waves of the workgroup may have left):
// 8-bit digits below the leading bits the keys share, one LDS histogram of
// at most 256 bins in `hist` (the wave's own), stopping early once a bin is
// taken whole.  LDS operations of one wave take effect in program order; the
// fences keep the compiler from moving them across the phases.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ Kstar select_wave(const uint32_t (&o)[kKpt], uint32_t valid,
                                             uint32_t budget, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t mn = ~0u, mx = 0u;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool ok = (valid >> e) & 1u;
    mn = ok && o[e] < mn ? o[e] : mn;
    mx = ok && o[e] > mx ? o[e] : mx;
  }
  mn = __builtin_amdgcn_readlane(wave_scan<OpMin>(mn, ~0u), 63);
  mx = __builtin_amdgcn_readlane(wave_scan<OpMax>(mx, 0u), 63);
  int hi = mn == mx ? 0 : 32 - __clz(mn ^ mx);
  uint32_t prefix = hi == 32 ? 0u : (mn >> hi) << hi, need = budget;
  while (hi > 0) {
    const int w = hi < 8 ? hi : 8, shift = hi - w, nb = 1 << w;
    const uint32_t fixed = hi >= 32 ? 0u : ~0u << hi;   // the bits already decided
    if (4 * lane < nb) reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_fence();
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if (((valid >> e) & 1u) && ((o[e] ^ prefix) & fixed) == 0u)
        atomicAdd(&hist[(o[e] >> shift) & (uint32_t)(nb - 1)], 1u);
    wave_lds_fence();
    // lane l holds bins nb-1-4l .. nb-4-4l, the highest first
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bin = nb - 1 - 4 * lane - j;
      c[j] = bin >= 0 ? hist[bin] : 0u;
    }
    const uint32_t ls = c[0] + c[1] + c[2] + c[3];
    const uint32_t inc = wave_scan<OpAdd>(ls, 0u);
    const int L = (int)__builtin_ctzll(__ballot(inc >= need));
    uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(inc - ls), L);
    uint32_t cl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cl[j] = (uint32_t)__builtin_amdgcn_readlane((int)c[j], L);
    int j = 0;
    while (j < 3 && above + cl[j] < need) above += cl[j++];
    need -= above;
    hi = shift;
    prefix |= (uint32_t)(nb - 1 - 4 * L - j) << shift;
    wave_lds_fence();   // the reads are done before the next pass clears the bins
    if (need == cl[j]) break;   // the bin is taken whole
  }
  return {0u, prefix, need};
}

// Output slot of this lane's first chosen element and the rank of its first
// K*-equal element within one wave (place for a single wave).
__device__ __forceinline__ void place_wave(uint32_t gt, uint32_t eq, uint32_t need_eq,
                                           uint32_t& pos, uint32_t& rank) {
  const uint32_t v = ((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(eq);
  const uint32_t before = wave_scan<OpAdd>(v, 0u) - v;
  const uint32_t gb = before >> 16, eb = before & 0xFFFFu;
  pos = gb + min(eb, need_eq);
  rank = eb;
}

// Chosen-key masks of this thread: gt = above K*, eq = equal to K*.
__device__ __forceinline__ void classify(const uint32_t (&o)[kKpt], uint32_t pb, uint32_t valid,
                                         const Kstar& ks, uint32_t& gt, uint32_t& eq) {
  const uint32_t cm = valid & (ks.cls ? pb : ~pb);
  gt = ks.cls ? 0u : (valid & pb);
  eq = 0u;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool in = (cm >> e) & 1u;
    gt |= (in && o[e] > ks.value) ? (1u << e) : 0u;
    eq |= (in && o[e] == ks.value) ? (1u << e) : 0u;
  }
}

// Output slot of this thread's first chosen element and the rank of its first
// K*-equal element, from one prefix sum of the packed counts (gt << 16 | eq;
// each total is at most 16384): an element's slot is the number of keys above
// K* before it plus min(K*-equal keys before it, need_eq).  gt_base / eq_base
// count the elements of earlier tiles or parts; tot_gt / tot_eq return this
// workgroup's totals.
template <int NT>
__device__ __forceinline__ void place(uint32_t gt, uint32_t eq, uint32_t need_eq, uint32_t gt_base,
                                      uint32_t eq_base, Shared& sh, int& ph, uint32_t& pos,
                                      uint32_t& rank, uint32_t& tot_gt, uint32_t& tot_eq) {
  uint32_t total;
  const uint32_t before =
      block_scan<NT>(((uint32_t)__popc(gt) << 16) | (uint32_t)__popc(eq), sh, ph, total);
  const uint32_t gb = gt_base + (before >> 16), eb = eq_base + (before & 0xFFFFu);
  pos = gb + min(eb, need_eq);
  rank = eb;
  tot_gt = total >> 16;
  tot_eq = total & 0xFFFFu;
}

}  // namespace
}  // namespace kvs

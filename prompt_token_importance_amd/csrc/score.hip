// Window-attention column scores on gfx950 (kvs_score).
//
// Computes, per KV head g, the column sums over the window rows (and the G
// query heads sharing g) of the causally masked softmax of scale * Q K^T, as
// the ClusterAttn page defines feature aggregation ("Background and key
// observations": window logits, window mask, softmax, column sum) and the
// CLAA page defines the FastKV / per-layer window score ("Three
// representative token-ranking methods", "Three design decisions").  The
// DELTA page's max over heads ("Key design 2") is the GROUP_MAX output.
//
// Design (MI355X / CDNA4):
//  * One 32 x 32 x 16 bf16 MFMA tile = 32 keys (M) x 32 query rows (N); the
//    contraction runs over d_k.  All R = rows_pad (<= 128) query rows of the
//    group stay in VGPRs as B operands for the whole kernel; each wave streams
//    its own 32-key tiles of K straight from HBM into A operands with 16-byte
//    loads, one tile ahead.  A lane owns the contiguous d_k/2 half-row of one
//    key, so every byte of K fetched is used and no LDS staging is needed.
//  * Pass 1 keeps, per lane and query row, an online (max, sum of exp2)
//    over the keys it sees, in log2 units (x = s * scale * log2 e).  Lane
//    halves and waves are merged in LDS and written per split of the key range;
//    a small merge kernel folds the splits by log-sum-exp into one constant
//    b_r = m_r + log2 Z_r per row (+inf for padding rows).
//  * Pass 2 recomputes the tile, forms p = exp2(x - b_r) (no division), adds
//    the rows a lane holds, transposes the 32 x 32 tile of partial sums
//    through a per-wave LDS buffer and adds across lanes.  Every output element
//    is written by exactly one lane, in a fixed order: results are
//    bit-reproducible and no atomics are used.
//  * No R x L logit matrix is ever stored: K is read once per pass.
#include <math.h>

#include "kvs_internal.h"

namespace kvs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStride = 36;  // floats per row of the LDS transpose buffers
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

struct KArgs {
  ScoreLaunch p;
  int head_rows, rows_pad, n_split, tps, n_tiles, g0, min_vis;
};

__device__ __forceinline__ bf16x8 load16(const uint16_t* ptr) {
  u32x4 v = *reinterpret_cast<const u32x4*>(ptr);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D>
struct KTile {
  bf16x8 v[D / 16];
};

// Lane l holds key t0 + l%32 and the d range [(l/32) * D/2, (l/32 + 1) * D/2):
// k-step s covers d = (l/32) * D/2 + 8s + e, e < 8, i.e. MFMA k = 8 * (l/32) + e.
template <int D>
__device__ __forceinline__ void load_k(KTile<D>& kt, const uint16_t* kbase, int64_t kts, int t0,
                                       int L, int lane) {
  int t = t0 + (lane & 31);
  t = t < L ? t : L - 1;  // clamp the ragged tail; masked later
  const uint16_t* ptr = kbase + (int64_t)t * kts + (lane >> 5) * (D / 2);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kt.v[s] = load16(ptr + 8 * s);
}

// Query row fragments (B operand): N-tile T, lane l -> padded row 32T + l%32.
template <int D, int NT>
__device__ __forceinline__ void load_q(bf16x8 (&q)[NT][D / 16], int (&vis)[NT], const KArgs& a,
                                       int g, int lane) {
  const int nl = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int r = 32 * T + nl;
    const int hq = r / a.head_rows, j = r % a.head_rows;
    const bool valid = hq < a.p.G && j < a.p.W;
    const int64_t pos = a.p.q_pos0 + j;
    vis[T] = valid ? (int)(pos < (int64_t)a.p.L - 1 ? pos : (int64_t)a.p.L - 1) : -1;
    const uint16_t* qp =
        a.p.Q + (int64_t)(g * a.p.G + (valid ? hq : 0)) * a.p.qhs + (int64_t)(valid ? j : 0) * a.p.qrs +
        hl * (D / 2);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 v = load16(qp + 8 * s);
      q[T][s] = valid ? v : bf16x8{};
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void tile_logits(f32x16 (&acc)[NT], const KTile<D>& kt,
                                            const bf16x8 (&q)[NT][D / 16]) {
#pragma unroll
  for (int T = 0; T < NT; ++T) acc[T] = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int T = 0; T < NT; ++T)
      acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt.v[s], q[T][s], acc[T], 0, 0, 0);
}

// Key index of accumulator element i for lane half hl (32x32 MFMA output layout).
__device__ __forceinline__ int key_of(int i, int hl) { return 8 * (i >> 2) + 4 * hl + (i & 3); }

// ------------------------------------------------------------------ pass 1
template <int D, int NT>
__global__ __launch_bounds__(kThreads, 1) void score_stats_kernel(KArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hl = lane >> 5;
  const int g = a.g0 + blockIdx.y;
  const int split = blockIdx.x;
  const int tb = split * a.tps;
  const int te = min(tb + a.tps, a.n_tiles);
  const float c = a.p.c;

  bf16x8 q[NT][D / 16];
  int vis[NT];
  load_q<D, NT>(q, vis, a, g, lane);

  float m[NT], z[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    m[T] = kNegInf;
    z[T] = 0.f;
  }

  const uint16_t* kbase = a.p.K + (int64_t)g * a.p.khs;
  KTile<D> cur, nxt;
  int tile = tb + wave;
  if (tile < te) load_k<D>(cur, kbase, a.p.kts, tile * 32, a.p.L, lane);
  for (; tile < te; tile += kWaves) {
    const int tn = tile + kWaves;
    if (tn < te) load_k<D>(nxt, kbase, a.p.kts, tn * 32, a.p.L, lane);
    f32x16 acc[NT];
    tile_logits<D, NT>(acc, cur, q);
    const int t0 = tile * 32;
    if (t0 + 31 <= a.min_vis) {
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        float mx = acc[T][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[T][i]);
        const float mn = fmaxf(m[T], mx * c);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += ex2(fmaf(acc[T][i], c, -mn));
        z[T] = z[T] * ex2(m[T] - mn) + sum;
        m[T] = mn;
      }
    } else {
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        float v[16];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = (t0 + key_of(i, hl) <= vis[T]) ? acc[T][i] : kNegInf;
          mx = fmaxf(mx, v[i]);
        }
        const float mn = fmaxf(m[T], mx * c);
        if (mn != kNegInf) {
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += ex2(fmaf(v[i], c, -mn));
          z[T] = z[T] * ex2(m[T] - mn) + sum;
          m[T] = mn;
        }
      }
    }
    cur = nxt;
  }

  __shared__ float2 sm[kWaves][32 * NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const float m2 = __shfl_xor(m[T], 32);
    const float z2 = __shfl_xor(z[T], 32);
    const float mm = fmaxf(m[T], m2);
    const float zz = (mm == kNegInf) ? 0.f : z[T] * ex2(m[T] - mm) + z2 * ex2(m2 - mm);
    if (hl == 0) sm[wave][32 * T + nl] = make_float2(mm, zz);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < 32 * NT; r += kThreads) {
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm[w][r].x);
    float zz = 0.f;
    if (mm != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) zz += sm[w][r].y * ex2(sm[w][r].x - mm);
    }
    a.p.stats[((int64_t)g * a.n_split + split) * a.rows_pad + r] = make_float2(mm, zz);
  }
}

// ------------------------------------------------------------------ merge
__global__ __launch_bounds__(128) void score_merge_kernel(KArgs a) {
  const int g = a.g0 + blockIdx.x;
  for (int r = threadIdx.x; r < a.rows_pad; r += blockDim.x) {
    const float2* st = a.p.stats + (int64_t)g * a.n_split * a.rows_pad + r;
    float mm = kNegInf;
    for (int s = 0; s < a.n_split; ++s) mm = fmaxf(mm, st[(int64_t)s * a.rows_pad].x);
    float zz = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
      const float2 v = st[(int64_t)s * a.rows_pad];
      if (v.x != kNegInf) zz += v.y * exp2f(v.x - mm);
    }
    const int hq = r / a.head_rows, j = r % a.head_rows;
    const bool valid = hq < a.p.G && j < a.p.W && mm != kNegInf;
    a.p.rowc[(int64_t)g * a.rows_pad + r] = valid ? mm + log2f(zz) : kPosInf;
  }
}

// ------------------------------------------------------------------ pass 2
__device__ __forceinline__ void store_out(float* o, float v, int accumulate) {
  *o = accumulate ? *o + v : v;
}

// MODE 0: sum over every row of the group (GROUP_SUM).
// MODE 1: per query head sums (NONE) or their maximum (GROUP_MAX).
template <int D, int NT, int MODE>
__global__ __launch_bounds__(kThreads, 1) void score_colsum_kernel(KArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 31, hl = lane >> 5;
  const int g = a.g0 + blockIdx.y;
  const int split = blockIdx.x;
  const int tb = split * a.tps;
  const int te = min(tb + a.tps, a.n_tiles);
  const float c = a.p.c;
  const int L = a.p.L;

  bf16x8 q[NT][D / 16];
  int vis[NT];
  load_q<D, NT>(q, vis, a, g, lane);
  float b[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) b[T] = a.p.rowc[(int64_t)g * a.rows_pad + 32 * T + nl];

  __shared__ float tr[kWaves][32 * kStride];
  __shared__ float hacc[MODE == 1 ? kWaves : 1][MODE == 1 ? 32 * 32 : 1];
  float* wl = tr[wave];

  const uint16_t* kbase = a.p.K + (int64_t)g * a.p.khs;
  KTile<D> cur, nxt;
  int tile = tb + wave;
  if (tile < te) load_k<D>(cur, kbase, a.p.kts, tile * 32, L, lane);
  for (; tile < te; tile += kWaves) {
    const int tn = tile + kWaves;
    if (tn < te) load_k<D>(nxt, kbase, a.p.kts, tn * 32, L, lane);
    f32x16 acc[NT];
    tile_logits<D, NT>(acc, cur, q);
    const int t0 = tile * 32;
    const bool full = t0 + 31 <= a.min_vis;
    float p[NT][16];
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = ex2(fmaf(acc[T][i], c, -b[T]));
        p[T][i] = (full || t0 + key_of(i, hl) <= vis[T]) ? e : 0.f;
      }
    const int k = lane & 31;
    const int t = t0 + k;
    if constexpr (MODE == 0) {
      float part[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = p[0][i];
#pragma unroll
        for (int T = 1; T < NT; ++T) s += p[T][i];
        part[i] = s;
      }
#pragma unroll
      for (int aa = 0; aa < 4; ++aa)
        *reinterpret_cast<f32x4*>(&wl[nl * kStride + 8 * aa + 4 * hl]) =
            f32x4{part[4 * aa], part[4 * aa + 1], part[4 * aa + 2], part[4 * aa + 3]};
      lds_order();
      float v = 0.f;
#pragma unroll
      for (int n = 0; n < 16; ++n) v += wl[(16 * hl + n) * kStride + k];
      v += __shfl_xor(v, 32);
      if (hl == 0 && t < L) store_out(a.p.S + (int64_t)g * a.p.s_ld + t, v, a.p.accumulate);
      lds_order();
    } else {
      float* ha = hacc[wave];
      for (int x = lane; x < a.p.G * 32; x += 64) ha[x] = 0.f;
#pragma unroll
      for (int T = 0; T < NT; ++T) {
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
          *reinterpret_cast<f32x4*>(&wl[nl * kStride + 8 * aa + 4 * hl]) =
              f32x4{p[T][4 * aa], p[T][4 * aa + 1], p[T][4 * aa + 2], p[T][4 * aa + 3]};
        lds_order();
        const int r0 = 32 * T;
        const int h_first = r0 / a.head_rows;
        int h_last = (r0 + 31) / a.head_rows;
        h_last = h_last < a.p.G - 1 ? h_last : a.p.G - 1;
        for (int hq = h_first; hq <= h_last; ++hq) {
          if ((hq & 1) != hl) continue;
          int lo = hq * a.head_rows, hi = lo + a.p.W;
          lo = lo > r0 ? lo : r0;
          hi = hi < r0 + 32 ? hi : r0 + 32;
          float v = 0.f;
          for (int r = lo; r < hi; ++r) v += wl[(r - r0) * kStride + k];
          ha[hq * 32 + k] += v;
        }
        lds_order();
      }
      if (a.p.heads == KVS_HEADS_NONE) {
        for (int hq = hl; hq < a.p.G; hq += 2)
          if (t < L)
            store_out(a.p.S + (int64_t)(g * a.p.G + hq) * a.p.s_ld + t, ha[hq * 32 + k],
                      a.p.accumulate);
      } else {
        float mx = kNegInf;
        for (int hq = hl; hq < a.p.G; hq += 2) mx = fmaxf(mx, ha[hq * 32 + k]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (hl == 0 && t < L) store_out(a.p.S + (int64_t)g * a.p.s_ld + t, mx, a.p.accumulate);
      }
      lds_order();
    }
    cur = nxt;
  }
}

template <int D, int NT>
kvs_status launch_rounds(const ScorePlan& pl, const ScoreLaunch& p, hipStream_t stream) {
  for (int g0 = 0; g0 < p.H_kv; g0 += pl.head_batch) {
    const int nb = min(pl.head_batch, p.H_kv - g0);
    KArgs a;
    a.p = p;
    a.head_rows = pl.head_rows;
    a.rows_pad = pl.rows_pad;
    a.n_split = pl.n_split;
    a.tps = pl.tiles_per_split;
    a.n_tiles = pl.n_tiles;
    a.g0 = g0;
    const int64_t mv = p.q_pos0 < (int64_t)p.L - 1 ? p.q_pos0 : (int64_t)p.L - 1;
    a.min_vis = (int)mv;
    dim3 grid(pl.n_split, nb);
    hipLaunchKernelGGL((score_stats_kernel<D, NT>), grid, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(score_merge_kernel, dim3(nb), dim3(128), 0, stream, a);
    if (p.heads == KVS_HEADS_GROUP_SUM)
      hipLaunchKernelGGL((score_colsum_kernel<D, NT, 0>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((score_colsum_kernel<D, NT, 1>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

template <int D>
kvs_status launch_d(const ScorePlan& pl, const ScoreLaunch& p, hipStream_t stream) {
  switch (pl.rows_pad / 32) {
    case 1: return launch_rounds<D, 1>(pl, p, stream);
    case 2: return launch_rounds<D, 2>(pl, p, stream);
    case 3: return launch_rounds<D, 3>(pl, p, stream);
    case 4: return launch_rounds<D, 4>(pl, p, stream);
    default: return KVS_EUNSUPPORTED;
  }
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

}  // namespace

kvs_status score_plan(const kvs_score_args* a, ScorePlan* pl) {
  const int G = a->H_q / a->H_kv;
  const int W = a->W;
  const int hr = W <= 4 ? 4 : W <= 8 ? 8 : W <= 16 ? 16 : (W + 31) / 32 * 32;
  if ((int64_t)G * hr > 128) return KVS_EUNSUPPORTED;
  pl->head_rows = hr;
  pl->rows_pad = (G * hr + 31) / 32 * 32;
  pl->n_tiles = (a->L + 31) / 32;
  // KV heads per round: a round's K is re-read by pass 2 soon after pass 1
  // streamed it, so a round sized below the 256 MB Infinity Cache can serve
  // the second read from the cache.  Tunable for measurement.
  const int64_t head_bytes = (int64_t)a->L * a->d_k * 2;
  int batch = env_int("KVS_SCORE_HEAD_BATCH", 0);
  if (batch <= 0) batch = a->H_kv;
  (void)head_bytes;
  batch = batch < a->H_kv ? batch : a->H_kv;
  pl->head_batch = batch;
  // Splits of the key range: about two 4-wave workgroups per CU per launch,
  // and at least 4 tiles (one per wave) per split.
  const int target_wg = env_int("KVS_SCORE_TARGET_WG", 512);
  int per_head = (target_wg + batch - 1) / batch;
  int max_split = pl->n_tiles / 4 > 1 ? pl->n_tiles / 4 : 1;
  int ns = per_head < max_split ? per_head : max_split;
  if (ns < 1) ns = 1;
  const int tps = (pl->n_tiles + ns - 1) / ns;
  pl->tiles_per_split = tps;
  pl->n_split = (pl->n_tiles + tps - 1) / tps;
  pl->ws_stats = align_up((size_t)a->H_kv * pl->n_split * pl->rows_pad * sizeof(float2), kWsAlign);
  pl->ws_rowc = align_up((size_t)a->H_kv * pl->rows_pad * sizeof(float), kWsAlign);
  pl->ws_total = pl->ws_stats + pl->ws_rowc;
  return KVS_OK;
}

kvs_status score_run(const ScorePlan& pl, const ScoreLaunch& p, hipStream_t stream) {
  if (p.d_k == 128) return launch_d<128>(pl, p, stream);
  if (p.d_k == 64) return launch_d<64>(pl, p, stream);
  return KVS_EUNSUPPORTED;
}

}  // namespace kvs

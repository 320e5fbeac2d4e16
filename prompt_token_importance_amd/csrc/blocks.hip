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
#include "wave_ops.h"

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

// Probability mass in fixed point, 2^-30 units, summed exactly with 32-bit
// integer adds: each term is truncated by less than 2^-30, the total stays
// below 2^31.
constexpr float kMassOne = 1073741824.0f;
__device__ __forceinline__ uint32_t mass_of(float p) { return (uint32_t)(p * kMassOne); }
// The 44-bit order key of block j: probability bits, then 4095 - j (ties go
// to the lower block index).
__device__ __forceinline__ uint64_t key44(uint32_t o, int j) {
  return ((uint64_t)o << 12) | (uint64_t)(4095 - j);
}

constexpr int kPerThread = kMaxKvb / kThreads;   // key blocks per thread
constexpr uint32_t kTopFinish = 32;              // crossing bins this small: one wave finishes

struct ToppShared {
  uint32_t hm[2048];          // mass histogram of one 11-bit digit
  uint32_t lo[kMaxKvb];       // keys of the crossing bin: probability bits
  uint16_t lj[kMaxKvb];       //   and block index
  float red[2][kThreads / 64];
  uint32_t digit, need, found, n;
  uint64_t kstar;
};

// Wave 0 fixes the digit whose bin holds the need-th unit of mass counted
// from the top of histogram hm (2048 bins): lane l owns 32 bins; a wave
// prefix sum of their masses finds the owner lane, whose bins are then spread
// over the lanes for a second one.  found = 0 when the histogram's whole mass
// is below need.  The caller synchronises.
__device__ __forceinline__ void topp_pick(ToppShared& sh, uint32_t need) {
  const int lane = threadIdx.x & 63;
  const int top = 2048 - 32 * lane;   // one past the lane's highest bin
  const uint4* h4 = reinterpret_cast<const uint4*>(sh.hm + top - 32);
  uint32_t ls = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 v = h4[k];
    ls += v.x + v.y + v.z + v.w;
  }
  const uint32_t inc = wave_scan<OpAdd>(ls, 0u);
  const uint64_t own = __ballot(inc - ls < need && need <= inc);
  if (own == 0) {
    if (lane == 0) sh.found = 0u;
    return;
  }
  const int L = (int)__builtin_ctzll(own);
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(inc - ls), L);
  const int topL = 2048 - 32 * L;
  const uint32_t c = lane < 32 ? sh.hm[topL - 1 - lane] : 0u;
  const uint32_t inc2 = above + wave_scan<OpAdd>(c, 0u);
  const uint64_t hit = __ballot(lane < 32 && inc2 - c < need && need <= inc2);
  if (lane == (int)__builtin_ctzll(hit)) {
    sh.digit = (uint32_t)(topL - 1 - lane);
    sh.need = need - (inc2 - c);
    sh.found = 1u;
  }
}

// ------------------------------------------------------------------ top-p per (head, query block)
// One workgroup per (head, query block); thread t holds key blocks t + 256 u,
// u < PT, with PT the fewest of 4, 8 and 16 that cover the KV blocks (every
// slot is worked through in every phase, filled or not).
// Softmax over the visible blocks with wave and workgroup reductions in a
// fixed order.  The kept blocks are a prefix of the order (probability desc,
// j asc): a block is kept while the mass ranked strictly before it is <
// p_mass, so the prefix ends at the block K* where the running mass first
// reaches p_mass.  K* is found by a radix select over the 44-bit key with
// per-digit histograms of mass instead of counts: the first 11-bit digit over
// all keys, then the keys of the crossing bin are compacted into a list; a
// short list is finished by one wave (each lane sums the mass of the keys
// above its own), a long one by three more digits over the list.
template <int PT>
__global__ __launch_bounds__(kThreads) void block_topp_kernel(
    const float* __restrict__ logit, int n_qb, int n_kvb, int block, int Lq,
    int64_t q_pos0, float p_mass, uint8_t* __restrict__ M) {
  __shared__ __attribute__((aligned(16))) ToppShared sh;
  const int i = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t last_row = min((int64_t)(i + 1) * block, (int64_t)Lq) - 1;
  const int64_t end_pos = q_pos0 + last_row;
  const float* lr = logit + ((int64_t)h * n_qb + i) * n_kvb;
  // 1. logits of the visible blocks and their maximum
  float v[PT];
  uint32_t vis = 0;
  float mloc = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int j = tid + kThreads * u;
    const bool in = j < n_kvb && (int64_t)j * block <= end_pos;
    v[u] = in ? lr[j] : -__builtin_inff();
    vis |= in ? (1u << u) : 0u;
    mloc = fmaxf(mloc, v[u]);
  }
  uint4* h4 = reinterpret_cast<uint4*>(sh.hm);
  for (int b = tid; b < 2048 / 4; b += kThreads) h4[b] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) sh.n = 0u;
  mloc = __uint_as_float(wave_scan<OpMaxF>(__float_as_uint(mloc), __float_as_uint(-__builtin_inff())));
  if (lane == 63) sh.red[0][wave] = mloc;
  __syncthreads();
  float mx = sh.red[0][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) mx = fmaxf(mx, sh.red[0][w]);
  // 2. softmax numerators and their sum
  float sloc = 0.f;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const float e = ((vis >> u) & 1u) ? expf(v[u] - mx) : 0.f;
    v[u] = e;
    sloc += e;
  }
  sloc = __uint_as_float(wave_scan<OpAddF>(__float_as_uint(sloc), 0u));
  if (lane == 63) sh.red[1][wave] = sloc;
  __syncthreads();
  float z = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) z += sh.red[1][w];
  const float inv_z = 1.0f / z;
  uint32_t o[PT];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    v[u] *= inv_z;   // probability
    o[u] = ord_pos(v[u]);
  }
  // 3. first digit: the 11 leading bits of the key (o >> 21), over every key
  const uint32_t need0 = (uint32_t)((double)p_mass * 1073741824.0);
#pragma unroll
  for (int u = 0; u < PT; ++u)
    if ((vis >> u) & 1u) atomicAdd(&sh.hm[o[u] >> 21], mass_of(v[u]));
  __syncthreads();
  if (wave == 0) topp_pick(sh, need0);
  __syncthreads();
  const bool all = sh.found == 0u;   // the whole mass stays below p_mass: keep every visible block
  uint64_t kstar = 0;
  if (!all) {
    const uint32_t d0 = sh.digit;
    uint32_t need = sh.need;
#pragma unroll
    for (int u = 0; u < PT; ++u)
      if (((vis >> u) & 1u) && (o[u] >> 21) == d0) {
        const uint32_t at = atomicAdd(&sh.n, 1u);
        sh.lo[at] = o[u];
        sh.lj[at] = (uint16_t)(tid + kThreads * u);
      }
    __syncthreads();
    const uint32_t n = sh.n;
    if (n <= kTopFinish) {
      if (wave == 0) {
        const bool ok = (uint32_t)lane < n;
        const uint32_t x = ok ? sh.lo[lane] : 0u;
        const int jx = ok ? (int)sh.lj[lane] : 0;
        const uint32_t mxs = mass_of(__uint_as_float(x & 0x7FFFFFFFu));
        uint32_t above = 0;   // mass of the list keys above this lane's key
        for (uint32_t y = 0; y < n; ++y) {
          const uint32_t xy = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)y);
          const int jy = __builtin_amdgcn_readlane(jx, (int)y);
          const uint32_t my = (uint32_t)__builtin_amdgcn_readlane((int)mxs, (int)y);
          above += (xy > x || (xy == x && jy < jx)) ? my : 0u;
        }
        const uint64_t hit = __ballot(ok && above < need && need <= above + mxs);
        if (lane == (int)__builtin_ctzll(hit)) sh.kstar = key44(x, jx);
      }
      __syncthreads();
      kstar = sh.kstar;
    } else {
      uint64_t prefix = (uint64_t)d0 << 33;
#pragma unroll 1
      for (int pass = 1; pass < 4; ++pass) {
        const int shift = 33 - 11 * pass;
        for (int b = tid; b < 2048 / 4; b += kThreads) h4[b] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        for (uint32_t idx = tid; idx < n; idx += kThreads) {
          const uint32_t x = sh.lo[idx];
          const uint64_t key = key44(x, sh.lj[idx]);
          if ((key >> (shift + 11)) == (prefix >> (shift + 11)))
            atomicAdd(&sh.hm[(key >> shift) & 2047u], mass_of(__uint_as_float(x & 0x7FFFFFFFu)));
        }
        __syncthreads();
        if (wave == 0) topp_pick(sh, need);
        __syncthreads();
        prefix |= (uint64_t)sh.digit << shift;
        need = sh.need;
      }
      kstar = prefix;
    }
  }
  // 4. keep the visible blocks at or above K* (every visible block when `all`)
  uint8_t* mrow = M + ((int64_t)h * n_qb + i) * n_kvb;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int j = tid + kThreads * u;
    if (j < n_kvb) mrow[j] = (((vis >> u) & 1u) && (all || key44(o[u], j) >= kstar)) ? 1 : 0;
  }
}

// ------------------------------------------------------------------ union
// OR over the heads and query blocks of a (sub)group, then an ascending CSR.
// union_group_kernel: one workgroup per (segment of kSeg KV blocks, group).
// Thread t reads 16 blocks (one 16-byte chunk, t % 8) of the rows t / 8,
// t / 8 + 32, ...; the partial ORs are combined across the lanes of a wave
// that share a chunk (shuffles), then across the waves in LDS, and wave 0
// writes the segment's set blocks in ascending order with their count.
// union_pack_kernel: one workgroup per (segment, group) piece adds up the
// counts of the pieces before it (groups in order, segments in order) and
// copies the piece's blocks to its place in the CSR.
constexpr int kSeg = 128;             // KV blocks per union segment
constexpr int kSegChunks = kSeg / 16; // 16-byte chunks per segment row

__global__ __launch_bounds__(kThreads) void union_group_kernel(const uint8_t* __restrict__ M,
                                                               int sg, int n_qb, int n_kvb,
                                                               int32_t* __restrict__ staging,
                                                               int32_t* __restrict__ counts) {
  __shared__ u32x4 part[kThreads / 64][kSegChunks];
  const int seg = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % kSegChunks, rl = tid / kSegChunks;
  const int j0 = seg * kSeg + 16 * c;   // first KV block of this thread's chunk
  const int nrows = sg * n_qb;
  const uint8_t* base = M + (int64_t)g * nrows * n_kvb;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (j0 < n_kvb) {
    if (n_kvb % 16 == 0 && ((uintptr_t)M & 15u) == 0) {
#pragma unroll 4
      for (int r = rl; r < nrows; r += kThreads / kSegChunks)
        acc |= *reinterpret_cast<const u32x4*>(base + (int64_t)r * n_kvb + j0);
    } else {
      for (int r = rl; r < nrows; r += kThreads / kSegChunks)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (j0 + e < n_kvb && base[(int64_t)r * n_kvb + j0 + e])
            acc[e / 4] |= 0xffu << (8 * (e % 4));
    }
  }
  // lanes l, l ^ 8, l ^ 16, ... of a wave hold the same chunk
#pragma unroll
  for (int d = kSegChunks; d < 64; d *= 2)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] |= (uint32_t)__shfl_xor((int)acc[q], d);
  if (lane < kSegChunks) part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    uint32_t bits = 0;
    if (lane < kSegChunks) {
      u32x4 o = part[0][lane];
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) o |= part[w][lane];
#pragma unroll
      for (int e = 0; e < 16; ++e) bits |= ((o[e / 4] >> (8 * (e % 4))) & 0xffu) ? (1u << e) : 0u;
    }
    const uint32_t cnt = (uint32_t)__popc(bits);
    const uint32_t inc = wave_scan<OpAdd>(cnt, 0u);
    uint32_t pos = inc - cnt;
    int32_t* st = staging + (int64_t)g * n_kvb + seg * kSeg;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((bits >> e) & 1u) st[pos++] = j0 + e;
    if (lane == 63) counts[(int64_t)g * gridDim.x + seg] = (int32_t)inc;
  }
}

__global__ __launch_bounds__(kThreads) void union_pack_kernel(const int32_t* __restrict__ staging,
                                                              const int32_t* __restrict__ counts,
                                                              int n_groups, int n_kvb,
                                                              int32_t* __restrict__ indptr,
                                                              int32_t* __restrict__ indices) {
  __shared__ uint32_t wsum[kThreads / 64];
  const int seg = blockIdx.x, g = blockIdx.y, n_seg = gridDim.x;
  const int64_t piece = (int64_t)g * n_seg + seg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t before = 0;
  for (int64_t x = tid; x < piece; x += kThreads) before += (uint32_t)counts[x];
  before = wave_scan<OpAdd>(before, 0u);
  if (lane == 63) wsum[wave] = before;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) off += wsum[w];
  const int c = counts[piece];
  const int32_t* st = staging + (int64_t)g * n_kvb + seg * kSeg;
  for (int x = tid; x < c; x += kThreads) indices[off + x] = st[x];
  if (tid == 0) {
    if (seg == 0) indptr[g] = (int32_t)off;
    if (g == n_groups - 1 && seg == n_seg - 1) indptr[n_groups] = (int32_t)(off + c);
  }
}

// ------------------------------------------------------------------ token page tables
// kvs_token_pagetable: the pages of kept token positions, per group of rows.
// A zeroed byte mask [group][page] (rows padded to 16 pages) is set by one
// thread per list entry (threads that hit the same page store the same byte),
// then lowered to CSR by the union kernels with one query block per group.
__global__ __launch_bounds__(kThreads) void zero16_kernel(u32x4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(kThreads) void token_pages_kernel(const int32_t* __restrict__ idx,
                                                               int n, int64_t idx_ld, int rpg,
                                                               int P, int n_pages, int64_t row_ld,
                                                               uint8_t* __restrict__ mask) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= n) return;
  const int i = idx[(int64_t)h * idx_ld + e];
  if (i >= 0 && i / P < n_pages) mask[(int64_t)(h / rpg) * row_ld + i / P] = 1;
}

}  // namespace

size_t token_pagetable_ws_bytes(int H, int rpg, int n_pages) {
  const int n_groups = H / rpg;
  const int ld = (n_pages + 15) / 16 * 16;
  return align_up((size_t)n_groups * ld, kWsAlign) + union_ws_bytes(n_groups, n_groups, 1, ld);
}

kvs_status token_pagetable_run(const int32_t* idx, int H, int n, int64_t idx_ld, int rpg, int P,
                               int n_pages, int32_t* indptr, int32_t* indices, void* ws,
                               hipStream_t stream) {
  const int n_groups = H / rpg;
  const int ld = (n_pages + 15) / 16 * 16;
  uint8_t* mask = static_cast<uint8_t*>(ws);
  void* uws = static_cast<char*>(ws) + align_up((size_t)n_groups * ld, kWsAlign);
  const int64_t n16 = (int64_t)n_groups * ld / 16;
  const int zb = (int)((n16 + kThreads - 1) / kThreads < 1024 ? (n16 + kThreads - 1) / kThreads : 1024);
  hipLaunchKernelGGL(zero16_kernel, dim3(zb), dim3(kThreads), 0, stream,
                     reinterpret_cast<u32x4*>(mask), n16);
  if (n > 0)
    hipLaunchKernelGGL(token_pages_kernel, dim3((n + kThreads - 1) / kThreads, H), dim3(kThreads), 0,
                       stream, idx, n, idx_ld, rpg, P, n_pages, (int64_t)ld, mask);
  if (hipGetLastError() != hipSuccess) return KVS_EHIP;
  return union_run(mask, n_groups, n_groups, 1, 1, ld, indptr, indices, uws, stream);
}

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
  const auto topp = pl.n_kvb <= 4 * kThreads   ? &block_topp_kernel<4>
                    : pl.n_kvb <= 8 * kThreads ? &block_topp_kernel<8>
                                               : &block_topp_kernel<kPerThread>;
  hipLaunchKernelGGL(topp, dim3(pl.n_qb, a->H_q), dim3(kThreads), 0, stream, logit, pl.n_qb,
                     pl.n_kvb, a->block, a->Lq, a->q_pos0, a->p_mass, M);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

size_t union_ws_bytes(int H_q, int H_kv, int sub_group, int n_kvb) {
  const int G = H_q / H_kv;
  const int sg = sub_group == 0 ? G : sub_group;
  const int n_groups = H_q / sg;
  const int n_seg = (n_kvb + kSeg - 1) / kSeg;
  return align_up((size_t)n_groups * n_kvb * sizeof(int32_t), kWsAlign) +
         align_up((size_t)n_groups * n_seg * sizeof(int32_t), kWsAlign);
}

kvs_status union_run(const uint8_t* M, int H_q, int H_kv, int sub_group, int n_qb, int n_kvb,
                     int32_t* indptr, int32_t* indices, void* ws, hipStream_t stream) {
  const int G = H_q / H_kv;
  const int sg = sub_group == 0 ? G : sub_group;
  const int n_groups = H_q / sg;
  int32_t* staging = static_cast<int32_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(
      static_cast<char*>(ws) + align_up((size_t)n_groups * n_kvb * sizeof(int32_t), kWsAlign));
  const int n_seg = (n_kvb + kSeg - 1) / kSeg;
  hipLaunchKernelGGL(union_group_kernel, dim3(n_seg, n_groups), dim3(kThreads), 0, stream, M, sg,
                     n_qb, n_kvb, staging, counts);
  hipLaunchKernelGGL(union_pack_kernel, dim3(n_seg, n_groups), dim3(kThreads), 0, stream, staging,
                     counts, n_groups, n_kvb, indptr, indices);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

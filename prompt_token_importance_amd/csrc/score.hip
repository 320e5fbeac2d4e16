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
//    group stay in AGPRs as B operands for the whole kernel.  One 4-wave
//    workgroup per CU; each wave streams its own 32-key tiles of K through a
//    4-stage LDS ring with direct-to-LDS 16-byte loads (every load instruction
//    reads one contiguous 1 KiB run; rows are XOR-swizzled so the fragment
//    reads are bank-conflict free).
//  * Full tiles run a software pipeline: while the matrix cores compute tile
//    j's logits (all N-tiles, k-major, fragments in AGPRs), the VALU works on
//    tile j-1's logits, two of them per MFMA slot; tile j+3's loads go out
//    together in the first slot and tile j+1's fragments are read together
//    after the wait in the middle one.  Causally masked and ragged tiles take
//    a separate exact path.
//  * Pass 1 keeps, per lane and query row, sums of exp2(x - m) over the keys
//    it sees, in log2 units (x = s * scale * log2 e), against a max m fixed
//    from the wave's first tile, so the pipeline carries no branch; a wave
//    with a sum past 2^100 redoes its tiles with the exact online update.  Lane halves and waves are merged in LDS and written per split
//    of the key range; each pass-2 workgroup folds the splits of its group's
//    rows by log-sum-exp into one constant b_r = m_r + log2 Z_r per row (+inf
//    for padding rows) before its tile loop.
//  * Pass 2 recomputes the tile with the MFMA operands swapped, so a lane
//    holds one key against 16 rows of each row tile, and a ninth k-step adds
//    each row's -b_r (scaled and split into three bf16 parts) to its logits on
//    the matrix cores.  It forms p = exp2(c * acc) (no division), sums the
//    rows of the group, or of each head, inside the lane and across the two
//    lane halves, and stores one score per key (per head, or their maximum).
//    Every output element is written by exactly one lane, in a fixed order:
//    results are bit-reproducible and no atomics are used.
//  * No R x L logit matrix is ever stored: K is read once per pass.
#include <math.h>


#include <type_traits>

#include "kvs_internal.h"
#include "grid_sync.h"
#include "select_ops.h"

namespace kvs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;   // K tiles per wave in the LDS ring
static_assert((kStages & (kStages - 1)) == 0, "ring stages are indexed with a mask");
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// One launch covers the padded query rows [row0, row0 + 32 * NT) of every KV
// group (a row group: all of them when the padded rows fit 128, else one of
// two), the query heads [h0, h1) of each group.
struct KArgs {
  ScoreLaunch p;
  int head_rows, rows_pad, n_split, tps, n_tiles, g0, min_vis;
  int rev;        // pass 2 walks each wave's tiles last to first
  int row0;       // first padded row of this row group
  int h0, h1;     // query heads (inside the KV group) whose rows this launch holds
  int acc;        // column sums: 0 store, 1 add
  int per_head;   // MODE 1: 1 writes each head's row, 0 the maximum over the heads
  float* out;     // output rows (S, or the per-group / per-head workspace rows)
  int64_t out_ld;
  uint64_t* flag;     // fused launch: one word per (KV head, split), [H_kv][n_split]
  uint64_t epoch;     // this launch's tag, stored in a flag once its split is published
  int64_t wait_ticks; // bound on a fused workgroup's wait, in 100 MHz clock ticks
};


__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// K tiles travel HBM -> LDS with gfx950's direct-to-LDS 16-byte loads, so
// several tiles per wave are in flight without holding VGPRs.  Each wave owns
// a ring of kStages tile buffers.  A tile is 32 keys x CR 16-byte chunks
// (CR = D/8).  Load instruction j writes 64 x 16 bytes in lane order, i.e.
// rows 64/CR * j ... of the tile, and its lanes read one contiguous 1 KiB run
// of K, so each instruction touches only a few cache lines.  Inside a row the
// chunks are XOR-swizzled: LDS position p of key row t holds chunk p ^ (t % CR),
// which keeps the later fragment reads (32 rows, same chunk) spread over the
// LDS banks.
template <int D>
constexpr int tile_bytes() { return 32 * D * 2; }

typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* stage, const uint16_t* kbase, int64_t kts,
                                           int t0, int L, int lane) {
  constexpr int CR = D / 8;          // 16-byte chunks per key row
  constexpr int RPI = 64 / CR;       // key rows per load instruction
  const int p = lane % CR;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const int tr = j * RPI + lane / CR;          // row inside the tile
    int t = t0 + tr;
    t = t < L ? t : L - 1;                       // clamp the ragged tail; masked later
    const int c = p ^ (tr % CR);                 // global chunk stored at position p
    __builtin_amdgcn_global_load_lds(kbase + (int64_t)t * kts + 8 * c,
                                     (lds_void*)(stage + j * 1024), 16, 0, 0);
  }
}

// Byte offsets, inside a tile, of the A-operand fragment lane `lane` needs at
// k-step s: key row t = lane % 32, chunk (lane / 32) * CR/2 + s, stored at
// position chunk ^ (t % CR).
template <int D>
__device__ __forceinline__ void frag_offsets(uint32_t (&off)[D / 16], int lane) {
  constexpr int CR = D / 8;
  const int t = lane & 31;
  const int base = ((lane >> 5) * (CR / 2)) ^ (t % CR);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) off[s] = (uint32_t)((t * CR + (base ^ s)) * 16);
}

// Waits until at most N vector-memory operations of this wave are outstanding
// (vmcnt decrements in issue order), with a compiler memory barrier so no LDS
// read is hoisted above it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS accesses inside the tile loops are issued through inline asm: the
// compiler would otherwise guard every LDS read with a full vmcnt(0) wait
// (it cannot tell the ring stage being read from the ones still being
// filled), draining the load queue.  Each asm wait lists the registers it
// guards as operands, so no consumer is scheduled above it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int OFF>
__device__ __forceinline__ void ds_read_b128(u32x4& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
}

template <int N>
__device__ __forceinline__ void wait_lgkm(u32x4 (&v)[N]) {
  if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                   "+v"(v[6]), "+v"(v[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

template <int KS>
__device__ __forceinline__ void read_frags(u32x4 (&f)[KS], uint32_t base, const uint32_t (&off)[KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s) ds_read_b128<0>(f[s], base + off[s]);
}

// The same reads with AGPR destinations: the pipelined loops keep the K
// fragments, which only ever feed MFMAs, in the AGPR file next to Q.
template <int OFF>
__device__ __forceinline__ void ds_read_b128_a(u32x4& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=a"(v) : "v"(addr), "n"(OFF));
}

template <int KS>
__device__ __forceinline__ void read_frags_a(u32x4 (&f)[KS], uint32_t base,
                                             const uint32_t (&off)[KS]) {
#pragma unroll
  for (int s = 0; s < KS; ++s) ds_read_b128_a<0>(f[s], base + off[s]);
}

template <int N>
__device__ __forceinline__ void wait_lgkm_a(u32x4 (&v)[N]) {
  if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+a"(v[0]), "+a"(v[1]), "+a"(v[2]), "+a"(v[3]), "+a"(v[4]), "+a"(v[5]),
                   "+a"(v[6]), "+a"(v[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+a"(v[0]), "+a"(v[1]), "+a"(v[2]), "+a"(v[3]));
}

// Last visible key of the padded query rows a lane holds (N-tile T, lane l ->
// padded row 32T + l%32), -1 for padding rows.
template <int NT>
__device__ __forceinline__ void q_vis(int (&vis)[NT], const KArgs& a, int lane) {
  const int nl = lane & 31;
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int r = a.row0 + 32 * T + nl;
    const int hq = r / a.head_rows, j = r % a.head_rows;
    const int64_t pos = a.p.q_pos0 + j;
    vis[T] = hq < a.p.G && j < a.p.W ? (int)(pos < (int64_t)a.p.L - 1 ? pos : (int64_t)a.p.L - 1)
                                     : -1;
  }
}

// Padded query row row0 + r of group g.  Padding rows read row 0 of the group
// instead: their statistics are discarded and their row constant is +inf, so
// their logits never reach an output.
__device__ __forceinline__ const uint16_t* q_row(const KArgs& a, int g, int r) {
  r += a.row0;
  const int hq = r / a.head_rows, j = r % a.head_rows;
  const bool valid = hq < a.p.G && j < a.p.W;
  return a.p.Q + (int64_t)(g * a.p.G + (valid ? hq : 0)) * a.p.qhs +
         (int64_t)(valid ? j : 0) * a.p.qrs;
}

// Padded query rows 32w .. 32w+31 into an LDS stage with the K-tile layout
// (same chunk swizzle), so the fragment offsets of a K tile address them too.
// Loading a lane's fragments straight from global memory would touch a
// different cache line in every lane of every load; staged, each load
// instruction reads whole rows.
template <int D>
__device__ __forceinline__ void issue_q_rows(uint8_t* stage, const KArgs& a, int g, int w,
                                             int lane) {
  constexpr int CR = D / 8;
  constexpr int RPI = 64 / CR;
  const int p = lane % CR;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const int tr = j * RPI + lane / CR;
    const int c = p ^ (tr % CR);
    __builtin_amdgcn_global_load_lds(q_row(a, g, 32 * w + tr) + 8 * c,
                                     (lds_void*)(stage + j * 1024), 16, 0, 0);
  }
}

// Every wave's AGPR copy of all query fragments, from the rows staged by
// issue_q_rows: N-tile T sits at base + T * stride.  Returns once the reads
// have landed.
template <int D, int NT>
__device__ __forceinline__ void read_q_agpr(bf16x8 (&q)[NT][D / 16], uint32_t base,
                                            uint32_t stride, const uint32_t (&off)[D / 16]) {
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      asm volatile("ds_read_b128 %0, %1" : "=a"(q[T][s]) : "v"(base + T * stride + off[s]));
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    if constexpr (D / 16 == 8)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+a"(q[T][0]), "+a"(q[T][1]), "+a"(q[T][2]), "+a"(q[T][3]), "+a"(q[T][4]),
                     "+a"(q[T][5]), "+a"(q[T][6]), "+a"(q[T][7]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)" : "+a"(q[T][0]), "+a"(q[T][1]), "+a"(q[T][2]), "+a"(q[T][3]));
  }
}

// Key index of accumulator element i for lane half hl (32x32 MFMA output layout).
__device__ __forceinline__ int key_of(int i, int hl) { return 8 * (i >> 2) + 4 * hl + (i & 3); }


// The tile MFMAs are compiler builtins.  The query fragments (B operand) are
// read into AGPRs and stay there, leaving the VGPRs to the accumulators and
// the softmax work; the K fragments land in AGPRs too, and the compiler takes
// either operand from whichever file holds it.  Where its register copies
// (v_accvgpr_read/write) write an operand just before an MFMA, the compiler
// places the wait states itself, so only those MFMAs wait (an inline-asm MFMA
// would need an unconditional wait before it: the compiler checks no hazards
// into inline asm).
__device__ __forceinline__ void mfma_acc(f32x16& acc, const u32x4& kf, const bf16x8& qa) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qa, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_zero(f32x16& acc, const u32x4& kf, const bf16x8& qa) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qa, f32x16{}, 0, 0,
                                               0);
}

template <int D, int NT, int LO, int N>
__device__ __forceinline__ void mfma_part(f32x16 (&acc)[N > 0 ? N : 1], const u32x4 (&f)[D / 16],
                                          const bf16x8 (&q)[NT][D / 16]) {
  if constexpr (N > 0) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int T = 0; T < N; ++T) {
        if (s == 0)
          mfma_zero(acc[T], f[s], q[LO + T][s]);
        else
          mfma_acc(acc[T], f[s], q[LO + T][s]);
      }
  }
}

template <int D, int NT>
__device__ __forceinline__ void mfma_all_a(f32x16 (&acc)[NT], const u32x4 (&f)[D / 16],
                                           const bf16x8 (&q)[NT][D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      if (s == 0)
        mfma_zero(acc[T], f[s], q[T][s]);
      else
        mfma_acc(acc[T], f[s], q[T][s]);
    }
}

// Online (max, sum of exp2) update of query rows LO .. LO+N-1 for one tile.
// The running max m only stabilises the exponentials, so it may lag the true
// max: terms are summed against the current m, and m is refreshed (the whole
// half recomputed against its exact max) only when some lane's sum leaves
// [0, 2^64]; the first tile (m = -inf) always takes that path.  The branch is
// wave-uniform.
template <int NT, int LO, int N>
__device__ __forceinline__ void stats_part(const f32x16 (&acc)[N > 0 ? N : 1], float (&m)[NT],
                                           float (&z)[NT], float c, bool full, int t0, int hl,
                                           const int (&vis)[NT]) {
  if constexpr (N > 0) {
    if (full) {
      float sum[N];
      bool bad = false;
#pragma unroll
      for (int T = 0; T < N; ++T) {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          sa += ex2(fmaf(acc[T][i], c, -m[LO + T]));
          sb += ex2(fmaf(acc[T][i + 1], c, -m[LO + T]));
        }
        sum[T] = sa + sb;
        bad |= !(sum[T] <= 0x1p64f);
      }
      if (!__any(bad)) {
#pragma unroll
        for (int T = 0; T < N; ++T) z[LO + T] += sum[T];
        return;
      }
#pragma unroll
      for (int T = 0; T < N; ++T) {
        float mx = acc[T][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[T][i]);
        const float mn = fmaxf(m[LO + T], mx * c);
        float s2 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s2 += ex2(fmaf(acc[T][i], c, -mn));
        z[LO + T] = z[LO + T] * ex2(m[LO + T] - mn) + s2;
        m[LO + T] = mn;
      }
    } else {
#pragma unroll
      for (int T = 0; T < N; ++T) {
        float v[16];
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = (t0 + key_of(i, hl) <= vis[LO + T]) ? acc[T][i] : kNegInf;
          mx = fmaxf(mx, v[i]);
        }
        const float mn = fmaxf(m[LO + T], mx * c);
        if (mn != kNegInf) {
          float s2 = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) s2 += ex2(fmaf(v[i], c, -mn));
          z[LO + T] = z[LO + T] * ex2(m[LO + T] - mn) + s2;
          m[LO + T] = mn;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ pass 1
// One 16-byte-per-lane load instruction (1 KiB) of a tile: chunk jj of the KS
// that issue_tile issues together.
template <int D>
__device__ __forceinline__ void issue_chunk(uint8_t* stage, const uint16_t* kbase, int64_t kts,
                                            int t0, int L, int lane, int jj) {
  constexpr int CR = D / 8;
  constexpr int RPI = 64 / CR;
  const int p = lane % CR;
  const int tr = jj * RPI + lane / CR;
  int t = t0 + tr;
  t = t < L ? t : L - 1;
  const int c = p ^ (tr % CR);
  __builtin_amdgcn_global_load_lds(kbase + (int64_t)t * kts + 8 * c,
                                   (lds_void*)(stage + jj * 1024), 16, 0, 0);
}

// The same load for full tiles (no ragged end), addressed as a uniform tile
// base plus a per-lane byte offset: key row tr = jj * RPI + lane / CR of the
// tile, chunk p ^ (tr % CR).  (jj * RPI) % CR repeats every CR / RPI chunks,
// so a lane needs NQ = CR / RPI distinct offsets (chunk_offsets), and the
// load takes an SGPR base and a VGPR offset: no vector ALU work per load.
template <int D>
struct ChunkGeom {
  static constexpr int CR = D / 8;
  static constexpr int RPI = 64 / CR;
  static constexpr int NQ = CR / RPI;
};

template <int D>
__device__ __forceinline__ void chunk_offsets(uint32_t (&off)[ChunkGeom<D>::NQ], int lane,
                                              int64_t kts) {
  using G = ChunkGeom<D>;
  const int p = lane % G::CR, lq = lane / G::CR;
  const uint32_t row = (uint32_t)((int64_t)lq * kts * 2);
#pragma unroll
  for (int q2 = 0; q2 < G::NQ; ++q2)
    off[q2] = row + 16u * (uint32_t)(p ^ ((q2 * G::RPI + lq) % G::CR));
}

template <int D>
__device__ __forceinline__ void issue_chunk_full(uint8_t* stage, const uint8_t* tile_base,
                                                 int64_t kts,
                                                 const uint32_t (&off)[ChunkGeom<D>::NQ], int jj) {
  using G = ChunkGeom<D>;
  const uint8_t* src = tile_base + (int64_t)jj * G::RPI * kts * 2 + off[jj % G::NQ];
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + jj * 1024), 16, 0, 0);
}

// Slot schedule of a steady-state step with M MFMA slots and KS load/read
// instructions per tile: the loads of a new tile go out together in the
// first slot, the wait for the next tile and all its fragment reads in the
// middle one.  A direct-to-LDS load holds up the wave's instruction issue for
// tens of cycles; issued back to back they cost less of the VALU work that
// shares the wave than spread over the slots (5-7% fewer cycles per tile).
template <int M, int KS>
struct StepSlots {
  static constexpr int kWait = M / 2;
  static constexpr int issue(int) { return 0; }
  static constexpr int read(int) { return M / 2; }
};

// One step of the full-tile pipeline: the KS*NT MFMAs of the current tile
// (fragments fc) into accC, k-major so consecutive MFMAs use different
// accumulators, interleaved EPM logits per MFMA with WORK(T, i, x) on the
// previous tile's logits accP (x = accP[T][i]; the compiler places the wait
// states between the MFMA that wrote it and this read).  ISSUE: the loads of
// the tile at `issue_base` into `issue_stage` go out in the first slot.  NEXT: the next tile is waited for (WAITN
// loads may stay outstanding) and its fragments are read into fn.
template <int D, int NT, bool ISSUE, bool NEXT, int WAITN, typename Work, typename Side>
__device__ __forceinline__ void pipe_step(f32x16 (&accC)[NT], f32x16 (&accP)[NT],
                                          const u32x4 (&fc)[D / 16], u32x4 (&fn)[D / 16],
                                          const bf16x8 (&q)[NT][D / 16], uint8_t* issue_stage,
                                          const uint8_t* issue_base, int64_t kts,
                                          const uint32_t (&coff)[ChunkGeom<D>::NQ],
                                          uint32_t next_stage, const uint32_t (&foff)[D / 16],
                                          Work&& work, Side&& side) {
  constexpr int KS = D / 16;
  constexpr int M = KS * NT;
  constexpr int EPM = 16 / KS;
  using SL = StepSlots<M, KS>;
#pragma unroll
  for (int k = 0; k < M; ++k) {
    const int s = k / NT, T = k % NT;
    if (s == 0)
      mfma_zero(accC[T], fc[s], q[T][s]);
    else
      mfma_acc(accC[T], fc[s], q[T][s]);
#pragma unroll
    for (int u = 0; u < EPM; ++u) {
      const int e = k * EPM + u;
      work(e / 16, e % 16, accP[e / 16][e % 16]);
    }
    side(k, M);
    if constexpr (ISSUE) {
#pragma unroll
      for (int jj = 0; jj < KS; ++jj)
        if (SL::issue(jj) == k) issue_chunk_full<D>(issue_stage, issue_base, kts, coff, jj);
    }
    if constexpr (NEXT) {
      if (k == SL::kWait) wait_vm<WAITN>();
#pragma unroll
      for (int jj = 0; jj < KS; ++jj)
        if (SL::read(jj) == k) ds_read_b128_a<0>(fn[jj], next_stage + foff[jj]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (NEXT) wait_lgkm_a<KS>(fn);
}

// Swapped-operand tile: A = query fragments, B = K fragments, then a ninth
// k-step A = the rows' -b/c parts, B = ones.  acc[T] = (x - b/c) for rows
// 32T + 8(i/4) + 4hl + i%4 against key lane % 32.
__device__ __forceinline__ void mfma_rows(f32x16& acc, const bf16x8& qa, const u32x4& kf, bool zero) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, __builtin_bit_cast(bf16x8, kf),
                                               zero ? f32x16{} : acc, 0, 0, 0);
}

template <int D, int NT>
__device__ __forceinline__ void mfma_rows_all(f32x16 (&acc)[NT], const u32x4 (&f)[D / 16],
                                              const bf16x8 (&q)[NT][D / 16],
                                              const bf16x8 (&qx)[NT], const bf16x8& ones) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int T = 0; T < NT; ++T) mfma_rows(acc[T], q[T][s], f[s], s == 0);
#pragma unroll
  for (int T = 0; T < NT; ++T)
    acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qx[T], ones, acc[T], 0, 0, 0);
}

// pipe_step for the swapped-operand tile: (KS + 1) * NT MFMA slots, the
// 16 * NT elements of the previous tile spread over them.
template <int D, int NT, bool ISSUE, bool NEXT, int WAITN, typename Work>
__device__ __forceinline__ void pipe_step_rows(f32x16 (&accC)[NT], f32x16 (&accP)[NT],
                                               const u32x4 (&fc)[D / 16], u32x4 (&fn)[D / 16],
                                               const bf16x8 (&q)[NT][D / 16],
                                               const bf16x8 (&qx)[NT], const bf16x8& ones,
                                               uint8_t* issue_stage, const uint8_t* issue_base,
                                               int64_t kts,
                                               const uint32_t (&coff)[ChunkGeom<D>::NQ],
                                               uint32_t next_stage,
                                               const uint32_t (&foff)[D / 16], Work&& work) {
  constexpr int KS = D / 16;
  constexpr int M = (KS + 1) * NT;
  constexpr int E = 16 * NT;
  using SL = StepSlots<M, KS>;
#pragma unroll
  for (int k = 0; k < M; ++k) {
    if (k < KS * NT) {
      const int s = k / NT, T = k % NT;
      mfma_rows(accC[T], q[T][s], fc[s], s == 0);
    } else {
      const int T = k - KS * NT;
      accC[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qx[T], ones, accC[T], 0, 0, 0);
    }
#pragma unroll
    for (int e = (k * E) / M; e < ((k + 1) * E) / M; ++e) work(e / 16, e % 16, accP[e / 16][e % 16]);
    if constexpr (ISSUE) {
#pragma unroll
      for (int jj = 0; jj < KS; ++jj)
        if (SL::issue(jj) == k) issue_chunk_full<D>(issue_stage, issue_base, kts, coff, jj);
    }
    if constexpr (NEXT) {
      if (k == SL::kWait) wait_vm<WAITN>();
#pragma unroll
      for (int jj = 0; jj < KS; ++jj)
        if (SL::read(jj) == k) ds_read_b128_a<0>(fn[jj], next_stage + foff[jj]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (NEXT) wait_lgkm_a<KS>(fn);
}

// Pass 1: per (row, split) online (max, sum of exp2) of the logits.
// Full tiles (no causal masking) run a software pipeline: while the matrix
// cores compute tile j's logits, the VALU sums tile j-1's exponentials
// against a running max m that was set exactly from the wave's first tile
// and never changes in the pipeline, so the sums need no branch.  A lane
// whose row sum exceeds 2^100 (or is not finite) after the last full tile
// sets a flag; a wave with a flagged lane recomputes its full tiles with the
// exact online update.  The few masked
// tiles (causal window, ragged end) use the exact update directly.
// ATOMIC: the split statistics are stored with device-scope atomic stores,
// which reach the device's point of coherence, for a later reader in the
// same launch on another XCD (the fused launch); plain stores otherwise.
// Returns (per wave) whether the wave's ring still holds its last full tiles,
// tile j in stage j % kStages: true unless it had masked tiles or redid its
// full tiles, both of which pass through stage 0.
template <int D, int NT, bool ATOMIC>
__device__ __forceinline__ bool stats_body(const KArgs& a, int split,
                                           uint8_t (&ring)[kWaves][kStages][tile_bytes<D>()],
                                           float2 (&sm)[kWaves][32 * NT],
                                           bf16x8 (&q)[NT][D / 16]) {
  constexpr int KS = D / 16;
  constexpr int S = kStages;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 31, hl = lane >> 5;
  const int g = a.g0 + blockIdx.y;
  const int tb = split * a.tps;
  const int te = min(tb + a.tps, a.n_tiles);
  const float c = a.p.c;
  const int L = a.p.L;

  int vis[NT];
  q_vis<NT>(vis, a, lane);
  float m[NT], z[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    m[T] = kNegInf;
    z[T] = 0.f;
  }
  const uint16_t* kbase = a.p.K + (int64_t)g * a.p.khs;
  const int64_t kts = a.p.kts;
  uint32_t foff[KS];
  frag_offsets<D>(foff, lane);
  const uint32_t ring0 = lds_addr(ring[wave][0]);
  // this wave's tiles: tb + wave + j * kWaves; the first nf need no masking
  const int nt = te > tb + wave ? (te - tb - wave + kWaves - 1) / kWaves : 0;
  const int full_end = (a.min_vis - 31) >= 0 ? (a.min_vis - 31) / 32 + 1 : 0;  // tiles < full_end are full
  int nf = full_end > tb + wave ? (full_end - tb - wave + kWaves - 1) / kWaves : 0;
  nf = nf < nt ? nf : nt;
  bool kept = nf > 0 && nf == nt;
  const auto tile_t0 = [&](int j) { return (tb + wave + j * kWaves) * 32; };
  const auto stage_of = [&](int j) { return ring[wave][j & (S - 1)]; };
  const auto tile_base = [&](int j) {
    return reinterpret_cast<const uint8_t*>(kbase) + (int64_t)tile_t0(j) * kts * 2;
  };
  uint32_t coff[ChunkGeom<D>::NQ];
  chunk_offsets<D>(coff, lane, kts);

  // Tiles 0 .. S-1 fill the ring; step j then refills tile j-1's stage.  The
  // query rows travel first, through every wave's last stage, while tiles
  // 0 .. S-2 are queued behind them (vector memory operations complete in
  // issue order); tile S-1 follows once every wave has its copy of Q.  The
  // barriers are bare: a fenced one would wait for the queued tiles too.
  const int pre = nf < S ? nf : S;
  if (wave < NT) issue_q_rows<D>(ring[wave][S - 1], a, g, wave, lane);
  for (int j = 0; j < pre && j < S - 1; ++j)
    issue_tile<D>(stage_of(j), kbase, kts, tile_t0(j), L, lane);
  if (pre >= S - 1)
    wait_vm<(S - 1) * KS>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  read_q_agpr<D, NT>(q, lds_addr(ring[0][S - 1]), S * tile_bytes<D>(), foff);
  __builtin_amdgcn_s_barrier();
  if (pre == S) issue_tile<D>(stage_of(S - 1), kbase, kts, tile_t0(S - 1), L, lane);

  if (nf > 0) {
    f32x16 acc0[NT], acc1[NT];
    u32x4 f0[KS], f1[KS];
    if (pre == S)
      wait_vm<(S - 1) * KS>();
    else
      wait_vm<0>();
    read_frags_a<KS>(f0, ring0, foff);
    wait_lgkm_a<KS>(f0);
    mfma_all_a<D, NT>(acc0, f0, q);
    if (nf > 1) {
      if (pre == S)
        wait_vm<(S - 2) * KS>();
      else
        wait_vm<0>();
      read_frags_a<KS>(f1, ring0 + tile_bytes<D>(), foff);
      wait_lgkm_a<KS>(f1);
    }
    // the running max: exact max of the wave's first tile, per lane and row
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      float mx = acc0[T][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc0[T][i]);
      m[T] = mx * c;
    }
    float sa[NT], sb[NT], nm[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) nm[T] = -m[T];
#pragma unroll
    for (int T = 0; T < NT; ++T) sa[T] = sb[T] = 0.f;
    const auto no_side = [](int, int) {};
    // step j: MFMAs of tile j (fc) || sums of tile j-1 (accP); loads of tile
    // j + S - 1 while it exists; then tile j + 1's fragments into fn.
    const auto step = [&](f32x16(&accC)[NT], f32x16(&accP)[NT], const u32x4(&fc)[KS],
                          u32x4(&fn)[KS], int j) {
      const auto work = [&](int T, int i, float x) {
        if (i & 1)
          sb[T] += ex2(fmaf(x, c, nm[T]));
        else
          sa[T] += ex2(fmaf(x, c, nm[T]));
      };
      const uint32_t nxt = ring0 + ((j + 1) & (S - 1)) * tile_bytes<D>();
      if (j + S - 1 < nf)
        pipe_step<D, NT, true, true, (S - 2) * KS>(accC, accP, fc, fn, q, stage_of(j + S - 1),
                                                    tile_base(j + S - 1), kts, coff, nxt, foff,
                                                    work, no_side);
      else if (j + 1 < nf)
        pipe_step<D, NT, false, true, 0>(accC, accP, fc, fn, q, nullptr, nullptr, kts, coff, nxt,
                                         foff, work, no_side);
      else
        pipe_step<D, NT, false, false, 0>(accC, accP, fc, fn, q, nullptr, nullptr, kts, coff,
                                          nxt, foff, work, no_side);
    };
    int j = 1;
    for (; j + 1 < nf; j += 2) {
      step(acc1, acc0, f1, f0, j);
      step(acc0, acc1, f0, f1, j + 1);
    }
    if (j < nf) step(acc1, acc0, f1, f0, j);
    // the last full tile's sums
    const auto tail = [&](f32x16(&accP)[NT]) {
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i & 1)
            sb[T] += ex2(fmaf(accP[T][i], c, -m[T]));
          else
            sa[T] += ex2(fmaf(accP[T][i], c, -m[T]));
        }
    };
    if ((nf - 1) & 1)
      tail(acc1);
    else
      tail(acc0);
    // The sums run over every full tile against the first tile's max.  A sum
    // keeps its full relative precision however far the row's max rose above
    // that reference; it only has to stay far enough inside the float range
    // for the merges of lane halves, waves and splits (at most 2^27 partial
    // sums of at most 2^100 each), and a term or sum past the range shows as
    // inf or NaN, which fails the same test.
    bool flag = false;
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      z[T] = sa[T] + sb[T];
      flag |= !(z[T] <= 0x1p100f);
    }
    if (__any(flag)) {
      // some logit rose about 100 log2 units above the first tile's max:
      // redo the full tiles with the exact online update
      kept = false;
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        m[T] = kNegInf;
        z[T] = 0.f;
      }
      for (int jj = 0; jj < nf; ++jj) {
        issue_tile<D>(stage_of(0), kbase, kts, tile_t0(jj), L, lane);
        wait_vm<0>();
        read_frags_a<KS>(f0, ring0, foff);
        wait_lgkm_a<KS>(f0);
        mfma_all_a<D, NT>(acc0, f0, q);
        stats_part<NT, 0, NT>(acc0, m, z, c, true, 0, hl, vis);
      }
    }
  }
  // masked tiles: exact online update with the causal / ragged-end mask
  for (int j = nf; j < nt; ++j) {
    f32x16 acc[NT];
    u32x4 f[KS];
    issue_tile<D>(stage_of(0), kbase, kts, tile_t0(j), L, lane);
    wait_vm<0>();
    read_frags<KS>(f, ring0, foff);
    wait_lgkm<KS>(f);
    mfma_part<D, NT, 0, NT>(acc, f, q);
    stats_part<NT, 0, NT>(acc, m, z, c, false, tile_t0(j), hl, vis);
  }

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
    float2* dst = a.p.stats + ((int64_t)g * a.rows_pad + a.row0 + r) * a.n_split + split;
    if constexpr (ATOMIC)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(dst),
                         __builtin_bit_cast(uint64_t, make_float2(mm, zz)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      *dst = make_float2(mm, zz);
  }
  return kept;
}

template <int D, int NT>
__global__ __launch_bounds__(kThreads, 1) void score_stats_kernel(KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kStages][tile_bytes<D>()];
  __shared__ float2 sm[kWaves][32 * NT];
  bf16x8 q[NT][D / 16];
  stats_body<D, NT, false>(a, blockIdx.x, ring, sm, q);
}

// ------------------------------------------------------------------ merge
// Folds the per-split (max, sum) pairs of each of the group's rows by
// log-sum-exp into the row constant b = m + log2 Z (+inf for padding rows),
// inside the pass-2 workgroup: two threads per row, each folding every other
// split online in a fixed order, then combined.  The pairs are loaded in
// batches of kMergeBatch independent loads, so a row costs one memory round
// trip per batch rather than one per split.  Leaves b for rows [0, rows_pad)
// in brow.
constexpr int kMergeBatch = 16;

__device__ __forceinline__ void fold_pair(float& mm, float& zz, float2 v) {
  if (v.x > mm) {
    zz = (mm == kNegInf ? 0.f : zz * exp2f(mm - v.x)) + v.y;
    mm = v.x;
  } else if (v.x != kNegInf) {
    zz += v.y * exp2f(v.x - mm);
  }
}

// ATOMIC: the pairs were written earlier in the same launch (by workgroups
// on other XCDs) and are read with device-scope atomic loads.
template <bool ATOMIC>
__device__ __forceinline__ void merge_rows(const KArgs& a, int g, int rows, float* brow) {
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  if (r < rows) {
    const float2* st = a.p.stats + ((int64_t)g * a.rows_pad + a.row0 + r) * a.n_split;
    float mm = kNegInf, zz = 0.f;
    for (int s0 = half; s0 < a.n_split; s0 += 2 * kMergeBatch) {
      float2 v[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int s = s0 + 2 * i;
        if constexpr (ATOMIC)
          v[i] = s < a.n_split
                     ? __builtin_bit_cast(float2, __hip_atomic_load(
                                                      reinterpret_cast<const uint64_t*>(st + s),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                     : make_float2(kNegInf, 0.f);
        else
          v[i] = s < a.n_split ? st[s] : make_float2(kNegInf, 0.f);
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) fold_pair(mm, zz, v[i]);
    }
    const float m2 = __shfl_xor(mm, 1), z2 = __shfl_xor(zz, 1);
    const float mx = fmaxf(mm, m2);
    const float zt = mx == kNegInf ? 0.f
                                   : (mm == kNegInf ? 0.f : zz * exp2f(mm - mx)) +
                                         (m2 == kNegInf ? 0.f : z2 * exp2f(m2 - mx));
    if (half == 0) {
      const int hq = (a.row0 + r) / a.head_rows, jr = (a.row0 + r) % a.head_rows;
      const bool valid = hq < a.p.G && jr < a.p.W && mx != kNegInf;
      brow[r] = valid ? mx + log2f(zt) : kPosInf;
    }
  }
  wait_vm<0>();   // also every load the caller queued before the merge
  __syncthreads();
}

// ------------------------------------------------------------------ pass 2
__device__ __forceinline__ void store_out(float* o, float v, int accumulate) {
  *o = accumulate ? *o + v : v;
}

// MODE 0: sum over every row of the group (GROUP_SUM, ALL_SUM's group rows,
// and a query head whose rows span both row groups).
// MODE 1: per query head sums (NONE) or their maximum (GROUP_MAX).
// Both run the same swapped-operand pipeline; only the per-tile finish differs.
// FUSED: the query fragments are already in q (the statistics pass of the
// same launch loaded them), and the statistics come from that pass: settle()
// returns once all of the head's splits are published, true if it had to use
// the ring to compute some of them itself.  kept: the statistics pass left
// this wave's last full tiles in the ring (tile j in stage j % kStages), and
// this pass, walking the full tiles last to first, starts on them without
// loading them again.
template <int D, int NT, int MODE, bool FUSED, class Settle>
__device__ __forceinline__ void colsum_body(const KArgs& a,
                                            uint8_t (&ring)[kWaves][kStages][tile_bytes<D>()],
                                            int (&rvis)[128], float (&brow)[128],
                                            bf16x8 (&q)[NT][D / 16], bool kept,
                                            Settle&& settle) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 31, hl = lane >> 5;
  const int g = a.g0 + blockIdx.y;
  const int split = blockIdx.x;
  const int tb = split * a.tps;
  const int te = min(tb + a.tps, a.n_tiles);
  const float c = a.p.c;
  const int L = a.p.L;

  constexpr int S = kStages;
  const uint16_t* kbase = a.p.K + (int64_t)g * a.p.khs;
  const int64_t kts = a.p.kts;
  const int nt = te > tb + wave ? (te - tb - wave + kWaves - 1) / kWaves : 0;
  // tiles j = 0 .. nt-1 of this wave are tb + wave + j * kWaves; the first nf
  // need no masking
  const int full_end = (a.min_vis - 31) >= 0 ? (a.min_vis - 31) / 32 + 1 : 0;
  int nf = full_end > tb + wave ? (full_end - tb - wave + kWaves - 1) / kWaves : 0;
  nf = nf < nt ? nf : nt;
  // Pass 2 may walk the full tiles in the reverse of pass 1's order, so that
  // the keys pass 1 streamed last, the likeliest to still sit in the
  // memory-side cache, are read first.  x-th processed full tile:
  const auto tj = [&](int x) { return a.rev ? nf - 1 - x : x; };
  const auto t0_of = [&](int x) { return (tb + wave + tj(x) * kWaves) * 32; };
  kept = FUSED && kept && a.rev;

  // The query rows (through every wave's last ring stage, see the pass-1
  // kernel) and the first full tile load while the row constants are merged;
  // the merge's barrier waits for all three.
  if (!FUSED && wave < NT) issue_q_rows<D>(ring[wave][S - 1], a, g, wave, lane);
  if (nf > 0 && !kept) issue_tile<D>(ring[wave][0], kbase, kts, t0_of(0), L, lane);
  // last visible key of every padded row (-1 for padding rows), for the
  // masked tiles
  if (threadIdx.x < 32 * NT) {
    const int r = a.row0 + threadIdx.x;
    const int hq = r / a.head_rows, jr = r % a.head_rows;
    const int64_t pos = a.p.q_pos0 + jr;
    rvis[threadIdx.x] = hq < a.p.G && jr < a.p.W
                            ? (int)(pos < (int64_t)a.p.L - 1 ? pos : (int64_t)a.p.L - 1)
                            : -1;
  }
  // row constants from pass 1's split statistics (the merge's barrier also
  // orders rvis); in a fused launch, once every split of the head is in
  if constexpr (FUSED) {
    if (settle()) {
      kept = false;
      if (nf > 0) issue_tile<D>(ring[wave][0], kbase, kts, t0_of(0), L, lane);
    }
  }
  merge_rows<FUSED>(a, g, 32 * NT, brow);
  float b[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) b[T] = brow[32 * T + nl];
  __builtin_amdgcn_s_waitcnt(0);   // Q, the first tile and the row constants are in

  uint32_t foff[D / 16];
  frag_offsets<D>(foff, lane);
  if constexpr (!FUSED) {
    read_q_agpr<D, NT>(q, lds_addr(ring[0][S - 1]), S * tile_bytes<D>(), foff);
    __builtin_amdgcn_s_barrier();   // every wave has its copy before the stage is refilled
  }
  {
    // Column sums with the MFMA operands swapped: A = the query rows, B = the
    // K fragments, so lane l holds key l % 32 of the tile against 16 rows of
    // each row tile, and a key's sum over rows is a sum inside the lane plus
    // one exchange between the lane halves.  Each row's constant b enters the
    // MFMA as a ninth k-step: the rows carry -b/c split into three bf16 parts
    // (about 24 bits), the keys carry ones, so the accumulators hold x - b/c
    // and p = exp2(c * acc).
    constexpr int KS = D / 16;
    const uint32_t ring0 = lds_addr(ring[wave][0]);
    bf16x8 qx[NT];
    bf16x8 ones{};
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      qx[T] = bf16x8{};
      if (hl == 0) {
        const float v = -b[T] / c;
        if (v == kNegInf || v == kPosInf) {
          qx[T][0] = (__bf16)v;
        } else {
          const __bf16 h1 = (__bf16)v;
          const float r1 = v - (float)h1;
          const __bf16 h2 = (__bf16)r1;
          const __bf16 h3 = (__bf16)(r1 - (float)h2);
          qx[T][0] = h1;
          qx[T][1] = h2;
          qx[T][2] = h3;
        }
      }
    }
    if (hl == 0) {
      ones[0] = (__bf16)1.f;
      ones[1] = (__bf16)1.f;
      ones[2] = (__bf16)1.f;
    }
    // A tile's partial sums per lane: MODE 0 two per row tile (every row of
    // the group is summed); MODE 1 one per block of 4 rows (rows 8q + 4hl ..
    // 8q + 4hl + 3 of a row tile), the unit a head is made of.
    constexpr int NPC = MODE == 0 ? 2 * NT : 4 * NT;
    const auto pc_of = [](int T, int i) { return MODE == 0 ? 2 * T + (i & 1) : 4 * T + (i >> 2); };
    // the partner lane's value (lane l xor 32)
    const auto other_half = [&](float v) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                       false, false);
      return __uint_as_float(hl ? sw[0] : sw[1]);
    };
    const auto finish = [&](float (&pc)[NPC], int t0) {
      const int tt = t0 + nl;
      if constexpr (MODE == 0) {
        float v = 0.f;
#pragma unroll
        for (int u = 0; u < NPC; ++u) v += pc[u];
        v += other_half(v);
        if (hl == 0 && tt < L) store_out(a.out + (int64_t)g * a.out_ld + tt, v, a.acc);
      } else {
        // Heads are runs of head_rows consecutive padded rows (4, 8, 16 or a
        // multiple of 32, inside one row group): with 4 a block is a whole
        // head of its lane half; otherwise the two halves' blocks q of a row
        // tile (rows 8q .. 8q+7) lie in one head, added across the halves,
        // and a head is the run of such blocks in (T, q) order.
        float mx = kNegInf;
        const auto put = [&](int hq, float v, bool lane_ok) {
          if (hq >= a.h0 && hq < a.h1) {
            if (a.per_head) {
              if (lane_ok && tt < L)
                store_out(a.out + (int64_t)(g * a.p.G + hq) * a.out_ld + tt, v, a.acc);
            } else {
              mx = fmaxf(mx, v);
            }
          }
        };
        if (a.head_rows == 4) {
#pragma unroll
          for (int T = 0; T < NT; ++T)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
              put((a.row0 + 32 * T + 8 * qb + 4 * hl) >> 2, pc[4 * T + qb], true);
          if (!a.per_head) mx = fmaxf(mx, other_half(mx));
        } else {
          // a head's blocks are added inside the lane first, then once
          // across the halves
          int cur_h = a.row0 / a.head_rows;
          float cur = 0.f;
#pragma unroll
          for (int T = 0; T < NT; ++T)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) {
              const int hq = (a.row0 + 32 * T + 8 * qb) / a.head_rows;
              if (hq != cur_h) {
                put(cur_h, cur + other_half(cur), hl == 0);
                cur_h = hq;
                cur = 0.f;
              }
              cur += pc[4 * T + qb];
            }
          put(cur_h, cur + other_half(cur), hl == 0);
        }
        if (!a.per_head && hl == 0 && tt < L)
          store_out(a.out + (int64_t)g * a.out_ld + tt, mx, a.acc);
      }
    };
    if (nf > 0) {
      // tile x's stage: x % S, or, on the tiles the statistics pass left,
      // (nf - 1 - x) % S; either way tile x + S reuses tile x's stage
      const int s0 = kept ? nf - 1 : 0, sd = kept ? -1 : 1;
      const auto sidx = [&](int x) { return (s0 + sd * x) & (S - 1); };
      const auto stage_of = [&](int x) { return ring[wave][sidx(x)]; };
      uint32_t coff[ChunkGeom<D>::NQ];
      chunk_offsets<D>(coff, lane, kts);
      f32x16 acc0[NT], acc1[NT];
      u32x4 f0[KS], f1[KS];
      const int pre = nf < S ? nf : S;
      // tile 0 was issued before the merge and has arrived (or was kept)
      if (!kept)
        for (int x = 1; x < pre; ++x) issue_tile<D>(stage_of(x), kbase, kts, t0_of(x), L, lane);
      if (pre == S)
        wait_vm<(S - 1) * KS>();
      else
        wait_vm<0>();
      read_frags_a<KS>(f0, ring0 + sidx(0) * tile_bytes<D>(), foff);
      wait_lgkm_a<KS>(f0);
      mfma_rows_all<D, NT>(acc0, f0, q, qx, ones);
      if (nf > 1) {
        if (pre == S)
          wait_vm<(S - 2) * KS>();
        else
          wait_vm<0>();
        read_frags_a<KS>(f1, ring0 + sidx(1) * tile_bytes<D>(), foff);
        wait_lgkm_a<KS>(f1);
      }
      // step x: MFMAs of tile x || probabilities of tile x-1, whose sums
      // are stored after the step
      const auto step = [&](f32x16(&accC)[NT], f32x16(&accP)[NT], const u32x4(&fc)[KS],
                            u32x4(&fn)[KS], int x) {
        float pc[NPC];
#pragma unroll
        for (int u = 0; u < NPC; ++u) pc[u] = 0.f;
        const auto work = [&](int T, int i, float v) { pc[pc_of(T, i)] += ex2(v * c); };
        const uint32_t nxt = ring0 + sidx(x + 1) * tile_bytes<D>();
        if (x + S - 1 < nf)
          pipe_step_rows<D, NT, true, true, (S - 2) * KS>(
              accC, accP, fc, fn, q, qx, ones, stage_of(x + S - 1),
              reinterpret_cast<const uint8_t*>(kbase) + (int64_t)t0_of(x + S - 1) * kts * 2, kts,
              coff, nxt, foff, work);
        else if (x + 1 < nf)
          pipe_step_rows<D, NT, false, true, 0>(accC, accP, fc, fn, q, qx, ones, nullptr, nullptr,
                                                kts, coff, nxt, foff, work);
        else
          pipe_step_rows<D, NT, false, false, 0>(accC, accP, fc, fn, q, qx, ones, nullptr,
                                                 nullptr, kts, coff, nxt, foff, work);
        finish(pc, t0_of(x - 1));
      };
      int x = 1;
      for (; x + 1 < nf; x += 2) {
        step(acc1, acc0, f1, f0, x);
        step(acc0, acc1, f0, f1, x + 1);
      }
      if (x < nf) step(acc1, acc0, f1, f0, x);
      // the last full tile's sums
      const auto tail = [&](f32x16(&accP)[NT]) {
        float pc[NPC];
#pragma unroll
        for (int u = 0; u < NPC; ++u) pc[u] = 0.f;
#pragma unroll
        for (int T = 0; T < NT; ++T)
#pragma unroll
          for (int i = 0; i < 16; ++i) pc[pc_of(T, i)] += ex2(accP[T][i] * c);
        finish(pc, t0_of(nf - 1));
      };
      if ((nf - 1) & 1)
        tail(acc1);
      else
        tail(acc0);
    }
    // masked tiles (causal window, ragged end): key nl of the tile against
    // each row's last visible key
    for (int j = nf; j < nt; ++j) {
      f32x16 acc[NT];
      u32x4 f[KS];
      const int t0 = (tb + wave + j * kWaves) * 32;
      issue_tile<D>(ring[wave][0], kbase, kts, t0, L, lane);
      wait_vm<0>();
      read_frags<KS>(f, ring0, foff);
      wait_lgkm<KS>(f);
      mfma_rows_all<D, NT>(acc, f, q, qx, ones);
      float pc[NPC];
#pragma unroll
      for (int u = 0; u < NPC; ++u) pc[u] = 0.f;
#pragma unroll
      for (int T = 0; T < NT; ++T) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int4 vv = *reinterpret_cast<const int4*>(&rvis[32 * T + 8 * i4 + 4 * hl]);
          const int vr[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
          for (int i1 = 0; i1 < 4; ++i1) {
            const int i = 4 * i4 + i1;
            const float e = ex2(acc[T][i] * c);
            pc[pc_of(T, i)] += (t0 + nl <= vr[i1]) ? e : 0.f;
          }
        }
      }
      finish(pc, t0);
    }
  }
}

template <int D, int NT, int MODE>
__global__ __launch_bounds__(kThreads, 1) void score_colsum_kernel(KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kStages][tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) int rvis[128];
  __shared__ float brow[128];
  bf16x8 q[NT][D / 16];
  colsum_body<D, NT, MODE, false>(a, ring, rvis, brow, q, false, [] { return false; });
}

// Both passes of one row group in one launch (see grid_sync.h).
template <int D, int NT, int MODE>
__global__ __launch_bounds__(kThreads, 1) void score_fused_kernel(KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kStages][tile_bytes<D>()];
  __shared__ float2 sm[kWaves][32 * NT];
  __shared__ __attribute__((aligned(16))) int rvis[128];
  __shared__ float brow[128];
  __shared__ int sh;
  bf16x8 q[NT][D / 16];
  uint64_t* flags = a.flag + (int64_t)(a.g0 + blockIdx.y) * a.n_split;
  const bool kept = stats_body<D, NT, true>(a, blockIdx.x, ring, sm, q);
  publish_flag(flags + blockIdx.x, a.epoch);
  const auto settle = [&]() -> bool {
    if (wait_flags(flags, a.epoch, a.n_split, a.wait_ticks, &sh)) return false;
    // some split is late: compute it here (its first tile's load lands first)
    wait_vm<0>();
    __syncthreads();
    for (int s = 0; s < a.n_split; ++s) {
      if (threadIdx.x == 0)
        sh = __hip_atomic_load(flags + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
      __syncthreads();
      const int done = __builtin_amdgcn_readfirstlane(sh);
      __syncthreads();
      if (!done) {
        stats_body<D, NT, true>(a, s, ring, sm, q);
        publish_flag(flags + s, a.epoch);
      }
    }
    return true;
  };
  colsum_body<D, NT, MODE, true>(a, ring, rvis, brow, q, kept, settle);
}

// ------------------------------------------------------------------ raw logits
// kvs_score_raw: R[j][t] = SUM or MAX over all query heads of scale * q.k, in
// one pass over K.  Each workgroup owns a run of key tiles for every KV head,
// so the reduction over heads, and over KV heads, happens in registers in a
// fixed order: no atomics, no second kernel, bit-reproducible.  The padded
// query rows of all KV heads sit in LDS for the whole kernel (staged once
// with coalesced loads, in the K-tile layout); each (key tile, KV head) step
// reads its K tile from the wave's 3-stage ring and the head's query
// fragments from LDS, the next step's fragments being read while this step's
// MFMAs run.
// The MFMA tile is 32 padded query rows (M) x 32 keys (N), so a lane holds one
// key and 16 rows: rows 8(i/4) + 4(l/32) + i%4 of each row tile.  Each head's
// W rows are padded to HR = 8, 16 or 32 rows, which puts the rows of every
// head that share a query index j in the same lane: the reduction over heads
// is in-lane, and each output row j is stored as 32 consecutive keys.
constexpr int kRawStages = 3;
template <int D>
constexpr int raw_q_tiles() { return D == 128 ? 8 : 28; }   // LDS left beside the ring

struct RawArgs {
  RawLaunch p;
  int n_tiles, tps;
};

// Padded query rows 32T .. 32T+31 of KV head g into an LDS tile (layout of
// issue_tile).  Padding rows read the group's first row; they are dropped
// before the reduction.
template <int D>
__device__ __forceinline__ void issue_raw_q(uint8_t* dst, const RawArgs& a, int g, int T, int lane) {
  constexpr int CR = D / 8;
  constexpr int RPI = 64 / CR;
  const int p = lane % CR;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const int tr = j * RPI + lane / CR;
    const int r = 32 * T + tr;
    const int hq = r / a.p.head_rows, jr = r % a.p.head_rows;
    const bool valid = hq < a.p.G && jr < a.p.W;
    const uint16_t* row = a.p.Q + (int64_t)(g * a.p.G + (valid ? hq : 0)) * a.p.qhs +
                          (int64_t)(valid ? jr : 0) * a.p.qrs;
    const int c = p ^ (tr % CR);
    __builtin_amdgcn_global_load_lds(row + 8 * c, (lds_void*)(dst + j * 1024), 16, 0, 0);
  }
}

template <bool MAX>
__device__ __forceinline__ float raw_combine(float x, float y) {
  return MAX ? fmaxf(x, y) : x + y;
}

template <int D, int HR, int NT, bool MAX>
__global__ __launch_bounds__(kThreads, 1) void score_raw_kernel(RawArgs a) {
  constexpr int KS = D / 16;
  constexpr int S = kRawStages;
  constexpr int TB = tile_bytes<D>();
  constexpr int NS = HR / 2;   // output rows j a lane holds
  __shared__ __attribute__((aligned(16))) uint8_t qs[raw_q_tiles<D>()][TB];
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][S][TB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 31, hl = lane >> 5;
  const int H = a.p.H_kv;
  const int tb = blockIdx.x * a.tps;
  const int te = min(tb + a.tps, a.n_tiles);
  const int nt = te > tb + wave ? (te - tb - wave + kWaves - 1) / kWaves : 0;
  const int steps = nt * H;   // (key tile, KV head) pairs, KV head fastest
  const auto kbase = [&](int s) { return a.p.K + (int64_t)(s % H) * a.p.khs; };
  const auto t0_of = [&](int s) { return (tb + wave + (s / H) * kWaves) * 32; };
  const auto issue_k = [&](int s) {
    issue_tile<D>(ring[wave][s % S], kbase(s), a.p.kts, t0_of(s), a.p.L, lane);
  };

  // query rows of every KV head, then the first K tiles behind them
  for (int u = wave; u < H * NT; u += kWaves) issue_raw_q<D>(qs[u], a, u / NT, u % NT, lane);
  const int pre = steps < S - 1 ? steps : S - 1;
  for (int s = 0; s < pre; ++s) issue_k(s);
  if (pre == 2)
    wait_vm<2 * KS>();
  else if (pre == 1)
    wait_vm<KS>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();   // bare: a fenced barrier would wait for the K tiles too

  uint32_t foff[KS];
  frag_offsets<D>(foff, lane);
  const uint32_t q0 = lds_addr(qs[0]);
  const auto read_k = [&](int s, u32x4(&f)[KS]) {
    read_frags<KS>(f, lds_addr(ring[wave][s % S]), foff);
  };
  const auto read_q = [&](int s, u32x4(&f)[NT][KS]) {
#pragma unroll
    for (int T = 0; T < NT; ++T) read_frags<KS>(f[T], q0 + ((s % H) * NT + T) * TB, foff);
  };
  const auto wait_frags = [&](u32x4(&k)[KS], u32x4(&q)[NT][KS]) {
    wait_lgkm<KS>(k);
#pragma unroll
    for (int T = 0; T < NT; ++T) wait_lgkm<KS>(q[T]);
  };
  float run[NS];
  // step s: MFMAs on the fragments in kc/qc while tile s+1's are read into kn/qn
  const auto step = [&](int s, u32x4(&kc)[KS], u32x4(&qc)[NT][KS], u32x4(&kn)[KS],
                        u32x4(&qn)[NT][KS]) {
    const int g = s % H;
    const bool last = g == H - 1;
    const int t = t0_of(s) + nl;
    // the values an accumulating call combines with, queued before the next tile
    float prev[NS];
    if (last && a.p.accumulate != KVS_ACC_WRITE) {
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const int j = 8 * (q / 4) + 4 * hl + (q % 4);
        prev[q] = (j < a.p.W && t < a.p.L) ? a.p.S[(int64_t)j * a.p.s_ld + t] : 0.f;
      }
    }
    if (s + S - 1 < steps) issue_k(s + S - 1);
    f32x16 acc[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      acc[T] = f32x16{};
#pragma unroll
      for (int k = 0; k < KS; ++k)
        acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qc[T][k]),
                                                         __builtin_bit_cast(bf16x8, kc[k]), acc[T],
                                                         0, 0, 0);
    }
    if (s + 1 < steps) {
      if (s + S - 1 < steps)
        wait_vm<KS>();   // tile s+1 in, tile s+2 may still be on its way
      else
        wait_vm<0>();
      read_k(s + 1, kn);
      read_q(s + 1, qn);
    }
    // reduce over the heads: row tile T, element i is head (32T + 8(i/4) + 4hl + i%4) / HR
    float v[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) v[q] = MAX ? kNegInf : 0.f;
#pragma unroll
    for (int T = 0; T < NT; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hq = (32 * T + 8 * (i / 4) + (i % 4)) / HR;   // same for both lane halves
        if (hq < a.p.G) v[i % NS] = raw_combine<MAX>(v[i % NS], acc[T][i] * a.p.scale);
      }
#pragma unroll
    for (int q = 0; q < NS; ++q) run[q] = g == 0 ? v[q] : raw_combine<MAX>(run[q], v[q]);
    if (last && t < a.p.L) {
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const int j = 8 * (q / 4) + 4 * hl + (q % 4);
        if (j < a.p.W) {
          float y = run[q];
          if (a.p.accumulate == KVS_ACC_ADD)
            y += prev[q];
          else if (a.p.accumulate == KVS_ACC_MAX)
            y = fmaxf(prev[q], y);
          a.p.S[(int64_t)j * a.p.s_ld + t] = y;
        }
      }
    }
    if (s + 1 < steps) wait_frags(kn, qn);
  };

  u32x4 k0[KS], k1[KS], q0f[NT][KS], q1f[NT][KS];
  if (steps > 0) {
    if (pre == 2)
      wait_vm<KS>();
    else
      wait_vm<0>();
    read_k(0, k0);
    read_q(0, q0f);
    wait_frags(k0, q0f);
  }
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, k0, q0f, k1, q1f);
    step(s + 1, k1, q1f, k0, q0f);
  }
  if (s < steps) step(s, k0, q0f, k1, q1f);
}

// ALL_SUM: the per-KV-head column sums the column-sum pass wrote into the
// workspace are added here in head order, S[0][t] (=|+=) sum over g.
__global__ __launch_bounds__(256) void score_head_sum_kernel(const float* __restrict__ rows,
                                                             int64_t rows_ld, int H, int L,
                                                             float* __restrict__ S,
                                                             int accumulate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  float v = 0.f;
  for (int g0 = 0; g0 < H; g0 += 8) {   // 8 rows loaded together, added in order
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = g0 + i < H ? rows[(int64_t)(g0 + i) * rows_ld + t] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (g0 + i < H) v = g0 + i == 0 ? x[i] : v + x[i];
  }
  store_out(S + t, v, accumulate);
}

// GROUP_MAX over two row groups: the per-head rows both groups wrote into the
// workspace are folded here, S[g][t] (=|+=) max over the G heads.
__global__ __launch_bounds__(256) void score_head_max_kernel(const float* __restrict__ rows,
                                                             int64_t rows_ld, int G, int L,
                                                             float* __restrict__ S, int64_t s_ld,
                                                             int accumulate) {
  const int g = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  const float* r = rows + (int64_t)g * G * rows_ld + t;
  float mx = r[0];
  for (int h0 = 1; h0 < G; h0 += 8) {   // 8 rows loaded together
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = h0 + i < G ? r[(int64_t)(h0 + i) * rows_ld] : mx;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, x[i]);
  }
  store_out(S + (int64_t)g * s_ld + t, mx, accumulate);
}

template <int D, int NT>
void launch_group(const KArgs& a, int pass, int mode, dim3 grid, hipStream_t stream) {
  if (pass == 1)
    hipLaunchKernelGGL((score_stats_kernel<D, NT>), grid, dim3(kThreads), 0, stream, a);
  else if (mode == 0)
    hipLaunchKernelGGL((score_colsum_kernel<D, NT, 0>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((score_colsum_kernel<D, NT, 1>), grid, dim3(kThreads), 0, stream, a);
}

// Launches the fused kernel; false (nothing launched) when the grid does not
// fit on the device at once.
template <int D, int NT>
bool launch_fused(const KArgs& a, int mode, dim3 grid, hipStream_t stream) {
  const void* fn = mode == 0 ? reinterpret_cast<const void*>(&score_fused_kernel<D, NT, 0>)
                             : reinterpret_cast<const void*>(&score_fused_kernel<D, NT, 1>);
  if ((int64_t)grid.x * grid.y > (int64_t)grid_capacity(fn, kThreads)) return false;
  if (mode == 0)
    hipLaunchKernelGGL((score_fused_kernel<D, NT, 0>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((score_fused_kernel<D, NT, 1>), grid, dim3(kThreads), 0, stream, a);
  return true;
}

template <int D>
bool launch_fused_nt(int nt, const KArgs& a, int mode, dim3 grid, hipStream_t stream) {
  switch (nt) {
    case 1: return launch_fused<D, 1>(a, mode, grid, stream);
    case 2: return launch_fused<D, 2>(a, mode, grid, stream);
    case 3: return launch_fused<D, 3>(a, mode, grid, stream);
    default: return launch_fused<D, 4>(a, mode, grid, stream);
  }
}

template <int D>
void launch_group_nt(int nt, const KArgs& a, int pass, int mode, dim3 grid, hipStream_t stream) {
  switch (nt) {
    case 1: launch_group<D, 1>(a, pass, mode, grid, stream); break;
    case 2: launch_group<D, 2>(a, pass, mode, grid, stream); break;
    case 3: launch_group<D, 3>(a, pass, mode, grid, stream); break;
    default: launch_group<D, 4>(a, pass, mode, grid, stream); break;
  }
}

// Pass 1 of every row group, then pass 2 of every row group.  With two row
// groups, GROUP_SUM (and any head mode of a single query head, whose rows are
// split) adds the second group's column sums to the first's; NONE writes each
// group's own heads; GROUP_MAX writes the per-head rows of both groups into
// the workspace and folds them with score_head_max_kernel.
template <int D>
kvs_status launch_d(const ScorePlan& pl, const ScoreLaunch& p, hipStream_t stream) {
  KArgs a;
  a.p = p;
  a.head_rows = pl.head_rows;
  a.rows_pad = pl.rows_pad;
  a.n_split = pl.n_split;
  a.tps = pl.tiles_per_split;
  a.n_tiles = pl.n_tiles;
  a.g0 = 0;
  const int64_t mv = p.q_pos0 < (int64_t)p.L - 1 ? p.q_pos0 : (int64_t)p.L - 1;
  a.min_vis = (int)mv;
  a.rev = pl.reverse;
  const dim3 grid(pl.n_split, p.H_kv);
  const bool split_max = pl.n_groups > 1 && p.heads == KVS_HEADS_GROUP_MAX && p.G > 1;
  const bool all_sum = p.heads == KVS_HEADS_ALL_SUM;
  const int mode =
      (p.heads == KVS_HEADS_GROUP_SUM || all_sum || pl.head_rows > 128) ? 0 : 1;
  a.flag = p.flags;
  a.epoch = 0;
  a.wait_ticks = grid_wait_ticks();
  // Both passes of a single row group in one launch when the device can hold
  // the whole grid at once.
  if (p.phase == 0 && pl.n_groups == 1 && p.flags) {
    a.row0 = pl.grp_row0[0];
    a.h0 = pl.grp_h0[0];
    a.h1 = pl.grp_h1[0];
    a.per_head = p.heads == KVS_HEADS_NONE;
    a.out = all_sum ? p.head_rows_ws : p.S;
    a.out_ld = all_sum ? (int64_t)p.L : p.s_ld;
    a.acc = all_sum ? 0 : p.accumulate;
    a.epoch = grid_epoch();
    if (launch_fused_nt<D>(pl.grp_rows[0] / 32, a, mode, grid, stream)) {
      if (all_sum)
        hipLaunchKernelGGL(score_head_sum_kernel, dim3((p.L + 255) / 256), dim3(256), 0, stream,
                           p.head_rows_ws, (int64_t)p.L, p.H_kv, p.L, p.S, p.accumulate);
      return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
    }
  }
  for (int pass = 1; pass <= 2; ++pass) {
    if ((pass == 1 && p.phase == 2) || (pass == 2 && p.phase == 1)) continue;
    for (int gr = 0; gr < pl.n_groups; ++gr) {
      a.row0 = pl.grp_row0[gr];
      a.h0 = pl.grp_h0[gr];
      a.h1 = pl.grp_h1[gr];
      a.acc = (mode == 0 && gr > 0) ? 1 : p.accumulate;
      a.per_head = p.heads == KVS_HEADS_NONE || split_max;
      a.out = (split_max || all_sum) ? p.head_rows_ws : p.S;
      a.out_ld = (split_max || all_sum) ? (int64_t)p.L : p.s_ld;
      if (split_max || all_sum) a.acc = gr > 0 && mode == 0 ? 1 : 0;
      launch_group_nt<D>(pl.grp_rows[gr] / 32, a, pass, mode, grid, stream);
    }
    if (pass == 2 && all_sum)
      hipLaunchKernelGGL(score_head_sum_kernel, dim3((p.L + 255) / 256), dim3(256), 0, stream,
                         p.head_rows_ws, (int64_t)p.L, p.H_kv, p.L, p.S, p.accumulate);
    if (pass == 2 && split_max)
      hipLaunchKernelGGL(score_head_max_kernel, dim3((p.L + 255) / 256, p.H_kv), dim3(256), 0,
                         stream, p.head_rows_ws, (int64_t)p.L, p.G, p.L, p.S, p.s_ld,
                         p.accumulate);
  }
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace

kvs_status score_plan(const kvs_score_args* a, ScorePlan* pl) {
  const int G = a->H_q / a->H_kv;
  const int W = a->W;
  const int hr = W <= 4 ? 4 : W <= 8 ? 8 : W <= 16 ? 16 : (W + 31) / 32 * 32;
  if ((int64_t)G * hr > 256) return KVS_EUNSUPPORTED;
  pl->head_rows = hr;
  pl->rows_pad = (G * hr + 31) / 32 * 32;
  pl->n_tiles = (a->L + 31) / 32;
  // Row groups of at most 128 padded rows, the query rows a wave keeps as
  // MFMA operands.  Two groups split at a head boundary, or, for a single
  // query head with more than 128 rows, at row 128.
  if (pl->rows_pad <= 128) {
    pl->n_groups = 1;
    pl->grp_row0[0] = 0;
    pl->grp_rows[0] = pl->rows_pad;
    pl->grp_h0[0] = 0;
    pl->grp_h1[0] = G;
  } else {
    pl->n_groups = 2;
    const int hpg = hr <= 128 ? 128 / hr : 0;   // heads in the first group (0: one head split)
    const int r1 = hr <= 128 ? hpg * hr : 128;
    pl->grp_row0[0] = 0;
    pl->grp_rows[0] = hr <= 128 ? (r1 + 31) / 32 * 32 : 128;
    pl->grp_row0[1] = r1;
    pl->grp_rows[1] = pl->rows_pad - r1;
    pl->grp_h0[0] = 0;
    pl->grp_h1[0] = hr <= 128 ? hpg : G;
    pl->grp_h0[1] = hr <= 128 ? hpg : 0;
    pl->grp_h1[1] = G;
  }
  // Every KV head in one round (one pass-1 launch, one pass-2 launch per row
  // group).  The key range of each head is cut into splits so that the grid
  // holds one 4-wave workgroup per CU (256 CUs), each streaming a contiguous
  // run of tiles, and at least 4 tiles (one per wave).  The plan depends only
  // on the arguments, so the workspace, phase 1 and phase 2 always agree.
  pl->head_batch = a->H_kv;
  pl->reverse = 1;
  const int per_head = (256 + a->H_kv - 1) / a->H_kv;
  const int max_split = pl->n_tiles / 4 > 1 ? pl->n_tiles / 4 : 1;
  int ns = per_head < max_split ? per_head : max_split;
  if (ns < 1) ns = 1;
  const int tps = (pl->n_tiles + ns - 1) / ns;
  pl->tiles_per_split = tps;
  pl->n_split = (pl->n_tiles + tps - 1) / tps;
  pl->ws_stats = align_up((size_t)a->H_kv * pl->n_split * pl->rows_pad * sizeof(float2), kWsAlign);
  // GROUP_MAX over two row groups keeps every query head's column sums; the
  // sum over every head keeps each KV head's
  const bool split_max = pl->n_groups > 1 && a->heads == KVS_HEADS_GROUP_MAX && G > 1;
  pl->ws_heads = split_max ? align_up((size_t)a->H_q * a->L * sizeof(float), kWsAlign)
                 : a->heads == KVS_HEADS_ALL_SUM
                     ? align_up((size_t)a->H_kv * a->L * sizeof(float), kWsAlign)
                     : 0;
  pl->ws_flags = align_up((size_t)a->H_kv * pl->n_split * sizeof(uint64_t), kWsAlign);
  pl->ws_total = pl->ws_stats + pl->ws_heads + pl->ws_flags;
  return KVS_OK;
}

namespace {

template <int D, int HR, int NT>
kvs_status raw_launch(const RawLaunch& p, hipStream_t stream) {
  if (p.H_kv * NT > raw_q_tiles<D>()) return KVS_EUNSUPPORTED;
  RawArgs a;
  a.p = p;
  a.n_tiles = (p.L + 31) / 32;
  // One 4-wave workgroup per CU, each over a contiguous run of key tiles (of
  // every KV head), at least one tile per wave.
  const int max_split = a.n_tiles / kWaves > 1 ? a.n_tiles / kWaves : 1;
  const int ns = 256 < max_split ? 256 : max_split;
  a.tps = (a.n_tiles + ns - 1) / ns;
  const int n_split = (a.n_tiles + a.tps - 1) / a.tps;
  if (p.reduce_max)
    hipLaunchKernelGGL((score_raw_kernel<D, HR, NT, true>), dim3(n_split), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((score_raw_kernel<D, HR, NT, false>), dim3(n_split), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

template <int D, int HR>
kvs_status raw_launch_hr(const RawLaunch& p, hipStream_t stream) {
  switch ((p.G * HR + 31) / 32) {
    case 1: return raw_launch<D, HR, 1>(p, stream);
    case 2: return raw_launch<D, HR, 2>(p, stream);
    case 3: return raw_launch<D, HR, 3>(p, stream);
    case 4: return raw_launch<D, HR, 4>(p, stream);
    default: return KVS_EUNSUPPORTED;
  }
}

template <int D>
kvs_status raw_launch_d(const RawLaunch& p, hipStream_t stream) {
  switch (p.head_rows) {
    case 8: return raw_launch_hr<D, 8>(p, stream);
    case 16: return raw_launch_hr<D, 16>(p, stream);
    case 32: return raw_launch_hr<D, 32>(p, stream);
    default: return KVS_EUNSUPPORTED;
  }
}

}  // namespace

namespace {

// ------------------------------------------------------------------ DELTA decode pages
// kvs_delta_pages, scores half: for every sequence of the batch, the decode
// query's logits against its cached keys and the softmax statistics per head
// (delta_logits_kernel), then the page scores: per token the maximum over heads
// of the softmax probability, summed over each page (delta_page_kernel).
// A decode query is one row per head, so the logits of all heads (128 B per
// token at 32 heads) are cheaper to keep than a second pass over K
// (2 KiB per token at 8 KV heads x 128 dims): the first kernel writes them,
// head-major and in log2 units, and the second reads them back.
// delta_logits_kernel: one workgroup per (chunk of keys, sequence); each wave
// streams (key tile, KV head) pairs like the raw-logit kernel, with all the
// sequence's query rows (one per head) in LDS and the MFMA tile oriented
// rows x keys.  A lane keeps, per key tile, the 16 logits of the rows it holds,
// each taken from the step whose KV head owns the row, then writes them and
// folds them into per-lane online statistics.
struct DeltaArgs {
  DeltaLaunch p;
  int sel;   // one-launch form: the last chunk of each sequence also selects its pages
};

// Log-sum-exp folds of the DELTA kernels with a fixed rounding order (the
// running sum's product rounded, the incoming term's fused), so that every
// kernel folds the same statistics to the same bits whatever contraction
// the compiler would otherwise choose in each.
// (m, z) <- (m, z) combined with (m2, z2):
__device__ __forceinline__ void lse_fold(float& m, float& z, float m2, float z2) {
  const float mx = fmaxf(m, m2);
  z = mx == kNegInf ? 0.f : __builtin_fmaf(z2, ex2(m2 - mx), z * ex2(m - mx));
  m = mx;
}
// (m, z) <- (m, z) with one more term x:
__device__ __forceinline__ void lse_add(float& m, float& z, float x) {
  const float mn = fmaxf(m, x);
  z = __builtin_fmaf(z, ex2(m - mn), ex2(x - mn));
  m = mn;
}

template <int D>
__device__ __forceinline__ void issue_delta_q(uint8_t* dst, const DeltaLaunch& p, int b, int T,
                                              int lane) {
  constexpr int CR = D / 8;
  constexpr int RPI = 64 / CR;
  const int pc = lane % CR;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const int tr = j * RPI + lane / CR;
    const int h = 32 * T + tr;
    const uint16_t* row = p.Q + ((int64_t)b * p.H_q + (h < p.H_q ? h : 0)) * D;
    const int c = pc ^ (tr % CR);
    __builtin_amdgcn_global_load_lds(row + 8 * c, (lds_void*)(dst + j * 1024), 16, 0, 0);
  }
}

template <int D, int NT>
__global__ __launch_bounds__(kThreads, 1) void delta_logits_kernel(DeltaArgs a) {
  constexpr int KS = D / 16;
  constexpr int S = kRawStages;
  constexpr int TB = tile_bytes<D>();
  __shared__ __attribute__((aligned(16))) uint8_t qs[NT][TB];
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][S][TB];
  __shared__ float2 red[kWaves][32 * NT];
  const DeltaLaunch& p = a.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 31, hl = lane >> 5;
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int Lb = min(max(p.L[b], 0), p.L_max);
  const int tb = chunk * p.chunk;
  if (tb >= Lb) return;   // the whole workgroup: nothing of this sequence here
  const int te = min(tb + p.chunk, Lb);
  const uint16_t* Kb = p.K[b];
  const int64_t khs = p.khs ? p.khs : (int64_t)Lb * D;
  const int H = p.H_kv;
  const int n_tiles = (te - tb + 31) / 32;
  const int nt = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;
  const int steps = nt * H;   // (key tile, KV head) pairs, KV head fastest
  const auto t0_of = [&](int s) { return tb + (wave + kWaves * (s / H)) * 32; };
  const auto issue_k = [&](int s) {
    issue_tile<D>(ring[wave][s % S], Kb + (int64_t)(s % H) * khs, p.kts, t0_of(s), Lb, lane);
  };

  for (int u = wave; u < NT; u += kWaves) issue_delta_q<D>(qs[u], p, b, u, lane);
  const int pre = steps < S - 1 ? steps : S - 1;
  for (int s = 0; s < pre; ++s) issue_k(s);
  if (pre == 2)
    wait_vm<2 * KS>();
  else if (pre == 1)
    wait_vm<KS>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();   // bare: a fenced barrier would wait for the K tiles too

  uint32_t foff[KS];
  frag_offsets<D>(foff, lane);
  const uint32_t q0 = lds_addr(qs[0]);
  float out[NT][16];
  float m[NT][16], z[NT][16];
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      out[T][i] = 0.f;
      m[T][i] = kNegInf;
      z[T][i] = 0.f;
    }
  float* x2b = p.x2 + (int64_t)b * p.H_q * p.x2_ld;
  // the KV head owning each of this lane's rows (H_kv for padding rows)
  int own[NT][16];
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = 32 * T + 8 * (i / 4) + 4 * hl + (i % 4);
      own[T][i] = h < p.H_q ? h / p.G : H;
    }
  // the row tiles holding KV head g's query heads
  const auto t_lo = [&](int g) { return (g * p.G) / 32; };
  const auto t_hi = [&](int g) { return (g * p.G + p.G - 1) / 32; };
  // With one row tile (H_q <= 32) the query fragments stay in registers for
  // the whole loop; with more, each step reads those of the row tiles it
  // needs.  The next step's K fragments are read while this step's MFMAs run.
  constexpr bool PQ = NT == 1;
  u32x4 qf[KS];
  const auto step = [&](int s, u32x4(&kc)[KS], u32x4(&kn)[KS]) {
    const int g = s % H;
    if (s + S - 1 < steps) issue_k(s + S - 1);
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      if (T < t_lo(g) || T > t_hi(g)) continue;
      if constexpr (!PQ) {
        read_frags<KS>(qf, q0 + T * TB, foff);
        wait_lgkm<KS>(qf);
      }
      const u32x4(&qc)[KS] = qf;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int k = 0; k < KS; ++k)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qc[k]),
                                                      __builtin_bit_cast(bf16x8, kc[k]), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) out[T][i] = own[T][i] == g ? acc[i] * p.c : out[T][i];
    }
    if (s + 1 < steps) {
      if (s + S - 1 < steps)
        wait_vm<KS>();   // tile s+1 in, tile s+2 may still be on its way
      else
        wait_vm<0>();
      read_frags<KS>(kn, lds_addr(ring[wave][(s + 1) % S]), foff);
    }
    if (g == H - 1) {
      // every head's logit of key t is in: store it and fold it into the statistics
      const int t = t0_of(s) + nl;
      const bool valid = t < Lb;
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int h = 32 * T + 8 * (i / 4) + 4 * hl + (i % 4);
          if (valid && own[T][i] < H) {
            const float x = out[T][i];
            x2b[(int64_t)h * p.x2_ld + t] = x;
            lse_add(m[T][i], z[T][i], x);
          }
        }
    }
    if (s + 1 < steps) wait_lgkm<KS>(kn);
  };
  u32x4 k0[KS], k1[KS];
  if (steps > 0) {
    if (pre == 2)
      wait_vm<KS>();
    else
      wait_vm<0>();
    read_frags<KS>(k0, lds_addr(ring[wave][0]), foff);
    wait_lgkm<KS>(k0);
    if constexpr (PQ) {
      read_frags<KS>(qf, q0, foff);
      wait_lgkm<KS>(qf);
    }
  }
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, k0, k1);
    step(s + 1, k1, k0);
  }
  if (s < steps) step(s, k0, k1);
  // statistics of each row over the workgroup's keys: lanes of a half, then waves
#pragma unroll
  for (int T = 0; T < NT; ++T)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float mm = m[T][i], zz = z[T][i];
#pragma unroll
      for (int d = 1; d < 32; d *= 2) {
        const float m2 = __shfl_xor(mm, d), z2 = __shfl_xor(zz, d);
        lse_fold(mm, zz, m2, z2);
      }
      if (nl == 0) red[wave][32 * T + 8 * (i / 4) + 4 * hl + (i % 4)] = make_float2(mm, zz);
    }
  __syncthreads();
  for (int h = threadIdx.x; h < p.H_q; h += kThreads) {
    float mm = kNegInf, zz = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 v = red[w][h];
      lse_fold(mm, zz, v.x, v.y);
    }
    p.cstats[((int64_t)b * p.n_chunk + chunk) * p.H_q + h] = make_float2(mm, zz);
  }
}

// delta_page_kernel: one workgroup per (chunk of kDeltaPageTokens tokens,
// sequence), a thread per token.  The thread first issues the loads of its
// token's logits for the first kDeltaBatch heads (coalesced over the
// head-major logits), then folds the sequence's per-chunk statistics into b_h
// = m_h + log2 Z_h per head while they are in flight, forms s_t = max over
// heads of exp2(x_t,h - b_h), and sums each page's tokens left to right.
constexpr int kDeltaPageTokens = 512;
constexpr int kDeltaBatch = 32;

__global__ __launch_bounds__(kDeltaPageTokens) void delta_page_kernel(DeltaArgs a) {
  constexpr int NTH = kDeltaPageTokens;   // threads
  __shared__ float bh[128];
  __shared__ float ys[kDeltaPageTokens];
  __shared__ float2 part[NTH];
  const DeltaLaunch& p = a.p;
  const int b = blockIdx.y;
  const int Lb = min(max(p.L[b], 0), p.L_max);
  const int t_begin = blockIdx.x * kDeltaPageTokens;
  if (t_begin >= Lb) return;
  const int t_end = min(t_begin + kDeltaPageTokens, Lb);
  const int t = t_begin + (int)threadIdx.x;
  const bool has_t = t < t_end;
  const float* x2b = p.x2 + (int64_t)b * p.H_q * p.x2_ld;
  // 0. this token's logits of the first heads, in flight during step 1
  float v[kDeltaBatch];
#pragma unroll
  for (int q = 0; q < kDeltaBatch; ++q)
    v[q] = has_t && q < p.H_q ? x2b[(int64_t)q * p.x2_ld + t] : kNegInf;
  // 1. row constants: threads per head fold a strided share of the chunks
  const int tph = NTH / p.H_q;                  // threads per head (H_q <= 128)
  const int h = threadIdx.x / tph, j = threadIdx.x % tph;
  const int nch = (Lb + p.chunk - 1) / p.chunk;
  float mm = kNegInf, zz = 0.f;
  if (h < p.H_q) {
    const float2* cs = p.cstats + (int64_t)b * p.n_chunk * p.H_q + h;
    constexpr int kCsBatch = 16;
    for (int c0 = j; c0 < nch; c0 += kCsBatch * tph) {
      float2 w[kCsBatch];
#pragma unroll
      for (int q = 0; q < kCsBatch; ++q) {
        const int c = c0 + q * tph;
        w[q] = c < nch ? cs[(int64_t)c * p.H_q] : make_float2(kNegInf, 0.f);
      }
#pragma unroll
      for (int q = 0; q < kCsBatch; ++q) lse_fold(mm, zz, w[q].x, w[q].y);
    }
  }
  part[threadIdx.x] = make_float2(mm, zz);
  __syncthreads();
  if (threadIdx.x < p.H_q) {
    float m2 = kNegInf, z2 = 0.f;
    for (int q = 0; q < tph; ++q) {
      const float2 w = part[threadIdx.x * tph + q];
      lse_fold(m2, z2, w.x, w.y);
    }
    bh[threadIdx.x] = m2 + log2f(z2);
  }
  __syncthreads();
  // 2. token score: max over heads of the softmax probability
  float sv = 0.f;
#pragma unroll
  for (int q = 0; q < kDeltaBatch; ++q)
    if (q < p.H_q) sv = fmaxf(sv, ex2(v[q] - bh[q]));
  for (int h0 = kDeltaBatch; h0 < p.H_q; h0 += kDeltaBatch) {
#pragma unroll
    for (int q = 0; q < kDeltaBatch; ++q)
      v[q] = has_t && h0 + q < p.H_q ? x2b[(int64_t)(h0 + q) * p.x2_ld + t] : kNegInf;
#pragma unroll
    for (int q = 0; q < kDeltaBatch; ++q)
      if (h0 + q < p.H_q) sv = fmaxf(sv, ex2(v[q] - bh[h0 + q]));
  }
  if (has_t) ys[t - t_begin] = sv;
  __syncthreads();
  // 3. page sums, left to right (chunk boundaries are multiples of P)
  const int u0 = t_begin / p.P, u1 = (t_end + p.P - 1) / p.P;
  float* Sb = p.S + (int64_t)b * p.n_pages_max;
  for (int u = u0 + (int)threadIdx.x; u < u1; u += NTH) {
    const int a0 = u * p.P, a1 = min(a0 + p.P, t_end);
    float acc = 0.f;
    for (int tt = a0; tt < a1; ++tt) acc += ys[tt - t_begin];
    Sb[u] = acc;
  }
}

// ------------------------------------------------------------------ DELTA in one launch
// When the logits of the whole batch fit in registers (one row tile, H_q <=
// 32, and at most kDeltaKeepTiles key tiles per wave: 16 floats per lane and
// tile) and the grid is resident at once, one launch does what the two
// kernels above do, without writing the logits anywhere: each workgroup
// streams its chunk as delta_logits_kernel does and keeps its logits in
// registers, publishes its chunk's statistics (flags as in the one-launch
// score form, see grid_sync.h), waits for the other chunks of its
// sequence, folds them into b_h in delta_page_kernel's order, and forms the
// token and page scores from its registers.  Results are bit-identical to
// the two kernels'.  A chunk still unpublished at the wait bound is computed
// by the waiter (statistics only), bit-identically.  With the selection in
// the launch too, the page scores also go out as words tagged with the
// launch, and the workgroup that finds all of its sequence's words tagged
// selects the pages (topk_delta_kernel's selection, in one wave when the
// pages fit it).
constexpr int kDeltaKeepTiles = 8;
// K ring stages per wave of the one-launch form (a fourth was no faster).
constexpr int kDeltaStages = 3;

// Streams chunk `chunk` of sequence b (logits of every head, as
// delta_logits_kernel) and stores its per-head statistics with device-scope
// atomic stores; RETAIN keeps tile j's logits (this lane's 16 rows of key
// t0 + lane % 32) in keep[j].
template <int D, bool RETAIN>
__device__ __forceinline__ void delta_chunk_pass(const DeltaLaunch& p, int b, int chunk,
                                                 uint8_t (&qs)[tile_bytes<D>()],
                                                 uint8_t (&ring)[kWaves][kDeltaStages][tile_bytes<D>()],
                                                 float2 (&red)[kWaves][32],
                                                 float (&keep)[kDeltaKeepTiles][16]) {
  constexpr int KS = D / 16;
  constexpr int S = kDeltaStages;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 31, hl = lane >> 5;
  const int Lb = min(max(p.L[b], 0), p.L_max);
  const int tb = chunk * p.chunk;
  const int te = min(tb + p.chunk, Lb);
  const uint16_t* Kb = p.K[b];
  const int64_t khs = p.khs ? p.khs : (int64_t)Lb * D;
  const int H = p.H_kv;
  // KV heads in an order rotated per workgroup, so that the workgroups do not
  // all read the same head's region at the same offset at once
  const int rot = (chunk + b) % H;
  const int n_tiles = (te - tb + 31) / 32;
  const int nt = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;
  const int steps = nt * H;   // (key tile, KV head) pairs, KV head fastest
  const auto t0_of = [&](int s) { return tb + (wave + kWaves * (s / H)) * 32; };
  const auto issue_k = [&](int s) {
    issue_tile<D>(ring[wave][s % S], Kb + (int64_t)((s % H + rot) % H) * khs, p.kts, t0_of(s), Lb, lane);
  };
  // at most n tiles' loads of this wave still in flight (n wave-uniform)
  const auto wait_tiles = [&](int n) {
    static_assert(S <= 4, "wait_tiles covers up to three tiles in flight");
    if (n >= 3)
      wait_vm<3 * KS>();
    else if (n == 2)
      wait_vm<2 * KS>();
    else if (n == 1)
      wait_vm<KS>();
    else
      wait_vm<0>();
  };
  if (wave == 0) issue_delta_q<D>(qs, p, b, 0, lane);
  const int pre = steps < S - 1 ? steps : S - 1;
  for (int s = 0; s < pre; ++s) issue_k(s);
  wait_tiles(pre);   // wave 0's query rows, issued first, are in
  __builtin_amdgcn_s_barrier();   // bare: a fenced barrier would wait for the K tiles too

  uint32_t foff[KS];
  frag_offsets<D>(foff, lane);
  float out[16], m[16], z[16];
  int own[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    out[i] = 0.f;
    m[i] = kNegInf;
    z[i] = 0.f;
    const int h = 8 * (i / 4) + 4 * hl + (i % 4);
    own[i] = h < p.H_q ? h / p.G : H;
  }
  u32x4 qf[KS];
  const auto step = [&](int s, u32x4(&kc)[KS], u32x4(&kn)[KS]) {
    const int g = (s % H + rot) % H;
    if (s + S - 1 < steps) issue_k(s + S - 1);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int k = 0; k < KS; ++k)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qf[k]),
                                                    __builtin_bit_cast(bf16x8, kc[k]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = own[i] == g ? acc[i] * p.c : out[i];
    if (s + 1 < steps) {
      // tile s+1 in; the tiles issued after it may still be on their way
      wait_tiles(min(S - 2, steps - 2 - s));
      read_frags<KS>(kn, lds_addr(ring[wave][(s + 1) % S]), foff);
    }
    if (s % H == H - 1) {   // the tile's last step
      // every head's logit of key t is in: keep it and fold it into the statistics
      const int t = t0_of(s) + nl;
      const bool valid = t < Lb;
      if constexpr (RETAIN) {
        const int j = s / H;
#pragma unroll
        for (int jj = 0; jj < kDeltaKeepTiles; ++jj)
#pragma unroll
          for (int i = 0; i < 16; ++i) keep[jj][i] = jj == j ? out[i] : keep[jj][i];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (valid && own[i] < H) lse_add(m[i], z[i], out[i]);
      }
    }
    if (s + 1 < steps) wait_lgkm<KS>(kn);
  };
  u32x4 k0[KS], k1[KS];
  if (steps > 0) {
    wait_tiles(pre - 1);
    read_frags<KS>(k0, lds_addr(ring[wave][0]), foff);
    wait_lgkm<KS>(k0);
    read_frags<KS>(qf, lds_addr(qs), foff);
    wait_lgkm<KS>(qf);
  }
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, k0, k1);
    step(s + 1, k1, k0);
  }
  if (s < steps) step(s, k0, k1);
  // statistics of each row over the workgroup's keys: lanes of a half, then waves
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float mm = m[i], zz = z[i];
#pragma unroll
    for (int d = 1; d < 32; d *= 2) {
      const float m2 = __shfl_xor(mm, d), z2 = __shfl_xor(zz, d);
      lse_fold(mm, zz, m2, z2);
    }
    if (nl == 0) red[wave][8 * (i / 4) + 4 * hl + (i % 4)] = make_float2(mm, zz);
  }
  __syncthreads();
  for (int h = threadIdx.x; h < p.H_q; h += kThreads) {
    float mm = kNegInf, zz = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 v = red[w][h];
      lse_fold(mm, zz, v.x, v.y);
    }
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p.cstats + ((int64_t)b * p.n_chunk + chunk) * p.H_q + h),
                       __builtin_bit_cast(uint64_t, make_float2(mm, zz)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// rho of sequence b from its page scores: the top K - L older pages
// (ascending), the last min(L, pages) pages, then -1, as topk_delta_kernel
// computes it, with kThreads threads of kKpt pages each.  The scores are the
// tagged words the chunks of the sequence stored earlier in the launch, read
// with device-scope loads; when any word does not carry `tag` yet, some
// chunk is still to store its pages, and the call returns (in every thread,
// having written nothing) with *all = 0.  *all must be 1 on entry, set
// before a barrier.
__device__ __forceinline__ void delta_select(const DeltaLaunch& p, int b, uint32_t* hist,
                                             Shared& sh, const uint64_t* words, uint32_t tag,
                                             int* all) {
  const int Lb = min(max(p.L[b], 0), p.L_max);
  const int n_pages = (Lb + p.P - 1) / p.P;
  const int n_recent = min(p.L_recent, n_pages);
  const int n_cand = n_pages - n_recent;
  const int keep = min(p.K_pages - p.L_recent, n_cand);
  int32_t* out = p.rho + (int64_t)b * p.K_pages;
  const int i0 = (int)threadIdx.x * kKpt;
  uint32_t o[kKpt], valid = 0;
  // Threads past the pages load nothing; within a thread the indices are
  // clamped with no branch, so all its loads are in flight at once.
  const int last = n_cand > 0 ? n_cand - 1 : 0;
  bool ok = true;
  if (i0 < n_cand) {
    uint64_t raw[kKpt];
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      raw[e] = __hip_atomic_load(words + min(i0 + e, last), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const bool in = i0 + e < n_cand;
      valid |= in ? (1u << e) : 0u;
      ok &= !in || (uint32_t)(raw[e] >> 32) == tag;
      o[e] = ord_key(in ? __uint_as_float((uint32_t)raw[e]) : 0.f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kKpt; ++e) o[e] = 0u;
  }
  if (!__all(ok) && (threadIdx.x & 63) == 0) *all = 0;
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*all)) return;
  if (n_cand <= 64 * kKpt) {
    // every page is in wave 0: it selects alone, the other waves are done
    if (threadIdx.x >= 64) return;
    Kstar ks{0u, 0u, 0u};
    uint32_t gt = valid, eq = 0u;
    if (keep == 0) {
      gt = 0u;
    } else if (keep < n_cand) {
      ks = select_wave(o, valid, (uint32_t)keep, hist);
      classify(o, 0u, valid, ks, gt, eq);
    }
    uint32_t pos, rank;
    place_wave(gt, eq, ks.need_eq, pos, rank);
#pragma unroll
    for (int e = 0; e < kKpt; ++e) {
      const bool q = (eq >> e) & 1u;
      if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) out[pos++] = i0 + e;
      rank += q;
    }
    for (int i = threadIdx.x; i < p.K_pages - keep; i += 64)
      out[keep + i] = i < n_recent ? n_cand + i : -1;
    return;
  }
  int ph = 0;
  Kstar ks{0u, 0u, 0u};
  uint32_t gt = valid, eq = 0u;
  if (keep == 0) {
    gt = 0u;
  } else if (keep < n_cand) {
    ks = select_regs<kThreads>(o, 0u, valid, (uint32_t)keep, hist, sh, ph);
    classify(o, 0u, valid, ks, gt, eq);
  }
  uint32_t pos, rank, tg, te;
  place<kThreads>(gt, eq, ks.need_eq, 0u, 0u, sh, ph, pos, rank, tg, te);
#pragma unroll
  for (int e = 0; e < kKpt; ++e) {
    const bool q = (eq >> e) & 1u;
    if (((gt >> e) & 1u) || (q && rank < ks.need_eq)) out[pos++] = i0 + e;
    rank += q;
  }
  for (int i = threadIdx.x; i < p.K_pages - keep; i += kThreads)
    out[keep + i] = i < n_recent ? n_cand + i : -1;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void delta_fused_kernel(DeltaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t qs[tile_bytes<D>()];
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kDeltaStages][tile_bytes<D>()];
  __shared__ float2 red[kWaves][32];
  __shared__ float bh[32];
  __shared__ float ys[kDeltaKeepTiles * kWaves * 32];
  __shared__ int sh;
  __shared__ Shared ssel;
  const DeltaLaunch& p = a.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 31, hl = lane >> 5;
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int Lb = min(max(p.L[b], 0), p.L_max);
  const int tb = chunk * p.chunk;
  if (tb >= Lb) {   // the whole workgroup: nothing of this sequence here
    if (a.sel && chunk == 0) {   // an empty sequence's row
      if (threadIdx.x == 0) sh = 1;
      __syncthreads();
      delta_select(p, b, nullptr, ssel, nullptr, 0u, &sh);
    }
    return;
  }
  const int te = min(tb + p.chunk, Lb);
  float keep[kDeltaKeepTiles][16];
  delta_chunk_pass<D, true>(p, b, chunk, qs, ring, red, keep);
  uint64_t* flags = p.flags + (int64_t)b * p.n_chunk;
  publish_flag(flags + chunk, p.epoch);
  const int nch = (Lb + p.chunk - 1) / p.chunk;
  if (!wait_flags(flags, p.epoch, nch, p.wait_ticks, &sh)) {
    for (int c = 0; c < nch; ++c) {
      if (threadIdx.x == 0)
        sh = __hip_atomic_load(flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.epoch;
      __syncthreads();
      const int done = __builtin_amdgcn_readfirstlane(sh);
      __syncthreads();
      if (!done) {
        delta_chunk_pass<D, false>(p, b, c, qs, ring, red, keep);
        publish_flag(flags + c, p.epoch);
      }
    }
  }
  // b_h = m_h + log2 Z_h over the sequence's chunks, folded in the order
  // delta_page_kernel folds them (strided shares of its threads per head,
  // then the shares in turn), so the two paths agree bit for bit.  The
  // statistics are first staged in the idle K ring, one load per thread, all
  // in flight together; a sequence with more than the ring holds is read in
  // place.
  {
    const float2* cs = p.cstats + (int64_t)b * p.n_chunk * p.H_q;
    float2* st = reinterpret_cast<float2*>(&ring[0][0][0]);
    constexpr int kStaged = (int)(sizeof(ring) / sizeof(float2));
    const int n_st = nch * p.H_q;
    const bool staged = n_st <= kStaged;
    if (staged) {
      for (int i = threadIdx.x; i < n_st; i += kThreads)
        st[i] = __builtin_bit_cast(
            float2, __hip_atomic_load(reinterpret_cast<const uint64_t*>(cs + i), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT));
      __syncthreads();
    }
    // Shares past the last chunk are empty, and folding an empty share leaves
    // finite statistics unchanged, so they are skipped.
    if (threadIdx.x < p.H_q) {
      const int h = threadIdx.x;
      const int tph = kDeltaPageTokens / p.H_q;
      float m2 = kNegInf, z2 = 0.f;
      if (staged && nch <= tph) {
        // share j is chunk j alone: the statistics are read ahead in batches,
        // so only the folds into (m2, z2) form a chain
        constexpr int kB = 8;
        for (int j0 = 0; j0 < nch; j0 += kB) {
          float2 w[kB];
#pragma unroll
          for (int q = 0; q < kB; ++q) w[q] = st[min(j0 + q, nch - 1) * p.H_q + h];
#pragma unroll
          for (int q = 0; q < kB; ++q) {
            if (j0 + q < nch) {
              float mm = kNegInf, zz = 0.f;
              lse_fold(mm, zz, w[q].x, w[q].y);
              lse_fold(m2, z2, mm, zz);
            }
          }
        }
      } else {
        for (int j = 0; j < min(tph, nch); ++j) {
          float mm = kNegInf, zz = 0.f;
          for (int c = j; c < nch; c += tph) {
            const float2 w =
                staged ? st[c * p.H_q + h]
                       : __builtin_bit_cast(
                             float2, __hip_atomic_load(
                                         reinterpret_cast<const uint64_t*>(cs + (int64_t)c * p.H_q + h),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            lse_fold(mm, zz, w.x, w.y);
          }
          lse_fold(m2, z2, mm, zz);
        }
      }
      bh[h] = m2 + log2f(z2);
    }
    __syncthreads();
  }
  // Token scores: the maximum over heads of exp2(x - b_h), this lane's 16
  // rows, then the other half's.  exp2 (v_exp_f32) is non-decreasing over
  // every non-NaN float, so that maximum is exp2 of the largest x - b_h: one
  // exp2 per token, the same value bit for bit.
  const int n_tiles = (te - tb + 31) / 32;
  const int nt = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;
  float bl[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h = 8 * (i / 4) + 4 * hl + (i % 4);
    bl[i] = h < p.H_q ? bh[h] : kPosInf;   // x - inf = -inf: no say in the maximum
  }
  // Page sums, left to right (the chunk is a whole number of pages).  With
  // pages of 16 tokens a page is one 16-lane row of a tile: after step s of a
  // running sum along the row, lane k (k <= s) holds the left-to-right sum of
  // the row's lanes 0..k, the order the other form sums in.
  const bool row_pages = p.P == 16;
  float* Sb = p.S + (int64_t)b * p.n_pages_max;
  uint64_t* Wb = p.pwords + (int64_t)b * p.n_pages_max;
  const uint32_t tag = (uint32_t)p.epoch;
  // a page's score: the output, and for the selection a word tagged with the
  // launch (device scope)
  const auto put_page = [&](int u, float v) {
    Sb[u] = v;
    if (a.sel)
      __hip_atomic_store(Wb + u, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };
  // every tile's scores first (tiles past this wave's are 0), so the tiles'
  // running sums below are independent chains that interleave
  float sv[kDeltaKeepTiles];
#pragma unroll
  for (int j = 0; j < kDeltaKeepTiles; ++j) {
    float y = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) y = fmaxf(y, keep[j][i] - bl[i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y),
                                                     false, false);
    y = fmaxf(y, __uint_as_float(hl ? sw[0] : sw[1]));
    const int t = tb + (wave + kWaves * j) * 32 + nl;
    sv[j] = j < nt && t < te ? ex2(y) : 0.f;   // tokens past the end add +0
  }
  if (row_pages) {
    float acc[kDeltaKeepTiles];
#pragma unroll
    for (int j = 0; j < kDeltaKeepTiles; ++j) acc[j] = sv[j];
#pragma unroll
    for (int k = 1; k < 16; ++k)
#pragma unroll
      for (int j = 0; j < kDeltaKeepTiles; ++j)
        acc[j] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[j]), 0x111, 0xF,
                                                            0xF, true)) + sv[j];   // row_shr:1
#pragma unroll
    for (int j = 0; j < kDeltaKeepTiles; ++j) {
      const int t = tb + (wave + kWaves * j) * 32 + nl;
      if (j < nt && hl == 0 && (nl & 15) == 15 && t - 15 < te) put_page((t - 15) / 16, acc[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kDeltaKeepTiles; ++j) {
      const int t = tb + (wave + kWaves * j) * 32 + nl;
      if (j < nt && hl == 0 && t < te) ys[t - tb] = sv[j];
    }
  }
  if (!row_pages) {
    __syncthreads();
    const int u0 = tb / p.P, u1 = (te + p.P - 1) / p.P;
    for (int u = u0 + (int)threadIdx.x; u < u1; u += kThreads) {
      const int a0 = u * p.P, a1 = min(a0 + p.P, te);
      float acc = 0.f;
      for (int tt = a0; tt < a1; ++tt) acc += ys[tt - tb];
      put_page(u, acc);
    }
  }
  if (!a.sel) return;
  // The workgroup that finds every page word of its sequence tagged selects
  // the pages, with no waiting: each workgroup reads the words once its own
  // stores have completed, so the last to complete sees all of them (two that
  // complete together both select and write the same row).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (threadIdx.x == 0) sh = 1;
  __syncthreads();
  delta_select(p, b, reinterpret_cast<uint32_t*>(&ring[0][0][0]), ssel, Wb, tag, &sh);
}

template <int D, int NT>
kvs_status delta_launch(const DeltaLaunch& p, hipStream_t stream, int* selected) {
  DeltaArgs a{p, 0};
  *selected = 0;
  if (NT == 1 && p.flags && p.chunk <= 32 * kWaves * kDeltaKeepTiles && p.chunk % p.P == 0 &&
      (int64_t)p.n_chunk * p.B <=
          (int64_t)grid_capacity(reinterpret_cast<const void*>(&delta_fused_kernel<D>), kThreads)) {
    a.p.epoch = grid_epoch();
    a.p.wait_ticks = grid_wait_ticks();
    a.sel = p.pwords && p.n_pages_max <= kThreads * kKpt;
    hipLaunchKernelGGL((delta_fused_kernel<D>), dim3(p.n_chunk, p.B), dim3(kThreads), 0, stream, a);
    *selected = a.sel;
    return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
  }
  hipLaunchKernelGGL((delta_logits_kernel<D, NT>), dim3(p.n_chunk, p.B), dim3(kThreads), 0, stream, a);
  const int n_page_wg = (p.L_max + kDeltaPageTokens - 1) / kDeltaPageTokens;
  hipLaunchKernelGGL(delta_page_kernel, dim3(n_page_wg, p.B), dim3(kDeltaPageTokens), 0, stream, a);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

template <int D>
kvs_status delta_launch_d(const DeltaLaunch& p, hipStream_t stream, int* selected) {
  switch ((p.H_q + 31) / 32) {
    case 1: return delta_launch<D, 1>(p, stream, selected);
    case 2: return delta_launch<D, 2>(p, stream, selected);
    case 3: return delta_launch<D, 3>(p, stream, selected);
    case 4: return delta_launch<D, 4>(p, stream, selected);
    default: return KVS_EUNSUPPORTED;
  }
}

}  // namespace

int delta_chunk(int B, int L_max) {
  const int64_t tiles = (int64_t)B * ((L_max + 31) / 32);
  int64_t tpw = tiles / (256 * kWaves);   // key tiles per wave for one workgroup per CU
  tpw = tpw < 1 ? 1 : tpw > 16 ? 16 : tpw;
  return (int)(32 * kWaves * tpw);
}

kvs_status delta_scores_run(const DeltaLaunch& p, hipStream_t stream, int* selected) {
  if (p.d_k == 128) return delta_launch_d<128>(p, stream, selected);
  if (p.d_k == 64) return delta_launch_d<64>(p, stream, selected);
  return KVS_EUNSUPPORTED;
}

kvs_status score_raw_run(const RawLaunch& p, hipStream_t stream) {
  if (p.d_k == 128) return raw_launch_d<128>(p, stream);
  if (p.d_k == 64) return raw_launch_d<64>(p, stream);
  return KVS_EUNSUPPORTED;
}

kvs_status score_run(const ScorePlan& pl, const ScoreLaunch& p, hipStream_t stream) {
  if (p.d_k == 128) return launch_d<128>(pl, p, stream);
  if (p.d_k == 64) return launch_d<64>(pl, p, stream);
  return KVS_EUNSUPPORTED;
}

}  // namespace kvs

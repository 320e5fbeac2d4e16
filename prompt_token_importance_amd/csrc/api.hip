// C ABI of libkvs: argument validation, workspace sizing and dispatch.
// Every check runs on the host before any kernel is enqueued; no call
// allocates, frees or synchronizes.
#include <math.h>

#include <mutex>

#include "kvs_internal.h"

using namespace kvs;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool mult8(int64_t x) { return (x & 7) == 0; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Fills defaults and validates everything but pointers.
kvs_status check_score(const kvs_score_args* in, kvs_score_args* a) {
  if (!in) return KVS_EINVAL;
  *a = *in;
  if (a->L < 1 || a->W < 1 || a->H_q < 1 || a->H_kv < 1 || a->d_k < 1) return KVS_EINVAL;
  if (a->H_q % a->H_kv) return KVS_EINVAL;
  if (a->q_pos0 < 0) return KVS_EINVAL;
  if (a->heads < KVS_HEADS_NONE || a->heads > KVS_HEADS_ALL_SUM) return KVS_EINVAL;
  if (a->accumulate != 0 && a->accumulate != 1) return KVS_EINVAL;
  if (a->phase < 0 || a->phase > 2) return KVS_EINVAL;
  if (!(a->scale >= 0.f) || isinf(a->scale)) return KVS_EINVAL;
  if (a->L > (1 << 30)) return KVS_EUNSUPPORTED;
  if (a->d_k != 64 && a->d_k != 128) return KVS_EUNSUPPORTED;
  if (a->q_head_stride == 0) a->q_head_stride = (int64_t)a->W * a->d_k;
  if (a->q_row_stride == 0) a->q_row_stride = a->d_k;
  if (a->k_head_stride == 0) a->k_head_stride = (int64_t)a->L * a->d_k;
  if (a->k_tok_stride == 0) a->k_tok_stride = a->d_k;
  if (a->s_ld == 0) a->s_ld = a->L;
  if (a->q_head_stride < 0 || a->q_row_stride < 0 || a->k_head_stride < 0 || a->k_tok_stride < 0)
    return KVS_EINVAL;
  if (!mult8(a->q_head_stride) || !mult8(a->q_row_stride) || !mult8(a->k_head_stride) ||
      !mult8(a->k_tok_stride))
    return KVS_EINVAL;
  if (a->s_ld < a->L) return KVS_EINVAL;
  return KVS_OK;
}

struct DeltaPlan {
  size_t x2, cstats, S, flags, pwords, total;   // byte offsets of the workspace parts
  int chunk, n_chunk, n_pages_max;
  int64_t x2_ld;
};

kvs_status delta_plan(const kvs_delta_args* a, DeltaPlan* pl) {
  if (!a) return KVS_EINVAL;
  if (a->B < 0 || a->H_q < 1 || a->H_kv < 1 || a->d_k < 1 || a->P < 1 || a->L_max < 1)
    return KVS_EINVAL;
  if (a->H_q % a->H_kv) return KVS_EINVAL;
  if (a->L_recent < 0 || a->K_pages < 1 || a->K_pages < a->L_recent) return KVS_EINVAL;
  if (!(a->scale >= 0.f) || isinf(a->scale)) return KVS_EINVAL;
  if (a->k_head_stride < 0 || a->k_tok_stride < 0 || !mult8(a->k_head_stride) ||
      !mult8(a->k_tok_stride))
    return KVS_EINVAL;
  if (a->d_k != 64 && a->d_k != 128) return KVS_EUNSUPPORTED;
  if (a->H_q > 128 || 512 % a->P) return KVS_EUNSUPPORTED;
  const int64_t n_pages = ((int64_t)a->L_max + a->P - 1) / a->P;
  if (n_pages > 16384) return KVS_EUNSUPPORTED;
  pl->chunk = delta_chunk(a->B, a->L_max);
  pl->n_chunk = (a->L_max + pl->chunk - 1) / pl->chunk;
  pl->n_pages_max = (int)n_pages;
  size_t off = 0;
  // rows hold L_max rounded up to 32, then 32 spare columns
  pl->x2_ld = ((int64_t)a->L_max + 31) / 32 * 32 + 32;
  pl->x2 = off;
  off = align_up(off + (size_t)a->B * a->H_q * pl->x2_ld * sizeof(float), kWsAlign);
  pl->cstats = off;
  off = align_up(off + (size_t)a->B * pl->n_chunk * a->H_q * sizeof(float2), kWsAlign);
  pl->S = off;
  off = align_up(off + (size_t)a->B * n_pages * sizeof(float), kWsAlign);
  pl->flags = off;
  off = align_up(off + (size_t)a->B * pl->n_chunk * sizeof(uint64_t), kWsAlign);
  pl->pwords = off;
  off = align_up(off + (size_t)a->B * n_pages * sizeof(uint64_t), kWsAlign);
  pl->total = off;
  return KVS_OK;
}

// ---------------------------------------------------------------- static scratch
// kvs_score_noalloc's workspace: one array of kScratchBytes on every GPU the
// library runs on, held until the process ends.  In host code `scratch` names
// a host-side stand-in, never the device memory: the device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is handed to kernels.
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, or null

// Device address of the scratch array on the device that runs `stream`.
kvs_status scratch_on(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return KVS_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return KVS_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KVS_EHIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return KVS_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return KVS_EHIP;
    if (e != hipSuccess || !p) return KVS_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVS_OK;
}

}  // namespace

extern "C" {

const char* kvs_status_string(kvs_status s) {
  switch (s) {
    case KVS_OK: return "KVS_OK";
    case KVS_EINVAL: return "KVS_EINVAL: invalid argument";
    case KVS_EUNSUPPORTED: return "KVS_EUNSUPPORTED: a valid shape outside what the kernels cover";
    case KVS_EWORKSPACE: return "KVS_EWORKSPACE: workspace too small";
    case KVS_EHIP: return "KVS_EHIP: kernel launch failed";
    case KVS_ESCRATCH:
      return "KVS_ESCRATCH: the call needs more scratch than the library's static buffer holds";
    default: return "KVS: unknown status";
  }
}

int32_t kvs_version(void) { return 100; }

size_t kvs_score_workspace(const kvs_score_args* in) {
  kvs_score_args a;
  if (check_score(in, &a) != KVS_OK) return 0;
  ScorePlan pl;
  if (score_plan(&a, &pl) != KVS_OK) return 0;
  return pl.ws_total;
}

int32_t kvs_wait_limit(int32_t microseconds) { return kvs::wait_limit(microseconds); }

kvs_status kvs_score(const kvs_score_args* in, const void* Q, const void* K, float* S, void* ws,
                     size_t ws_bytes, void* stream) {
  kvs_score_args a;
  kvs_status st = check_score(in, &a);
  if (st != KVS_OK) return st;
  if (!Q || !K || !S) return KVS_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || ((uintptr_t)S & 3u)) return KVS_EINVAL;
  ScorePlan pl;
  st = score_plan(&a, &pl);
  if (st != KVS_OK) return st;
  if (!ws || ws_bytes < pl.ws_total) return KVS_EWORKSPACE;
  if (!aligned16(ws)) return KVS_EINVAL;
  ScoreLaunch p;
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = static_cast<const uint16_t*>(K);
  p.S = S;
  p.stats = static_cast<float2*>(ws);
  p.head_rows_ws = pl.ws_heads ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.ws_stats)
                               : nullptr;
  p.flags = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + pl.ws_stats + pl.ws_heads);
  p.qhs = a.q_head_stride;
  p.qrs = a.q_row_stride;
  p.khs = a.k_head_stride;
  p.kts = a.k_tok_stride;
  p.s_ld = a.s_ld;
  p.q_pos0 = a.q_pos0;
  p.L = a.L;
  p.W = a.W;
  p.G = a.H_q / a.H_kv;
  p.H_kv = a.H_kv;
  p.d_k = a.d_k;
  p.heads = a.heads;
  p.accumulate = a.accumulate;
  p.phase = a.phase;
  const double scale = a.scale > 0.f ? (double)a.scale : 1.0 / sqrt((double)a.d_k);
  p.c = (float)(scale * 1.4426950408889634073599246810018921);  // scale * log2(e)
  return score_run(pl, p, as_stream(stream));
}

kvs_status kvs_score_noalloc(const kvs_score_args* in, const void* Q, const void* K, float* S,
                             void* stream) {
  kvs_score_args a;
  kvs_status st = check_score(in, &a);
  if (st != KVS_OK) return st;
  ScorePlan pl;
  st = score_plan(&a, &pl);
  if (st != KVS_OK) return st;
  if (pl.ws_total > kScratchBytes) return KVS_ESCRATCH;
  void* ws = nullptr;
  st = scratch_on(as_stream(stream), &ws);
  if (st != KVS_OK) return st;
  return kvs_score(in, Q, K, S, ws, kScratchBytes, stream);
}

kvs_status kvs_score_raw(const kvs_raw_args* in, const void* Q, const void* K, float* S,
                         void* stream) {
  if (!in) return KVS_EINVAL;
  kvs_raw_args a = *in;
  if (a.L < 1 || a.W < 1 || a.H_q < 1 || a.H_kv < 1 || a.d_k < 1) return KVS_EINVAL;
  if (a.H_q % a.H_kv) return KVS_EINVAL;
  if (a.reduce != KVS_RED_SUM && a.reduce != KVS_RED_MAX) return KVS_EINVAL;
  if (a.accumulate < KVS_ACC_WRITE || a.accumulate > KVS_ACC_MAX) return KVS_EINVAL;
  if (!(a.scale >= 0.f) || isinf(a.scale)) return KVS_EINVAL;
  if (a.q_pos0 < (int64_t)a.L - 1) return KVS_EUNSUPPORTED;   // rows that see only part of the keys
  if (a.L > (1 << 30)) return KVS_EUNSUPPORTED;
  if (a.d_k != 64 && a.d_k != 128) return KVS_EUNSUPPORTED;
  if (a.W > 32) return KVS_EUNSUPPORTED;
  if (a.q_head_stride == 0) a.q_head_stride = (int64_t)a.W * a.d_k;
  if (a.q_row_stride == 0) a.q_row_stride = a.d_k;
  if (a.k_head_stride == 0) a.k_head_stride = (int64_t)a.L * a.d_k;
  if (a.k_tok_stride == 0) a.k_tok_stride = a.d_k;
  if (a.s_ld == 0) a.s_ld = a.L;
  if (a.q_head_stride < 0 || a.q_row_stride < 0 || a.k_head_stride < 0 || a.k_tok_stride < 0)
    return KVS_EINVAL;
  if (!mult8(a.q_head_stride) || !mult8(a.q_row_stride) || !mult8(a.k_head_stride) ||
      !mult8(a.k_tok_stride))
    return KVS_EINVAL;
  if (a.s_ld < a.L) return KVS_EINVAL;
  const int G = a.H_q / a.H_kv;
  const int hr = a.W <= 8 ? 8 : a.W <= 16 ? 16 : 32;   // a head's rows, padded
  if ((int64_t)G * hr > 128) return KVS_EUNSUPPORTED;
  if (!Q || !K || !S) return KVS_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || ((uintptr_t)S & 3u)) return KVS_EINVAL;
  RawLaunch p;
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = static_cast<const uint16_t*>(K);
  p.S = S;
  p.qhs = a.q_head_stride;
  p.qrs = a.q_row_stride;
  p.khs = a.k_head_stride;
  p.kts = a.k_tok_stride;
  p.s_ld = a.s_ld;
  p.L = a.L;
  p.W = a.W;
  p.G = G;
  p.H_kv = a.H_kv;
  p.d_k = a.d_k;
  p.head_rows = hr;
  p.reduce_max = a.reduce == KVS_RED_MAX;
  p.accumulate = a.accumulate;
  p.scale = a.scale > 0.f ? a.scale : (float)(1.0 / sqrt((double)a.d_k));
  return score_raw_run(p, as_stream(stream));
}

size_t kvs_delta_workspace(const kvs_delta_args* a) {
  DeltaPlan pl;
  return delta_plan(a, &pl) == KVS_OK ? pl.total : 0;
}

kvs_status kvs_delta_pages(const kvs_delta_args* a, const void* Q, const void* const* K,
                           const int32_t* L, int32_t* rho, float* page_scores, void* ws,
                           size_t ws_bytes, void* stream) {
  DeltaPlan pl;
  kvs_status st = delta_plan(a, &pl);
  if (st != KVS_OK) return st;
  if (a->B == 0) return KVS_OK;
  if (!Q || !K || !L || !rho) return KVS_EINVAL;
  if (!aligned16(Q) || ((uintptr_t)K & 7u) || ((uintptr_t)L & 3u) || ((uintptr_t)rho & 3u) ||
      ((uintptr_t)page_scores & 3u))
    return KVS_EINVAL;
  if (!ws || ws_bytes < pl.total) return KVS_EWORKSPACE;
  if (!aligned16(ws)) return KVS_EINVAL;
  uint8_t* w = static_cast<uint8_t*>(ws);
  DeltaLaunch p;
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = reinterpret_cast<const uint16_t* const*>(K);
  p.L = L;
  p.x2 = reinterpret_cast<float*>(w + pl.x2);
  p.cstats = reinterpret_cast<float2*>(w + pl.cstats);
  p.S = page_scores ? page_scores : reinterpret_cast<float*>(w + pl.S);
  p.rho = rho;
  p.flags = reinterpret_cast<uint64_t*>(w + pl.flags);
  p.pwords = reinterpret_cast<uint64_t*>(w + pl.pwords);
  p.epoch = 0;
  p.wait_ticks = 0;
  p.khs = a->k_head_stride;
  p.kts = a->k_tok_stride ? a->k_tok_stride : a->d_k;
  p.B = a->B;
  p.H_q = a->H_q;
  p.H_kv = a->H_kv;
  p.G = a->H_q / a->H_kv;
  p.d_k = a->d_k;
  p.P = a->P;
  p.K_pages = a->K_pages;
  p.L_recent = a->L_recent;
  p.L_max = a->L_max;
  p.chunk = pl.chunk;
  p.x2_ld = pl.x2_ld;
  p.n_chunk = pl.n_chunk;
  p.n_pages_max = pl.n_pages_max;
  const double scale = a->scale > 0.f ? (double)a->scale : 1.0 / sqrt((double)a->d_k);
  p.c = (float)(scale * 1.4426950408889634073599246810018921);  // scale * log2(e)
  hipStream_t s = as_stream(stream);
  int selected = 0;
  st = delta_scores_run(p, s, &selected);
  if (st != KVS_OK) return st;
  return selected ? KVS_OK : delta_topk_run(p, s);
}

kvs_status kvs_gather_kv(const void* K, const void* V, int32_t H, int32_t L, int32_t d_k,
                         int64_t head_stride, int64_t tok_stride, const int32_t* indices,
                         int64_t idx_ld, const int32_t* indptr, int32_t n, int32_t unit,
                         void* K_out, void* V_out, void* stream) {
  if (H < 0 || L < 0 || n < 0 || unit < 1 || idx_ld < 0 || d_k < 8 || d_k % 8 || d_k > 2048)
    return KVS_EINVAL;
  if (head_stride == 0) head_stride = (int64_t)L * d_k;
  if (tok_stride == 0) tok_stride = d_k;
  if (head_stride < 0 || tok_stride < 0 || !mult8(head_stride) || !mult8(tok_stride))
    return KVS_EINVAL;
  if (H == 0 || n == 0) return KVS_OK;
  if (!K || !K_out || !indices || (V && !V_out) || (!V && V_out)) return KVS_EINVAL;
  if (!aligned16(K) || !aligned16(K_out) || (V && (!aligned16(V) || !aligned16(V_out))) ||
      ((uintptr_t)indices & 3u) || ((uintptr_t)indptr & 3u))
    return KVS_EINVAL;
  GatherLaunch p;
  p.K = static_cast<const uint16_t*>(K);
  p.V = static_cast<const uint16_t*>(V);
  p.K_out = static_cast<uint16_t*>(K_out);
  p.V_out = static_cast<uint16_t*>(V_out);
  p.indices = indices;
  p.indptr = indptr;
  p.idx_ld = idx_ld;
  p.khs = head_stride;
  p.kts = tok_stride;
  p.H = H;
  p.L = L;
  p.d_k = d_k;
  p.n = n;
  p.unit = unit;
  return gather_run(p, as_stream(stream));
}

kvs_status kvs_pool_pages(const float* S, int32_t H, int32_t n, int64_t ld, int32_t head_reduce,
                          int32_t pool, int32_t pool_k, int32_t P, int32_t page_reduce,
                          float* pooled, float* page, int32_t* page_arg, void* stream) {
  if (!S || H < 1 || n < 1 || ld < n) return KVS_EINVAL;
  if (head_reduce != KVS_RED_NONE && head_reduce != KVS_RED_SUM && head_reduce != KVS_RED_MAX &&
      head_reduce != KVS_RED_MEAN)
    return KVS_EINVAL;
  if (pool != KVS_RED_NONE && pool != KVS_RED_MAX && pool != KVS_RED_MEAN) return KVS_EINVAL;
  if (pool != KVS_RED_NONE && (pool_k < 1 || (pool_k & 1) == 0)) return KVS_EINVAL;
  if (pool != KVS_RED_NONE && pool_k > 129) return KVS_EUNSUPPORTED;
  if (P < 0) return KVS_EINVAL;
  if (P > 0 && page_reduce != KVS_RED_SUM && page_reduce != KVS_RED_MAX) return KVS_EINVAL;
  if (P > 2048) return KVS_EUNSUPPORTED;
  if (P == 0 && !pooled) return KVS_EINVAL;
  if (P > 0 && !pooled && !page && !page_arg) return KVS_EINVAL;
  if (((uintptr_t)S & 3u) || ((uintptr_t)pooled & 3u) || ((uintptr_t)page & 3u) ||
      ((uintptr_t)page_arg & 3u))
    return KVS_EINVAL;
  return pool_pages_run(S, H, n, ld, head_reduce, pool, pool_k, P, page_reduce, pooled, page,
                        page_arg, as_stream(stream));
}

size_t kvs_topk_workspace(int32_t H, int32_t n, int32_t budget) {
  if (H < 0 || H > 65535 || n < 1 || budget < 0 || budget > n) return 0;
  return topk_ws_bytes(H, n, budget);
}

namespace {
kvs_status check_select(const SelectCall& c, size_t ws_bytes) {
  if (!c.S || !c.idx || c.H < 0 || c.n < 1 || c.ld < c.n) return KVS_EINVAL;
  if (c.H > 65535) return KVS_EUNSUPPORTED;
  if (c.budget < 0 || c.budget > c.n || c.n_forced < 0) return KVS_EINVAL;
  if ((int64_t)c.n + c.n_forced > 0x7fffffff) return KVS_EINVAL;
  if (((uintptr_t)c.S & 3u) || ((uintptr_t)c.idx & 3u)) return KVS_EINVAL;
  if (c.pool != KVS_RED_NONE && c.pool != KVS_RED_MAX && c.pool != KVS_RED_MEAN) return KVS_EINVAL;
  if (c.pool != KVS_RED_NONE && (c.pool_k < 1 || (c.pool_k & 1) == 0)) return KVS_EINVAL;
  if (c.pool != KVS_RED_NONE && (c.pool_k - 1) / 2 > kSelHaloMax) return KVS_EUNSUPPORTED;
  if (c.cluster_P < 0 || c.cluster_r < 0) return KVS_EINVAL;
  if (c.cluster_P > 0 && isnan(c.cluster_theta)) return KVS_EINVAL;
  if (c.cluster_P > 0 && (int64_t)c.cluster_P + c.cluster_r > kSelHaloMax) return KVS_EUNSUPPORTED;
  if (c.cluster_P > 0 && c.pool != KVS_RED_NONE) return KVS_EUNSUPPORTED;
  const size_t need = c.H > 0 ? topk_ws_bytes(c.H, c.n, c.budget) : 0;
  if (need && (!c.ws || ws_bytes < need)) return KVS_EWORKSPACE;
  if (need && !aligned16(c.ws)) return KVS_EINVAL;
  return KVS_OK;
}
}  // namespace

kvs_status kvs_topk(const float* S, int32_t H, int32_t n, int64_t ld, int32_t budget,
                    const uint8_t* priority, int32_t n_forced, int32_t* idx, float* val, void* ws,
                    size_t ws_bytes, void* stream) {
  SelectCall c{S, H, n, ld, budget, n_forced, priority, KVS_RED_NONE, 0, 0, 0.f, 0, idx, ws, val};
  if ((uintptr_t)val & 3u) return KVS_EINVAL;
  const kvs_status st = check_select(c, ws_bytes);
  if (st != KVS_OK) return st;
  return select_run(c, as_stream(stream));
}

size_t kvs_select_workspace(int32_t H, int32_t n, int32_t budget) {
  if (H < 0 || H > 65535 || n < 1 || budget < 0 || budget > n) return 0;
  return topk_ws_bytes(H, n, budget);
}

kvs_status kvs_select(const float* S, int32_t H, int32_t n, int64_t ld, const kvs_select_args* a,
                      int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (!a) return KVS_EINVAL;
  SelectCall c{S,          H,        n,         ld,           a->budget,        a->n_forced,
               nullptr,    a->pool,  a->pool_k, a->cluster_P, a->cluster_theta, a->cluster_r,
               idx,        ws,       nullptr};
  const kvs_status st = check_select(c, ws_bytes);
  if (st != KVS_OK) return st;
  return select_run(c, as_stream(stream));
}

size_t kvs_block_union_workspace(int32_t H_q, int32_t H_kv, int32_t sub_group, int32_t n_kvb) {
  if (H_q < 1 || H_kv < 1 || H_q % H_kv || n_kvb < 1 || sub_group < 0) return 0;
  const int G = H_q / H_kv;
  if (sub_group && G % sub_group) return 0;
  return union_ws_bytes(H_q, H_kv, sub_group, n_kvb);
}

kvs_status kvs_block_union_pagetable(const uint8_t* M, int32_t H_q, int32_t H_kv, int32_t sub_group,
                                     int32_t n_qb, int32_t n_kvb, int32_t* kv_indptr,
                                     int32_t* kv_indices, void* ws, size_t ws_bytes, void* stream) {
  if (!M || !kv_indptr || !kv_indices) return KVS_EINVAL;
  if (H_q < 1 || H_kv < 1 || H_q % H_kv || n_qb < 1 || n_kvb < 1 || sub_group < 0) return KVS_EINVAL;
  const int G = H_q / H_kv;
  if (sub_group && G % sub_group) return KVS_EINVAL;
  if (((uintptr_t)kv_indptr & 3u) || ((uintptr_t)kv_indices & 3u)) return KVS_EINVAL;
  const size_t need = union_ws_bytes(H_q, H_kv, sub_group, n_kvb);
  if (!ws || ws_bytes < need) return KVS_EWORKSPACE;
  if (!aligned16(ws)) return KVS_EINVAL;
  return union_run(M, H_q, H_kv, sub_group, n_qb, n_kvb, kv_indptr, kv_indices, ws,
                   as_stream(stream));
}

size_t kvs_token_pagetable_workspace(int32_t H, int32_t rows_per_group, int32_t n_pages) {
  if (H < 1 || rows_per_group < 1 || H % rows_per_group || n_pages < 1 || n_pages > (1 << 26))
    return 0;
  return token_pagetable_ws_bytes(H, rows_per_group, n_pages);
}

kvs_status kvs_token_pagetable(const int32_t* idx, int32_t H, int32_t n, int64_t idx_ld,
                               int32_t rows_per_group, int32_t P, int32_t n_pages,
                               int32_t* kv_indptr, int32_t* kv_indices, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!kv_indptr || !kv_indices || (n > 0 && !idx)) return KVS_EINVAL;
  if (H < 1 || n < 0 || rows_per_group < 1 || H % rows_per_group || P < 1 || n_pages < 1)
    return KVS_EINVAL;
  if (idx_ld == 0) idx_ld = n;
  if (idx_ld < n) return KVS_EINVAL;
  if ((int64_t)n_pages * P > 0x7fffffff) return KVS_EINVAL;
  if (n_pages > (1 << 26)) return KVS_EUNSUPPORTED;
  if (((uintptr_t)idx & 3u) || ((uintptr_t)kv_indptr & 3u) || ((uintptr_t)kv_indices & 3u))
    return KVS_EINVAL;
  const size_t need = token_pagetable_ws_bytes(H, rows_per_group, n_pages);
  if (!ws || ws_bytes < need) return KVS_EWORKSPACE;
  if (!aligned16(ws)) return KVS_EINVAL;
  return token_pagetable_run(idx, H, n, idx_ld, rows_per_group, P, n_pages, kv_indptr, kv_indices,
                             ws, as_stream(stream));
}

size_t kvs_aggregate_workspace(int32_t n) {
  if (n < 1) return 0;
  return aggregate_ws_bytes(n);
}

kvs_status kvs_aggregate_layers(float* acc, const float* S, int32_t H, int32_t n, int64_t ld,
                                int32_t mode, int32_t first_layer, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!acc || !S || H < 1 || n < 1 || ld < n) return KVS_EINVAL;
  if (mode != KVS_RED_SUM_L1 && mode != KVS_RED_MAX) return KVS_EINVAL;
  if (first_layer != 0 && first_layer != 1) return KVS_EINVAL;
  if (((uintptr_t)acc & 3u) || ((uintptr_t)S & 3u)) return KVS_EINVAL;
  if (mode == KVS_RED_SUM_L1) {
    const size_t need = aggregate_ws_bytes(n);
    if (!ws || ws_bytes < need) return KVS_EWORKSPACE;
    if (((uintptr_t)ws & 7u)) return KVS_EINVAL;
  }
  return aggregate_run(acc, S, H, n, ld, mode, first_layer, ws, as_stream(stream));
}

kvs_status kvs_cluster_priority(const float* page, const int32_t* page_arg, int32_t H,
                                int32_t n_pages, int32_t P, int32_t n, float theta, int32_t r,
                                uint8_t* priority, void* stream) {
  if (!page || !page_arg || !priority) return KVS_EINVAL;
  if (H < 1 || n < 1 || P < 1 || r < 0 || n_pages != (n + P - 1) / P) return KVS_EINVAL;
  if (isnan(theta)) return KVS_EINVAL;
  return cluster_priority_run(page, page_arg, H, n_pages, P, n, theta, r, priority,
                              as_stream(stream));
}

size_t kvs_block_select_workspace(const kvs_block_select_args* a) {
  if (!a || a->Lq < 1 || a->L < 1 || a->block < 1 || a->H_q < 1 || a->H_kv < 1 ||
      a->H_q % a->H_kv || (a->d_k != 64 && a->d_k != 128))
    return 0;
  BlockPlan pl;
  if (block_plan(a, &pl) != KVS_OK) return 0;
  return pl.ws_total;
}

kvs_status kvs_block_select(const kvs_block_select_args* in, const void* Qc, const void* K,
                            uint8_t* M, void* ws, size_t ws_bytes, void* stream) {
  return kvs_block_select_cached(in, Qc, K, nullptr, 0, 0, M, ws, ws_bytes, stream);
}

kvs_status kvs_block_select_cached(const kvs_block_select_args* in, const void* Qc, const void* K,
                                   float* Kb, int32_t kb_cap, int32_t n_cached, uint8_t* M,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!in || !Qc || !K || !M) return KVS_EINVAL;
  kvs_block_select_args a = *in;
  if (a.Lq < 1 || a.L < 1 || a.block < 1 || a.H_q < 1 || a.H_kv < 1 || a.d_k < 1) return KVS_EINVAL;
  if (a.H_q % a.H_kv || a.q_pos0 < 0) return KVS_EINVAL;
  if (a.q_pos0 + a.Lq > a.L) return KVS_EINVAL;  // the chunk's own keys are part of K
  if (!(a.p_mass > 0.f) || a.p_mass > 1.f) return KVS_EINVAL;
  if (!(a.scale >= 0.f) || isinf(a.scale)) return KVS_EINVAL;
  if (a.d_k != 64 && a.d_k != 128) return KVS_EUNSUPPORTED;
  if (a.q_head_stride == 0) a.q_head_stride = (int64_t)a.Lq * a.d_k;
  if (a.q_row_stride == 0) a.q_row_stride = a.d_k;
  if (a.k_head_stride == 0) a.k_head_stride = (int64_t)a.L * a.d_k;
  if (a.k_tok_stride == 0) a.k_tok_stride = a.d_k;
  if (!mult8(a.q_head_stride) || !mult8(a.q_row_stride) || !mult8(a.k_head_stride) ||
      !mult8(a.k_tok_stride) || a.q_head_stride < 0 || a.q_row_stride < 0 || a.k_head_stride < 0 ||
      a.k_tok_stride < 0)
    return KVS_EINVAL;
  if (!aligned16(Qc) || !aligned16(K)) return KVS_EINVAL;
  BlockPlan pl;
  kvs_status st = block_plan(&a, &pl);
  if (st != KVS_OK) return st;
  if (Kb) {
    if (((uintptr_t)Kb & 15u) || kb_cap < pl.n_kvb || n_cached < 0 || n_cached > a.L / a.block)
      return KVS_EINVAL;
  }
  if (!ws || ws_bytes < pl.ws_total) return KVS_EWORKSPACE;
  if (!aligned16(ws)) return KVS_EINVAL;
  return block_select_run(&a, pl, static_cast<const uint16_t*>(Qc),
                          static_cast<const uint16_t*>(K), M, ws, Kb, kb_cap, n_cached,
                          as_stream(stream));
}

}  // extern "C"

// Compaction of the selected tokens, pages or blocks of K and V (kvs_gather_kv).
//
// The CLAA page keeps each layer's KV cache for the indices top-k chose from
// that layer's scores ("Complete flow and cost"); the CompactAttention page
// measures such an explicit copy against its page-table path ("Core method",
// the execution ablation); DELTA reads whole pages ("Key design 3").  One
// kernel serves all three: head g's list comes from a CSR range, a fixed
// stride or one shared list, and each entry selects `unit` consecutive tokens.
//
// HBM-bound copy: each output row (d_k bf16 values) is read and written once
// in 16-byte pieces, consecutive threads on consecutive pieces of a row, so
// every load and store instruction covers whole rows.  Rows whose entry is
// negative, past the list, or whose token lies past L are written as zeros.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kIter = 8;   // rows per thread: a workgroup copies (256 / pieces per row) * 8 rows

__host__ __device__ inline int gather_rows(int d_k) { return kGatherThreads / (d_k / 8) * kIter; }

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherLaunch p) {
  const int g = blockIdx.y;
  const int cpr = p.d_k / 8;                 // 16-byte pieces per row
  const int rows_per_iter = kGatherThreads / cpr;
  const int piece = threadIdx.x % cpr;
  int lo = 0, count = p.n;
  const int32_t* list = p.indices + (int64_t)g * p.idx_ld;
  if (p.indptr) {
    lo = p.indptr[g];
    count = min(p.indptr[g + 1] - lo, p.n);
    list = p.indices + lo;
  }
  const int64_t out_rows = (int64_t)p.n * p.unit;
  // all of this thread's rows are loaded before any is stored, so the loads
  // of a workgroup are in flight together
  uint4 kv[kIter], vv[kIter];
  int64_t dst[kIter];
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int k = threadIdx.x / cpr + it * rows_per_iter;
    const int64_t r = (int64_t)blockIdx.x * rows_per_iter * kIter + k;
    dst[it] = -1;
    kv[it] = vv[it] = zero;
    if (threadIdx.x >= rows_per_iter * cpr || r >= out_rows) continue;
    const int e = (int)(r / p.unit), o = (int)(r % p.unit);
    int64_t t = -1;
    if (e < count) {
      const int i = list[e];
      if (i >= 0) t = (int64_t)i * p.unit + o;
    }
    dst[it] = ((int64_t)g * out_rows + r) * p.d_k + 8 * piece;
    if (t >= 0 && t < p.L) {
      const int64_t src = (int64_t)g * p.khs + t * p.kts + 8 * piece;
      kv[it] = *reinterpret_cast<const uint4*>(p.K + src);
      if (p.V) vv[it] = *reinterpret_cast<const uint4*>(p.V + src);
    }
  }
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    if (dst[it] < 0) continue;
    *reinterpret_cast<uint4*>(p.K_out + dst[it]) = kv[it];
    if (p.V) *reinterpret_cast<uint4*>(p.V_out + dst[it]) = vv[it];
  }
}

}  // namespace

kvs_status gather_run(const GatherLaunch& p, hipStream_t stream) {
  const int64_t out_rows = (int64_t)p.n * p.unit;
  if (out_rows == 0 || p.H == 0) return KVS_OK;
  const int64_t blocks = (out_rows + gather_rows(p.d_k) - 1) / gather_rows(p.d_k);
  if (blocks > 0x7fffffff) return KVS_EUNSUPPORTED;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks, p.H), dim3(kGatherThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

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
constexpr int kGatherRows = 64;   // output rows per workgroup per tensor

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
  for (int k = threadIdx.x / cpr; k < kGatherRows; k += rows_per_iter) {
    const int64_t r = (int64_t)blockIdx.x * kGatherRows + k;
    if (r >= out_rows) break;
    const int e = (int)(r / p.unit), o = (int)(r % p.unit);
    int64_t t = -1;
    if (e < count) {
      const int i = list[e];
      if (i >= 0) t = (int64_t)i * p.unit + o;
    }
    const bool valid = t >= 0 && t < p.L;
    const int64_t src = (int64_t)g * p.khs + (valid ? t : 0) * p.kts + 8 * piece;
    const int64_t dst = ((int64_t)g * out_rows + r) * p.d_k + 8 * piece;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const uint4 kv = valid ? *reinterpret_cast<const uint4*>(p.K + src) : zero;
    *reinterpret_cast<uint4*>(p.K_out + dst) = kv;
    if (p.V) {
      const uint4 vv = valid ? *reinterpret_cast<const uint4*>(p.V + src) : zero;
      *reinterpret_cast<uint4*>(p.V_out + dst) = vv;
    }
  }
}

}  // namespace

kvs_status gather_run(const GatherLaunch& p, hipStream_t stream) {
  const int64_t out_rows = (int64_t)p.n * p.unit;
  if (out_rows == 0 || p.H == 0) return KVS_OK;
  const int64_t blocks = (out_rows + kGatherRows - 1) / kGatherRows;
  if (blocks > 0x7fffffff) return KVS_EUNSUPPORTED;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks, p.H), dim3(kGatherThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_EHIP;
}

}  // namespace kvs

// Grid-wide exchanges inside one launch (the one-launch score, DELTA and
// top-k forms).
//
// A workgroup publishes data for the other workgroups of its group (the
// splits of a KV head, the chunks of a sequence, the parts of a row) and
// later waits for theirs.  Every (group, member) has a 64-bit flag in the
// workspace, and publishing stores the launch's epoch in it: a value no
// earlier launch of the process used, so flags left by earlier launches never
// read as published and the workspace needs no clearing.  Nothing is
// read-modify-written: the members of a group finish together, and updates
// of one shared counter would queue one device-scope round trip behind
// another.  The XCDs' L2 caches are not coherent with each other, so the
// data and the flags travel as device-scope atomic stores and loads, which
// reach the device's point of coherence, and a workgroup stores its flag only
// after its data stores have completed.  The host takes a one-launch form
// only when the whole grid fits on the device at once (grid_capacity); a wait
// is bounded all the same, and a waiter that reaches the bound (the device
// shared with other work) computes the missing members' data itself, which
// every form arranges to come out bit-identical to the owner's.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kvs {
namespace {

// Stores epoch into flag once this workgroup's earlier stores have completed.
__device__ __forceinline__ void publish_flag(uint64_t* flag, uint64_t epoch) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's data is stored
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls the n flags of a group (lane s reads members s, s + 64, ...)
// until all hold epoch or wait_ticks of the 100 MHz clock have passed (0:
// one poll).  Returns in every thread whether all were published.
__device__ __forceinline__ bool wait_flags(const uint64_t* flags, uint64_t epoch, int n,
                                           int64_t wait_ticks, int* sh) {
  if (threadIdx.x < 64) {
    const int64_t t0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    int all;
    for (;;) {
      int ok = 1;
      for (int s = threadIdx.x; s < n; s += 64)
        ok &= __hip_atomic_load(flags + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
      all = __all(ok);
      if (all || (int64_t)__builtin_amdgcn_s_memrealtime() - t0 >= wait_ticks) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (threadIdx.x == 0) *sh = all;
  }
  __syncthreads();
  const int r = __builtin_amdgcn_readfirstlane(*sh);
  __syncthreads();   // before sh is written again
  return r != 0;
}

// Whether flag holds epoch, in every thread of the workgroup.
__device__ __forceinline__ bool flag_set(const uint64_t* flag, uint64_t epoch, int* sh) {
  if (threadIdx.x == 0)
    *sh = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
  __syncthreads();
  const int r = __builtin_amdgcn_readfirstlane(*sh);
  __syncthreads();
  return r != 0;
}

}  // namespace
}  // namespace kvs

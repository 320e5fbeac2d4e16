// Host side of the one-launch forms (grid_sync.h): whether a grid fits on the
// device at once, the launch tags, and the bound on a workgroup's wait.
#include <atomic>
#include <chrono>
#include <mutex>

#include "kvs_internal.h"

namespace kvs {
namespace {

struct FitEntry {
  int dev;
  const void* fn;
  int threads;
  int blocks;   // resident workgroups the device holds, -1: unknown
};

// Bound on a one-launch workgroup's wait, in ticks of the 100 MHz clock; 2 ms.
std::atomic<int64_t> g_wait_ticks{200000};

}  // namespace

// A one-launch form needs every workgroup resident at once (workgroups wait
// for one another), so it is taken only when the occupancy the runtime
// reports for the kernel, times the device's CUs, covers the grid.  The answer
// is kept per device, kernel and workgroup size.
int grid_capacity(const void* fn, int threads) {
  static std::mutex mu;
  static FitEntry table[128];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (table[i].dev == dev && table[i].fn == fn && table[i].threads == threads)
      return table[i].blocks;
  int per_cu = 0, cus = 0;
  int blocks = -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    blocks = per_cu * cus;
  (void)hipGetLastError();
  if (used < 128) table[used++] = FitEntry{dev, fn, threads, blocks};
  return blocks;
}

// A fresh tag for every one-launch call of the process, never 0 (the value of
// a zeroed workspace); the start is drawn from the clock, so flags left in a
// recycled workspace by another process are not mistaken for this call's.
uint64_t grid_epoch() {
  static std::atomic<uint64_t> next{
      ((uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull) >> 8};
  return next.fetch_add(1, std::memory_order_relaxed) | (1ull << 63);
}

int64_t grid_wait_ticks() { return g_wait_ticks.load(std::memory_order_relaxed); }

int32_t wait_limit(int32_t us) {
  const int64_t prev = g_wait_ticks.load(std::memory_order_relaxed);
  if (us >= 0) g_wait_ticks.store((int64_t)us * 100, std::memory_order_relaxed);
  return (int32_t)(prev / 100);
}

}  // namespace kvs

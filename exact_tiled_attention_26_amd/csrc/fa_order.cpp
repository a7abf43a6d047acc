// Host side of the workgroup order (fa_order.h): how many heads go in one
// group, from how many workgroups the device holds at once.
#include <atomic>
#include <mutex>

#include "fa_launch.h"
#include "fa_order.h"

namespace fa {

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxKernels = 64;

// compute units per device, read once per device
int cu_count(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// workgroups of `kern` one CU holds at once (the same on every device of
// one architecture), read once per kernel; a reader that finds the kernel's
// key also sees its value (stored before the key is published)
int per_cu(const void* kern, int threads) {
  static std::atomic<const void*> keys[kMaxKernels];
  static int vals[kMaxKernels];
  static std::mutex insert;
  for (int i = 0; i < kMaxKernels; ++i) {
    const void* k = keys[i].load(std::memory_order_acquire);
    if (k == kern) return vals[i];
    if (k == nullptr) break;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  std::lock_guard<std::mutex> lock(insert);
  for (int i = 0; i < kMaxKernels; ++i) {
    const void* k = keys[i].load(std::memory_order_relaxed);
    if (k == kern) return vals[i];
    if (k == nullptr) {
      vals[i] = n;
      keys[i].store(kern, std::memory_order_release);
      break;
    }
  }
  return n;
}

// workgroups of `kern` the stream's device runs at once
int resident_workgroups(const void* kern, int threads, hipStream_t st) {
  int dev = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess) {
    (void)hipGetLastError();
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  }
  const int n = cu_count(dev) * per_cu(kern, threads);
  return n > 0 ? n : 1;
}

}  // namespace

int head_group(const void* kern, int threads, int bh, int ntiles, hipStream_t st) {
  return head_group_for(bh, ntiles, resident_workgroups(kern, threads, st));
}

}  // namespace fa

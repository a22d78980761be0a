// Per-device properties the launchers need, cached once per device.
#include <hip/hip_runtime.h>

#include <atomic>

#include "fp8vit_internal.h"

namespace fp8vit {

namespace {
constexpr int kMaxCachedDevices = 64;
// Zero means "not queried yet". Relaxed atomics: two threads that both miss
// query the same value and store it twice, which is harmless.
std::atomic<int> g_cus[kMaxCachedDevices];

int query_cus(int dev) {
  int v = 0;
  return hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? v : 0;
}
}  // namespace

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxCachedDevices) return query_cus(dev);
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    n = query_cus(dev);
    if (n > 0) g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fp8vit

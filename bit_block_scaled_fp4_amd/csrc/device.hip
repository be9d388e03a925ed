// Per-device facts the launchers read: the compute-unit count, cached per
// device (a device property, not state that calls share). The library keeps
// no other state and allocates nothing: scratch memory is the caller's
// workspace.
#include <atomic>

#include "fp4_internal.h"

namespace fp4 {
namespace {

constexpr int kMaxDevices = 64;

}  // namespace

int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fp4

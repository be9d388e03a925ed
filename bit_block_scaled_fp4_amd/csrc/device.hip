// Per-device state of the library: compute-unit counts, and the workspaces
// of the kernels that combine partial results across
// workgroups or launches (the small-M product's K-chunk partials, the row
// argmax's segment keys and counters, the prefill product's split-K tiles).
//
// One buffer per (device, purpose), allocated on first need, grown when a
// call needs more and never freed: kernels queued earlier may still use an
// older buffer, which is kept until the process ends. A buffer of counters
// is cleared by a fill kernel on the caller's stream when it is allocated;
// the kernels that use counters leave them at zero when they finish.
#include <atomic>
#include <mutex>

#include "fp4_internal.h"

namespace fp4 {
namespace {

constexpr int kMaxDevices = 64;

struct Buffer {
  void* p = nullptr;
  size_t bytes = 0;
};
std::mutex g_mu;
Buffer g_buf[kMaxDevices][kWsCount];

__global__ __launch_bounds__(256) void k_zero_u32(unsigned* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

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

hipError_t device_workspace(Workspace which, size_t bytes, bool zero_new, hipStream_t s, void** out) {
  if (which < 0 || which >= kWsCount) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  Buffer& b = g_buf[dev][which];
  if (b.bytes < bytes) {
    const size_t grown = (bytes + 255) & ~size_t(255);
    void* p = nullptr;
    e = hipMalloc(&p, grown);
    if (e != hipSuccess) return e;
    if (zero_new) {
      const int64_t n = (int64_t)(grown / 4);
      hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, static_cast<unsigned*>(p), n);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    b.p = p;
    b.bytes = grown;
  }
  *out = b.p;
  return hipSuccess;
}

}  // namespace fp4

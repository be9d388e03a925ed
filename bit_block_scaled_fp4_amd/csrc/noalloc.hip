// fp4_gemv_multi_noalloc: the fused small-M product for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). It is fp4_gemv_multi_ws with the
// workspace taken from a file-scope device array, `scratch`, of fixed size:
// each GPU the library runs on holds its own copy until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address; its address on a device comes from hipGetSymbolAddress, asked
// once per device (with that device current) on the entry point's first
// call there, and only that address reaches kernels. All calls on one GPU
// share the array, so calls that may overlap in time on one GPU race (use
// fp4_gemv_multi_ws with separate workspaces for those). The array starts
// zeroed (static storage), as the workspace contract asks: its header holds
// the arrival counters of the split products, which every call leaves at
// zero, and the rest partial sums that each call writes before it reads them.
#include "../../include/fp4.h"

#include <atomic>
#include <mutex>

#include "fp4_internal.h"

namespace {

constexpr size_t kNoAllocBytes = size_t(16) << 20;   // FP4_NOALLOC_SCRATCH_BYTES in include/fp4.h
static_assert(kNoAllocBytes == FP4_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

__device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_mu;

// The device address of `scratch` on the current device (nullptr on error).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" FP4_API int fp4_gemv_multi_noalloc(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K,
                                      void* stream) {
  if (!projs) return FP4_ERR_NULL;
  if (nproj < 1 || nproj > FP4_MAX_PROJ) return FP4_ERR_SHAPE;
  int64_t Ns[FP4_MAX_PROJ];
  for (int i = 0; i < nproj; ++i) Ns[i] = projs[i].N;
  size_t need = 0;
  if (int st = fp4_workspace_bytes(FP4_OP_GEMV, M, K, Ns, nproj, &need)) return st;
  if (need > kNoAllocBytes) return FP4_ERR_WORKSPACE;   // larger than the fixed scratch
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return FP4_ERR_HIP;
  }
  return fp4_gemv_multi_ws(projs, nproj, x_bf16, M, K, ws, ws ? kNoAllocBytes : 0, stream);
}

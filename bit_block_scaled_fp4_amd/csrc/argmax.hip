// Greedy next-token choice: for each row of fp32 logits, the first index of
// the largest value. The last vector of a decode step times the vocabulary
// matrix gives one logit per vocabulary entry, and greedy decoding takes the
// most likely one (page "1. The big picture", steps 4 and 5).
//
// Order. Each element becomes a 64-bit key: the high word maps the fp32
// value onto unsigned integers in the same order (any NaN above +inf, -0
// equal to +0), the low word is ~index, so among equal values the smaller
// index has the larger key. The answer is the largest key of the row, and
// max is associative and commutative: the result does not depend on how the
// row is split or in which order workgroups finish.
//
// Work split. A row is cut into segments of kSeg elements, one workgroup
// each (16 coalesced loads per thread, one round of loads). With one
// segment the workgroup writes the index. Otherwise every workgroup stores
// its key with a device-coherent store (through this XCD's L2), waits for
// the store to complete and counts itself in on the row's counter; the last
// of the row's S workgroups reads the S keys with device-coherent loads,
// writes the index and puts the counter back to zero. One launch, no
// cache-wide fences.
#include "fp4_internal.h"

namespace fp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kSeg = kThreads * kPerThread;   // elements per workgroup
constexpr int kCntStride = 32;                // one 128-byte line per row counter

__device__ __forceinline__ uint64_t key_of(float v, int n) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u)
    u = 0x7fc00000u;   // every NaN ranks as the largest value
  else if ((u & 0x7fffffffu) == 0)
    u = 0u;            // -0 equals +0
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (uint32_t)n);
}

__device__ __forceinline__ int32_t index_of(uint64_t key) { return (int32_t)(0xffffffffu - (uint32_t)key); }

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest key over the workgroup; the result is valid in thread 0.
__device__ __forceinline__ uint64_t wg_max(uint64_t k, uint64_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) k = umax64(k, __shfl_xor(k, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0)
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) k = umax64(k, red[w]);
  return k;
}

struct ArgmaxArgs {
  const float* y;
  int64_t ldy;
  int32_t* idx;
  uint64_t* keys;   // [M][S] partial keys (S > 1)
  unsigned* cnt;    // [M][kCntStride] arrivals per row (first word), zero between launches (S > 1)
  int32_t N;
  int32_t S;        // segments (workgroups) per row
};

// grid: S * M workgroups, workgroup b = m * S + s; block kThreads.
__global__ __launch_bounds__(kThreads) void k_argmax(const ArgmaxArgs a) {
  __shared__ uint64_t red[kThreads / 64];
  __shared__ int last;
  const int S = a.S;
  const int m = (int)(blockIdx.x / (unsigned)S), s = (int)(blockIdx.x - (unsigned)m * S);
  const float* row = a.y + (int64_t)m * a.ldy;
  const int n0 = s * kSeg + (int)threadIdx.x;
  float v[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int n = n0 + i * kThreads;
    v[i] = n < a.N ? row[n] : 0.0f;
  }
  uint64_t k = 0;   // below the key of every element
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int n = n0 + i * kThreads;
    if (n < a.N) k = umax64(k, key_of(v[i], n));
  }
  k = wg_max(k, red);
  if (S == 1) {
    if (threadIdx.x == 0) a.idx[m] = index_of(k);
    return;
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(a.keys + (int64_t)m * S + s, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the key is visible device-wide
    unsigned* c = a.cnt + (int64_t)m * kCntStride;
    last = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!last) return;
  k = 0;
  for (int t = (int)threadIdx.x; t < S; t += kThreads)
    k = umax64(k, __hip_atomic_load(a.keys + (int64_t)m * S + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  k = wg_max(k, red);
  if (threadIdx.x == 0) {
    a.idx[m] = index_of(k);
    // all S arrivals of this launch are in: back to zero for the next one
    __hip_atomic_store(a.cnt + (int64_t)m * kCntStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_argmax(int32_t* idx, const float* y, int64_t M, int64_t N, int64_t ldy, hipStream_t s) {
  ArgmaxArgs a{};
  a.y = y;
  a.ldy = ldy;
  a.idx = idx;
  a.N = (int32_t)N;
  a.S = (int32_t)((N + kSeg - 1) / kSeg);
  const int64_t wgs = M * a.S;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  if (a.S > 1) {
    // counters on separate lines: the atomics of different rows do not queue on one line
    void *keys = nullptr, *cnt = nullptr;
    hipError_t e = device_workspace(kWsArgmaxKeys, (size_t)wgs * sizeof(uint64_t), false, s, &keys);
    if (e == hipSuccess) e = device_workspace(kWsArgmaxCounters, (size_t)M * kCntStride * 4, true, s, &cnt);
    if (e != hipSuccess) return e;
    a.keys = static_cast<uint64_t*>(keys);
    a.cnt = static_cast<unsigned*>(cnt);
  }
  hipLaunchKernelGGL(k_argmax, dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fp4

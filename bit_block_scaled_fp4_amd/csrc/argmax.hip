// Greedy next-token choice: for each row of fp32 logits, the first index of
// the largest value. The last vector of a decode step times the vocabulary
// matrix gives one logit per vocabulary entry, and greedy decoding takes the
// most likely one (page "1. The big picture", steps 4 and 5).
//
// Order: the (value, index) keys of greedy.h; the answer is a row's largest
// key, whatever the split.
//
// Work split. With a workspace, a row is cut into segments of kSeg
// elements, one workgroup each (16 coalesced loads per thread, one round of
// loads). With one segment the workgroup writes the index. Otherwise every
// workgroup stores its key with a device-coherent store (through this XCD's
// L2), waits for the store to complete and counts itself in on the row's
// counter in the workspace header; the last of the row's S workgroups reads
// the S keys with device-coherent loads, writes the index and puts the
// counter back to zero. One launch per 512 rows (the header's counters), no
// cache-wide fences. Without a workspace one workgroup reads each whole row
// in rounds of kSeg elements.
#include <algorithm>

#include "greedy.h"

namespace fp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kSeg = kThreads * kPerThread;   // elements per workgroup round

struct ArgmaxArgs {
  const float* y;
  int64_t ldy;
  int32_t* idx;
  uint64_t* keys;   // [rows][S] partial keys (S > 1)
  unsigned* cnt;    // per row of the launch, kWsCounterWords apart (S > 1)
  int32_t N;
  int32_t S;        // segments (workgroups) per row
  int32_t seg;      // elements per segment (a multiple of kSeg)
};

// grid: S * rows workgroups, workgroup b = m * S + s; block kThreads.
__global__ __launch_bounds__(kThreads) void k_argmax(const ArgmaxArgs a) {
  __shared__ uint64_t red[kThreads / 64];
  __shared__ int last;
  const int S = a.S;
  const int m = (int)(blockIdx.x / (unsigned)S), s = (int)(blockIdx.x - (unsigned)m * S);
  const float* row = a.y + (int64_t)m * a.ldy;
  const int end = min(a.N, (s + 1) * a.seg);
  uint64_t k = 0;   // below the key of every element
  for (int n0 = s * a.seg + (int)threadIdx.x; n0 - (int)threadIdx.x < end; n0 += kSeg) {
    float v[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int n = n0 + i * kThreads;
      v[i] = n < end ? row[n] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int n = n0 + i * kThreads;
      if (n < end) k = umax64(k, greedy_key(v[i], n));
    }
  }
  k = block_max64(k, red);
  if (S == 1) {
    if (threadIdx.x == 0) a.idx[m] = greedy_index(k);
    return;
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(a.keys + (int64_t)m * S + s, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the key is visible device-wide
    unsigned* c = a.cnt + (int64_t)m * kWsCounterWords;
    last = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!last) return;
  k = 0;
  for (int t = (int)threadIdx.x; t < S; t += kThreads)
    k = umax64(k, __hip_atomic_load(a.keys + (int64_t)m * S + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  k = block_max64(k, red);
  if (threadIdx.x == 0) {
    a.idx[m] = greedy_index(k);
    // all S arrivals of this launch are in: back to zero for the next one
    __hip_atomic_store(a.cnt + (int64_t)m * kWsCounterWords, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

int64_t segments(int64_t N) { return (N + kSeg - 1) / kSeg; }

}  // namespace

size_t argmax_ws_bytes(int64_t M, int64_t N) {
  const int64_t S = segments(N);
  if (S <= 1) return 0;
  return kWsHeaderBytes + (size_t)(std::min<int64_t>(M, kWsCounters) * S) * 8;
}

hipError_t launch_argmax(int32_t* idx, const float* y, int64_t M, int64_t N, int64_t ldy, const Workspace& ws,
                         hipStream_t s) {
  ArgmaxArgs a{};
  a.ldy = ldy;
  a.N = (int32_t)N;
  const bool split = ws.valid() && segments(N) > 1;
  a.S = split ? (int32_t)segments(N) : 1;
  a.seg = split ? kSeg : (int32_t)(segments(N) * kSeg);
  const int64_t rows_per_launch = split ? kWsCounters : M;
  if (split) {
    a.keys = reinterpret_cast<uint64_t*>(ws.scratch());
    a.cnt = ws.counter(0);
  }
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_launch) {
    const int64_t rows = std::min(rows_per_launch, M - r0);
    const int64_t wgs = rows * a.S;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    a.y = y + r0 * ldy;
    a.idx = idx + r0;
    hipLaunchKernelGGL(k_argmax, dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp4

// Greedy next-token choice, device side: the order of (value, index) keys
// and the combine of per-workgroup results through a caller's workspace.
//
// The last vector of a decode step times the vocabulary matrix gives one
// logit per vocabulary entry; greedy decoding takes the most likely (page
// "1. The big picture", steps 4 and 5). Here: the first index of the largest
// value, a NaN ranking above every number, -0 equal to +0.
//
// Each value becomes a 64-bit key: the high word maps the fp32 value onto
// unsigned integers in the same order (every NaN as one value above +inf,
// -0 folded onto +0), the low word is the complement of the index, so of two
// equal values the smaller index has the larger key. Every key is nonzero
// (the smallest high word, that of -inf, is 0x007FFFFF), so 0 can stand for
// "no element". The answer is the largest key; max is associative and
// commutative, so the result does not depend on how the work is split or in
// which order workgroups finish.
#pragma once

#include "fp4_internal.h"

namespace fp4 {

__device__ __forceinline__ uint64_t greedy_key(float v, int n) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u)
    u = 0x7fc00000u;   // every NaN ranks as the largest value
  else if ((u & 0x7fffffffu) == 0)
    u = 0u;            // -0 equals +0
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (uint32_t)n);
}

__device__ __forceinline__ int32_t greedy_index(uint64_t key) { return (int32_t)(0xffffffffu - (uint32_t)key); }

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max64(uint64_t k) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) k = umax64(k, __shfl_xor(k, d));
  return k;
}

// Largest key over the workgroup, valid in thread 0. `red` is LDS of at
// least blockDim.x / 64 entries; every thread of the workgroup must call.
__device__ __forceinline__ uint64_t block_max64(uint64_t k, uint64_t* red) {
  const int nw = blockDim.x >> 6;
  k = wave_max64(k);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < nw; ++w) k = umax64(k, red[w]);
  return k;
}

// End of a product launch with the greedy epilogue (GreedyArgs). Called by
// every thread of the workgroup, in uniform control flow, after the
// workgroup's outputs are written; k[m] is the thread's largest key of row m
// (0 where it wrote none), m < M <= NR. `red` is LDS of 16 * NR entries.
//
// Every workgroup stores its largest key per row (never 0: each workgroup
// writes at least one output of every row) into its slot of the zeroed key
// array and is done: no counters, nothing to wait for. The workgroup with the
// last index then reads the M x S slots until none is 0, takes each row's
// largest key, writes idx and zeroes the slots for the next launch. Only that
// one workgroup waits, after its own work, so the others always find a free
// slot to run in whatever the dispatch order; the wait is bounded (about a
// second): a timeout writes idx = -1 and leaves the slots as they are (the
// workspace must then be zeroed again).
constexpr int kGreedyMaxPolls = 1 << 18;

template <int NR>
__device__ void greedy_finish(const GreedyArgs& g, const uint64_t (&k)[NR], int M, uint64_t* red, int* flag) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const int wg = blockIdx.x, S = g.S;
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const uint64_t v = wave_max64(k[m]);
    if (lane == 0) red[wave * NR + m] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    uint64_t v = 0;
    for (int w = 0; w < nw; ++w) v = umax64(v, red[w * NR + threadIdx.x]);
    __hip_atomic_store(g.keys + (int64_t)threadIdx.x * S + wg, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (wg != S - 1) return;
  // J keys per row and thread in one round of loads, NR * J = 8. MI355X,
  // LM head 151936 x 1024 at M = 1 (4748 slots), over the plain product:
  // +3.2-3.3 us with 8 keys a thread and round, +3.7-3.8 with 16, +3.4-3.7
  // with 4, +4.5-4.6 with 2, +7.2-7.3 with 24 (97 VGPRs: fewer waves for
  // the product itself).
  constexpr int J = NR >= 8 ? 1 : 8 / NR;
  uint64_t acc[NR];
  int poll = 0;
  for (;; ++poll) {
    int missing = 0;
#pragma unroll
    for (int m = 0; m < NR; ++m) acc[m] = 0;
    for (int base = 0; base < S; base += J * (int)blockDim.x) {
      uint64_t v[NR][J];
#pragma unroll
      for (int m = 0; m < NR; ++m)
#pragma unroll
        for (int u = 0; u < J; ++u) {
          const int t = base + u * (int)blockDim.x + (int)threadIdx.x;
          v[m][u] = (m < M && t < S)
                        ? __hip_atomic_load(g.keys + (int64_t)m * S + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 1;   // outside the array: counts as present
        }
#pragma unroll
      for (int m = 0; m < NR; ++m)
#pragma unroll
        for (int u = 0; u < J; ++u) {
          missing |= v[m][u] == 0;
          acc[m] = umax64(acc[m], v[m][u]);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) *flag = 0;
    __syncthreads();
    if (missing) *flag = 1;
    __syncthreads();
    if (!*flag || poll == kGreedyMaxPolls) break;
    __builtin_amdgcn_s_sleep(8);
  }
  const bool timed_out = *flag != 0;
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const uint64_t v = wave_max64(acc[m]);
    if (lane == 0) red[wave * NR + m] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    uint64_t v = 0;
    for (int w = 0; w < nw; ++w) v = umax64(v, red[w * NR + threadIdx.x]);
    g.idx[threadIdx.x] = timed_out ? -1 : greedy_index(v);
  }
  if (timed_out) return;
  for (int i = (int)threadIdx.x; i < M * S; i += (int)blockDim.x)
    __hip_atomic_store(g.keys + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace fp4

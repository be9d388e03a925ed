// Streaming-read ceiling probe (measurement aid, not part of the product
// path): reads a device buffer once with 16-byte buffer loads and no
// arithmetic beyond folding the words, so its time is what a kernel that
// only streams the same bytes in the same launch shape can reach. The decode
// kernels are judged against it next to the HBM peak: decode speed is bounded
// by bandwidth over bytes read, and real engines reach only part of that
// ceiling (page "1. The big picture", "The most important number in this
// book").
//
// A wave moves one kilobyte per load instruction (64 lanes x 16 bytes) and
// keeps `unroll` of them in flight. Two orders:
//   mode 0: the 1 KB blocks go round-robin over all waves of the grid;
//   mode 1: each wave streams one contiguous range of blocks.
// Loads past `bytes` read zero without touching memory (buffer bounds). The
// folded value is stored only when it equals a constant no buffer the
// benchmark passes holds everywhere, so the loads cannot be dropped and
// nothing is written in practice.
#include "../../include/fp4_bench.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kNever = 0x9E3779B9u;

template <int U, int AUX>
__global__ __launch_bounds__(1024) void k_stream_read(const uint8_t* buf, uint32_t bytes, int mode,
                                                      uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0,
                                                                     (int)bytes, kRsrcWord3);
  const int lane = threadIdx.x & 63;
  const int waves = blockDim.x >> 6;
  const uint32_t gw = blockIdx.x * (uint32_t)waves + (threadIdx.x >> 6);
  const uint32_t T = gridDim.x * (uint32_t)waves;
  const uint32_t nblk = (bytes + 1023) >> 10;
  uint32_t acc = 0;
  if (mode == 0) {
    for (uint32_t b = gw; b < nblk; b += U * T) {
      u32x4_t v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const uint32_t blk = b + j * T < nblk ? b + j * T : nblk;   // past the end: reads zero
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (blk << 10) + lane * 16, 0, AUX);
      }
#pragma unroll
      for (int j = 0; j < U; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
  } else {
    const uint32_t b0 = (uint32_t)((uint64_t)gw * nblk / T), b1 = (uint32_t)((uint64_t)(gw + 1) * nblk / T);
    for (uint32_t b = b0; b < b1; b += U) {
      u32x4_t v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const uint32_t blk = b + j < b1 ? b + j : nblk;   // past the range: past the buffer, reads zero
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (blk << 10) + lane * 16, 0, AUX);
      }
#pragma unroll
      for (int j = 0; j < U; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
  }
  if (acc == kNever) sink[gw] = acc;
}

template <int AUX>
hipError_t launch_aux(const uint8_t* buf, uint32_t bytes, int wgs, int waves, int unroll, int mode, uint32_t* sink,
                      hipStream_t s) {
  const dim3 g((unsigned)wgs), b((unsigned)(64 * waves));
  switch (unroll) {
    case 1: hipLaunchKernelGGL((k_stream_read<1, AUX>), g, b, 0, s, buf, bytes, mode, sink); break;
    case 2: hipLaunchKernelGGL((k_stream_read<2, AUX>), g, b, 0, s, buf, bytes, mode, sink); break;
    case 4: hipLaunchKernelGGL((k_stream_read<4, AUX>), g, b, 0, s, buf, bytes, mode, sink); break;
    case 8: hipLaunchKernelGGL((k_stream_read<8, AUX>), g, b, 0, s, buf, bytes, mode, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int fp4_bench_stream_read(const void* buf, size_t bytes, int workgroups, int waves, int unroll, int mode,
                                     int nontemporal, uint32_t* sink, void* stream) {
  if (!buf || !sink) return -1;
  if (bytes == 0 || bytes % 1024 != 0 || bytes >= (size_t(1) << 31)) return -2;
  if (workgroups < 1 || workgroups > (1 << 20) || waves < 1 || waves > 16 || (mode != 0 && mode != 1)) return -2;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return -3;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = nontemporal ? launch_aux<2>(static_cast<const uint8_t*>(buf), (uint32_t)bytes, workgroups, waves,
                                                   unroll, mode, sink, s)
                                   : launch_aux<0>(static_cast<const uint8_t*>(buf), (uint32_t)bytes, workgroups, waves,
                                                   unroll, mode, sink, s);
  return e == hipSuccess ? 0 : (e == hipErrorInvalidValue ? -2 : -5);
}

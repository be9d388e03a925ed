// The steps on either side of the decode product, as separate kernels for
// the activation rows whose products run on the matrix cores (the
// vector-ALU product does both inside its own launch, gemv.hip).
//
// A decode layer runs attention and then the MLP on the residual stream
// (page "1. The big picture", step 3). For the Qwen3 family the pages use as
// their example, the MLP is gated, h = silu(gate(x)) * up(x) feeding the
// down projection, and attention's Q, K and V products read the RMS-normalised
// stream x * rsqrt(mean(x^2) + eps) * gain. Both results are bf16, the
// activation type of the next product.
#include <algorithm>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One workgroup per row: the sum of squares in fp32, then each element
// times 1 / sqrt(mean + eps) times its gain, rounded once to bf16.
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* x, const uint16_t* gain, float eps, int K,
                                                 uint16_t* out) {
  __shared__ float red[4];
  __shared__ float rinv;
  const int64_t row = blockIdx.x;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + row * K, K * 2);
  const __amdgpu_buffer_rsrc_t rg = rsrc(gain, K * 2);
  float ss = 0.0f;
  for (int u = threadIdx.x; u < K / 8; u += 256) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, u * 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ss = fmaf(lo(v[i]), lo(v[i]), ss);
      ss = fmaf(hi(v[i]), hi(v[i]), ss);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) rinv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)K + eps);
  __syncthreads();
  const float r = rinv;
  for (int u = threadIdx.x; u < K / 8; u += 256) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, u * 16, 0, 0);
    const u32x4_t g = __builtin_amdgcn_raw_buffer_load_b128(rg, u * 16, 0, 0);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)bf16_rne(lo(v[i]) * r * lo(g[i])) | ((uint32_t)bf16_rne(hi(v[i]) * r * hi(g[i])) << 16);
    *reinterpret_cast<u32x4_t*>(out + row * K + (int64_t)u * 8) = o;
  }
}

// h[m][n] = bf16(silu(g[m][n]) * u[m][n]), silu(z) = z / (1 + e^-z).
__global__ __launch_bounds__(256) void k_swiglu(const float* g, const float* u, int64_t M, int64_t N, uint16_t* h,
                                                int64_t ldh) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / N, n = i - m * N;
    const float z = g[i];
    h[m * ldh + n] = bf16_rne(z / (1.0f + __expf(-z)) * u[i]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t K, uint16_t* out,
                          hipStream_t s) {
  if (M < 1 || M > INT32_MAX || K % 16 != 0 || K * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)M), dim3(256), 0, s, x, gain, eps, (int)K, out);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* g, const float* u, int64_t M, int64_t N, uint16_t* h, int64_t ldh,
                         hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((M * N + 255) / 256, 4096);
  hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, g, u, M, N, h, ldh);
  return hipGetLastError();
}

}  // namespace fp4

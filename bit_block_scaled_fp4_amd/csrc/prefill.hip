// NVFP4 weights x bf16 activations for prefill-sized M on the matrix cores.
//
// Prefill pushes hundreds or thousands of prompt tokens through each layer
// at once, so the product is a real dense contraction and compute-bound
// (page "imp" README, the prefill paragraph; page "1. The big picture",
// "Two phases with very different costs"). Here it runs on gfx950 bf16 MFMA:
// each workgroup decodes its weight tile into LDS as bf16 values
// E2M1 * E4M3 (at most 6 significant bits, inside bf16 range, so exact),
// stages the activation tile in LDS, and accumulates in fp32. The tensor
// scale multiplies the fp32 result once in the epilogue.
//
// Tile: 128 activation rows x 128 weight rows per 256-thread workgroup,
// K in steps of 64; wave (wm, wn) of the 2x2 wave grid owns a 64x64 block
// made of 2x2 v_mfma_f32_32x32x16_bf16 tiles.
#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA = BK + 8;   // bf16 elements per LDS row (16 B pad against bank conflicts)

__device__ __forceinline__ f32x2_t fp4x2_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // one v_cvt_pk_bf16_f32; exact: both values have <= 6 significant bits
  // and lie in bf16 range
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__global__ __launch_bounds__(256) void k_prefill(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                 const uint8_t* __restrict__ tiles,
                                                 const float* __restrict__ gscale, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int C = (K + kChunkK - 1) / kChunkK;
  const int G = (N + 7) >> 3;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // ---- activations: 128 rows x 64 bf16 = 1024 pieces of 16 B, 4 per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * 256, row = idx >> 3, col = (idx & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + row < M && k0 + col < K)
        v = *reinterpret_cast<const uint4*>(x + (int64_t)(m0 + row) * K + k0 + col);
      *reinterpret_cast<uint4*>(&As[row * LDA + col]) = v;
    }
    // ---- weights: 128 rows x 64 elements; thread -> (row, 32-element half)
    {
      const int row = tid >> 1, piece = tid & 1;
      const int n = n0 + row, g = n >> 3, r = n & 7;
      const int c = k0 / kChunkK, l = (k0 % kChunkK) / 32 + piece;
      uint32_t out[16];
      if (g < G && k0 + piece * 32 < K) {
        const uint8_t* tile = tiles + ((int64_t)g * C + c) * kTileBytes;
        const uint4 w = *reinterpret_cast<const uint4*>(tile + r * 512 + l * 16);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(tile + tile_scale_offset(r, 2 * l));
        const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
        const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const f32x2_t e = fp4x2_f32(word(w, i >> 2), i & 3);
          const float s = i < 8 ? s0 : s1;
          out[i] = pack_bf16(e[0] * s, e[1] * s);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = 0;
      }
      uint4* dst = reinterpret_cast<uint4*>(&Bs[row * LDA + piece * 32]);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kof = kk * 16 + (lane >> 5) * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + i * 32 + (lane & 31)) * LDA + kof]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(wn * 64 + j * 32 + (lane & 31)) * LDA + kof]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  const float gs = *gscale;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (m < M && n < N) y[(int64_t)m * N + n] = gs * acc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_prefill(float* y, const uint16_t* x, const uint8_t* tiles, const float* gscale, int64_t M,
                          int64_t N, int64_t K, hipStream_t s) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (grid.y > 65535u) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefill, grid, dim3(256), 0, s, y, x, tiles, gscale, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace fp4

// MXFP4 x MXFP4 product on gfx950's block-scaled FP4 matrix cores.
//
// The imp README's feature table names MXFP4 beside NVFP4 (quantisation row)
// and a block-scaled matrix multiply (engine row). Here both operands are
// MXFP4: the activation rows, quantised by the weights' own MXFP4 rule
// (fp4_quantize_mx, row-major), and the weights in the MX tiled layout. One
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 multiplies a
// 32 x 64 activation block by a 64 x 32 weight block, each lane supplying
// the E8M0 scale of its own 32 elements, at the FP4 rate (10.1 PF/s dense on
// MI355X, four times bf16). Every product of two scaled E2M1 values is
// exact; the sums are fp32.
//
// Operand layouts (checked on MI355X with random operands against a CPU
// product): A lane l holds row l % 32, K elements 32 (l / 32) .. +31 as 16
// bytes (element 2j in the low nibble of byte j), its scale in the low byte
// of the scale operand; B lane l likewise holds column l % 32; result lane
// l holds column l % 32, rows (i % 4) + 8 (i / 4) + 4 (l / 32), i < 16.
//
// Tiling. A 256-thread workgroup computes 256 rows x 128 columns; its four
// waves form a 2 x 2 grid of 128 x 64 (4 x 2 result blocks each). K
// advances 128 per step (two MFMA steps). Each step's operands are loaded
// into registers one step ahead and written to one of two LDS stages: per
// row 64 code bytes (4 chunks of 16) and the 4 scale bytes of the step. A
// row's chunk j sits in slot j ^ ((row / 4) % 4), which keeps the 16-byte
// operand reads and the writes of a half-wave in distinct bank groups
// (rows r and r + 16 in the same group). One barrier per step.
//
// Bounds: K is a multiple of 128 (the launcher checks); activation rows
// past M and weight row groups past N read zeros (buffer loads past the
// resource; the tiled layout pads a ragged last group with zero codes), and
// the stores skip rows past M and columns past N.
#include <algorithm>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kBM = 256, kBN = 128, kKS = 128;
constexpr int kACodes = kBM * 64;              // one stage: 64 code bytes per row
constexpr int kAScales = kBM * 4;              // 4 scale bytes per row
constexpr int kBCodes = kBN * 64;
constexpr int kBScales = (kBN / 8) * 2 * 16;   // 16 row groups x 2 row parities x 16 bytes
constexpr int kStage = kACodes + kAScales + kBCodes + kBScales;

struct A4Args {
  const uint8_t* xa;   // activation codes [M][K/2]
  const uint8_t* xs;   // activation scales [M][K/32]
  const uint8_t* w;    // MX tiled weights, G * C tiles of kMxTileBytes
  float* y;            // [M][ldy]
  int M, N, K, G, C;
  int64_t ldy;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// slot of 16-byte chunk j of LDS row r
__device__ __forceinline__ int slot(int r, int j) { return (j ^ ((r >> 2) & 3)) << 4; }

__global__ __launch_bounds__(256) void k_mx_a4(const A4Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
  const int K = a.K, Kh = K >> 1, Ks = K >> 5;
  const int rows = min(kBM, a.M - m0);
  const __amdgpu_buffer_rsrc_t ra = rsrc(a.xa + (int64_t)m0 * Kh, (uint32_t)rows * Kh);
  const __amdgpu_buffer_rsrc_t rs = rsrc(a.xs + (int64_t)m0 * Ks, (uint32_t)rows * Ks);
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, (uint32_t)a.G * a.C * kMxTileBytes);

  // Loads of one step into registers, all unconditional: a row group past N
  // (or a lane without a scale chunk) takes an offset past the resource
  // instead of a branch, so the loads stay in flight through the step's
  // arithmetic. K is a multiple of the step. Thread t: activation row t
  // (four code chunks, the step's four scale bytes as one word); weight row
  // n = t % 128, code chunks 2 (t / 128) and 2 (t / 128) + 1; threads t <
  // 32: the scale chunk of row group t / 2, row parity t % 2.
  constexpr int kOut = 0x7ffffff0;   // past every resource (the launcher keeps them below 2^31 bytes)
  uint4 pa[4], pb[2], ps;
  uint32_t pas;
  const int bn = t & 127, bg = (n0 + bn) >> 3, br = (n0 + bn) & 7, bv0 = 2 * (t >> 7);
  const bool bvalid = bg < a.G;
  const int sg = (n0 >> 3) + (t >> 1), sh = t & 1;
  const bool svalid = t < 32 && sg < a.G;
  auto load = [&](int s) {
    const int k0 = s * kKS;
#pragma unroll
    for (int u = 0; u < 4; ++u) pa[u] = ld16(ra, t * Kh + ((k0 + 32 * u) >> 1));
    pas = __builtin_amdgcn_raw_buffer_load_b32(rs, t * Ks + (k0 >> 5), 0, 0);
    const int c = k0 >> 10, p0 = (k0 & 1023) >> 5;
    const int tile = (bg * a.C + c) * kMxTileBytes;
#pragma unroll
    for (int v = 0; v < 2; ++v)
      pb[v] = ld16(rw, bvalid ? tile + (br >> 1) * 1024 + (br & 1) * 512 + (p0 + bv0 + v) * 16 : kOut);
    ps = ld16(rw, svalid ? (sg * a.C + c) * kMxTileBytes + 4096 + sh * 128 + p0 * 4 : kOut);
  };
  auto store = [&](int st) {
    uint8_t* s = lds + st * kStage;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(s + t * 64 + slot(t, u)) = pa[u];
    *reinterpret_cast<uint32_t*>(s + kACodes + t * 4) = pas;
#pragma unroll
    for (int v = 0; v < 2; ++v)
      *reinterpret_cast<uint4*>(s + kACodes + kAScales + bn * 64 + slot(bn, bv0 + v)) = pb[v];
    if (t < 32) *reinterpret_cast<uint4*>(s + kACodes + kAScales + kBCodes + t * 16) = ps;
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int r32 = lane & 31, kb = lane >> 5;
  auto compute = [&](int st) {
    const uint8_t* s = lds + st * kStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int j = 2 * ks + kb;   // this lane's 32-element block of the step
      i32x8_t av[4], bv[2];
      int as[4], bs[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = 128 * wm + 32 * mt + r32;
        const uint4 v = *reinterpret_cast<const uint4*>(s + row * 64 + slot(row, j));
        av[mt] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        as[mt] = s[kACodes + row * 4 + j];
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = 64 * wn + 32 * nt + r32;
        const uint4 v = *reinterpret_cast<const uint4*>(s + kACodes + kAScales + n * 64 + slot(n, j));
        bv[nt] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        bs[nt] = s[kACodes + kAScales + kBCodes + ((n >> 3) * 2 + (n & 1)) * 16 + j * 4 + ((n & 7) >> 1)];
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[mt], bv[nt], acc[mt][nt], 4, 4, 0, as[mt], 0,
                                                                          bs[nt]);
    }
  };

  const int nsteps = (K + kKS - 1) / kKS;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) load(s + 1);
    // the next step's loads stay in flight through this step's arithmetic
    __builtin_amdgcn_sched_barrier(0);
    compute(s & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (more) store((s + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = n0 + 64 * wn + 32 * nt + r32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + 128 * wm + 32 * mt + (i & 3) + 8 * (i >> 2) + 4 * kb;
        if (row < a.M && col < a.N) a.y[(int64_t)row * a.ldy + col] = acc[mt][nt][i];
      }
    }
}

}  // namespace

hipError_t launch_mx_a4(float* y, const uint8_t* xq_codes, const uint8_t* xq_scales, const uint8_t* w_tiles, int64_t M,
                        int64_t N, int64_t K, hipStream_t s) {
  A4Args a{};
  a.xa = xq_codes;
  a.xs = xq_scales;
  a.w = w_tiles;
  a.y = y;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)((N + 7) / 8);
  a.C = (int)chunks_of(K);
  a.ldy = N;
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM)), block(256);
  hipLaunchKernelGGL(k_mx_a4, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace fp4

// MXFP4 x MXFP4 product on gfx950's block-scaled FP4 matrix cores.
//
// The imp README's feature table names MXFP4 beside NVFP4 (quantisation row)
// and a block-scaled matrix multiply (engine row). Here both operands are
// MXFP4: the activation rows, quantised by the weights' own MXFP4 rule
// (fp4_quantize_mx, activation layout: row-major codes, scales grouped by
// 128-column step), and the weights in the MX tiled layout. One
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
// Tiling. A 512-thread workgroup (one per CU: 136 KB of LDS) computes 256
// rows x 256 columns; its eight waves form a 2 x 4 grid of 128 x 64 (4 x 2
// result blocks each). K advances 256 per step (four MFMA steps). Every
// global read is a direct-to-LDS buffer load into one of two stages, issued
// one step ahead: per stage 256 activation and 256 weight rows of 128 code
// bytes (8 chunks of 16, a whole 128-byte line per row, so each load
// request moves a full line), the activations' 8 scale bytes per row (two
// contiguous runs in the activation layout) and the weight groups' 32-byte
// scale runs. A row's chunk j sits in slot j ^ ((row / 2) % 8): the MFMA
// operand reads (lane -> row lane % 32) then give 16 consecutive rows 16
// distinct 16-byte bank groups of the 256-byte bank window (rows r and r + 1
// fall in opposite halves). Each wave issues the same ten loads per step.
// The fragments of the next quarter step are read from LDS while the
// current quarter's MFMAs run. The grid is persistent (one workgroup per
// CU, tiles in row-major order, strided by the grid): a tile's last step
// loads the next tile's first, and its fp32 results go out as streaming
// stores.
//
// Bounds: K is a multiple of 128 (the launcher checks; a last half step adds
// exact zeros); activation rows
// past M and weight row groups past N read zeros (offsets past the
// resource; the tiled layout pads a ragged last group with zero codes), and
// the stores skip rows past M and columns past N.
#include <algorithm>
#include <atomic>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kBM = 256, kBN = 256, kKS = 256, kWaves = 8;
constexpr int kACodes = kBM * 128;             // one stage: 128 code bytes per row
constexpr int kAScales = kBM * 8;              // 8 scale bytes per row
constexpr int kBCodes = kBN * 128;
constexpr int kBScales = (kBN / 8) * 2 * 32;   // 32 row groups x 2 row parities x 32 bytes

struct A4Args {
  const uint8_t* xa;   // activation codes [M][K/2]
  const uint8_t* xs;   // activation scales [K/128][M][4]
  const uint8_t* w;    // MX tiled weights, G * C tiles of kMxTileBytes
  float* y;            // [M][ldy]
  int M, N, K, G, C;
  int gx, gy;          // column and row tiles
  int64_t ldy;
};

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// slot of 16-byte chunk j of LDS row r
__device__ __forceinline__ int slot(int r, int j) { return (j ^ ((r >> 1) & 7)) << 4; }

// Buffer resource as four scalars (base, num_records, raw 32-bit format):
// num_records bytes are readable, anything past them reads as zero.
__device__ __forceinline__ i32x4_t rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffff));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kRsrcWord3;
  return r;
}

// Direct-to-LDS loads: 16 (dma16) or 4 (dma4) bytes per lane, lane L's
// bytes landing at lds + 16 L (+ 4 L), lds wave-uniform. Written as
// assembly (no result registers: the data goes to LDS); completion is
// awaited explicitly with dma_wait before the barrier that publishes it. M0
// (reserved, so not listed as clobbered) is written by these statements
// only: nothing else in this kernel uses it.
// the resource (and below the LDS address) as scalars for the asm operands
// (no-ops where the compiler already keeps them in scalar registers)
__device__ __forceinline__ i32x4_t uniform(const i32x4_t& r) {
  i32x4_t u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}
__device__ __forceinline__ void dma16(const i32x4_t& r, uint32_t voff, uint32_t lds) {
  const i32x4_t rs = uniform(r);
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(l)
               : "memory");
}
__device__ __forceinline__ void dma4(const i32x4_t& r, uint32_t voff, uint32_t lds) {
  const i32x4_t rs = uniform(r);
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(l)
               : "memory");
}
template <int N>
__device__ __forceinline__ void dma_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

constexpr int kStages = 2;
constexpr int kDmaPerStep = 10;   // per wave: 4 activation code, 4 weight code, 1 activation scale, 1 weight scale
constexpr int kOffA = 0, kOffB = kACodes, kOffAS = kOffB + kBCodes, kOffBS = kOffAS + kAScales;
constexpr int kStageBytes = kOffBS + kBScales;
constexpr int kLdsBytes = kStages * kStageBytes;

__global__ __launch_bounds__(kWaves * 64) void k_mx_a4(const A4Args a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int K = a.K, Kh = K >> 1, Ks = K >> 5, C = a.C;
  const int T = a.gx * a.gy;
  // the whole scale array: a slab's rows past M read the next step's first
  // rows (scales of zero codes, in rows never stored) or, at the end, zeros
  const i32x4_t rs = rsrc4(a.xs, (uint32_t)a.M * Ks);
  // one tile: its origin, weight row groups and buffer resources (tiles in
  // row-major order, so consecutive workgroups share activation rows)
  struct Tile {
    int m0, n0, ngroups;
    i32x4_t ra, rw;
  };
  auto tile_at = [&](int id) {
    Tile u;
    const int tm = id / a.gx;
    u.m0 = tm * kBM;
    u.n0 = (id - tm * a.gx) * kBN;
    const int rows = min(kBM, a.M - u.m0), g0 = u.n0 >> 3;
    u.ngroups = min(kBN / 8, a.G - g0);
    u.ra = rsrc4(a.xa + (int64_t)u.m0 * Kh, (uint32_t)rows * Kh);
    u.rw = rsrc4(a.w + (int64_t)g0 * C * kMxTileBytes, (uint32_t)u.ngroups * C * kMxTileBytes);
    return u;
  };
  const uint32_t sbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;

  // DMA lane roles. A code instruction fills 8 LDS rows of 128 bytes: lane
  // -> row lane / 8 of the 8, slot lane % 8, which holds chunk (lane % 8) ^
  // ((row / 2) % 8): for rows 8 d .. 8 d + 7 that is (lane % 8) ^ (4 (d % 2)
  // + lane / 16).
  const int dr = lane >> 3, dj0 = (lane & 7) ^ (dr >> 1), dj1 = (lane & 7) ^ (4 + (dr >> 1));
  constexpr uint32_t kOut = 0x80000000u;   // an offset past every resource
  auto issue = [&](const Tile& u, int step, int stage) {
    const int k0 = step * kKS, c = k0 >> 10, p0 = (k0 & 1023) >> 5;
    const uint32_t st = sbase + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // activation codes: rows 8 d .. 8 d + 7, d = 4 wave + i
      const int d = 4 * wave + i, dj = (i & 1) ? dj1 : dj0;
      dma16(u.ra, (uint32_t)((8 * d + dr) * Kh + (k0 >> 1) + 16 * dj), st + kOffA + d * 1024);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // weight codes: group e = 4 wave + i, its rows 2 q + h = lane / 8
      const int e = 4 * wave + i, dj = (i & 1) ? dj1 : dj0;
      dma16(u.rw, (uint32_t)((e * C + c) * kMxTileBytes + (dr >> 1) * 1024 + (dr & 1) * 512 + (p0 + dj) * 16),
            st + kOffB + e * 1024);
    }
    {   // activation scales: sub-step v = wave / 4 (128 columns), rows 64 (wave % 4) + lane
      const int v = wave >> 2, r = 64 * (wave & 3) + lane;
      dma4(rs, (uint32_t)(((2 * step + v) * a.M + u.m0 + r) * 4), st + kOffAS + v * 1024 + (wave & 3) * 256);
    }
    if (lane < 16) {   // weight scales: 16-byte piece P = 16 wave + lane: group P / 4, parity (P / 2) % 2, half P % 2
      const int P = 16 * wave + lane, g = P >> 2;
      dma16(u.rw, g < u.ngroups ? (uint32_t)((g * C + c) * kMxTileBytes + 4096 + ((P >> 1) & 1) * 128 + p0 * 4 + (P & 1) * 16)
                            : kOut,
            st + kOffBS + wave * 256);
    }
  };

  f32x16_t acc[4][2];

  const int r32 = lane & 31, kb = lane >> 5;
  // One MFMA step's operands: 4 activation and 2 weight fragments with
  // their scales, for 32-element block 2 ks + kb of the stage.
  struct Frag {
    i32x8_t av[4], bv[2];
    int as[4], bs[2];
  };
  auto load = [&](int stage, int ks, Frag& f) {
    const uint8_t* s = lds + stage * kStageBytes;
    const int j = 2 * ks + kb;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 128 * wm + 32 * mt + r32;
      const uint4 v = *reinterpret_cast<const uint4*>(s + kOffA + row * 128 + slot(row, j));
      f.av[mt] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      f.as[mt] = s[kOffAS + (j >> 2) * 1024 + row * 4 + (j & 3)];
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = 64 * wn + 32 * nt + r32;
      const uint4 v = *reinterpret_cast<const uint4*>(s + kOffB + n * 128 + slot(n, j));
      f.bv[nt] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      f.bs[nt] = s[kOffBS + ((n >> 3) * 2 + (n & 1)) * 32 + j * 4 + ((n & 7) >> 1)];
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.av[mt], f.bv[nt], acc[mt][nt], 4, 4, 0,
                                                                        f.as[mt], 0, f.bs[nt]);
  };
  // 8 MFMAs with the 12 LDS reads of the other half-step between them
  auto interleave = [] {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  // Software pipeline: the first half of a step multiplies fragments read
  // before the barrier while the second half's fragments are read; the
  // second half multiplies while the next step's first fragments are read
  // (after the barrier that publishes that step's stage). The barrier's
  // fence completes every LDS read issued before it, so a stage is free for
  // the next load two steps later.
  // K % 256 == 128 ends with a half step: its second half reads zero
  // weight codes and scales (tile padding) and activation scales past the
  // array (zeros), so it adds exact zeros
  // Persistent: one workgroup per CU walks tiles blockIdx.x, + gridDim.x, ...
  // A tile's last step loads the next tile's first step, and the read after
  // its barrier takes that step's first fragments, so the next tile starts
  // at once while this tile's results are stored.
  const int nsteps = (K + kKS - 1) / kKS;
  int id = blockIdx.x, stage = 0;
  Tile cur = tile_at(id);
  issue(cur, 0, 0);
  dma_wait<0>();
  __syncthreads();
  Frag f0, f1;
  load(stage, 0, f0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const int nid = id + (int)gridDim.x;
    Tile nxt = cur;
    if (nid < T) nxt = tile_at(nid);
    for (int s = 0; s < nsteps; ++s) {
      if (s + 1 < nsteps)
        issue(cur, s + 1, stage ^ 1);   // the stage step s - 1 used
      else if (nid < T)
        issue(nxt, 0, stage ^ 1);       // the next tile's first step
      load(stage, 1, f1);
      mma(f0);
      interleave();
      load(stage, 2, f0);
      mma(f1);
      interleave();
      load(stage, 3, f1);
      mma(f0);
      interleave();
      dma_wait<0>();   // step s + 1 landed
      __syncthreads();
      stage ^= 1;
      load(stage, 0, f0);   // past the last step: the next tile's first fragments (or unused)
      mma(f1);
      interleave();
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = cur.n0 + 64 * wn + 32 * nt + r32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = cur.m0 + 128 * wm + 32 * mt + (i & 3) + 8 * (i >> 2) + 4 * kb;
          if (row < a.M && col < a.N) __builtin_nontemporal_store(acc[mt][nt][i], &a.y[(int64_t)row * a.ldy + col]);
        }
      }
    if (nid >= T) break;
    id = nid;
    cur = nxt;
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
  a.gx = (int)((N + kBN - 1) / kBN);
  a.gy = (int)((M + kBM - 1) / kBM);
  // more than 64 KB of dynamic LDS must be allowed once per device
  constexpr int kMaxDevices = 64;
  // (and the CU count, one persistent workgroup per CU, is read once)
  static std::atomic<int> cus_of[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int cus = cus_of[dev].load(std::memory_order_acquire);
  if (cus == 0) {   // racing first calls store the same values
    e = hipFuncSetAttribute((const void*)k_mx_a4, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus < 1) return hipErrorInvalidDevice;
    cus_of[dev].store(cus, std::memory_order_release);
  }
  const int64_t tiles = (int64_t)a.gx * a.gy;
  const dim3 grid((unsigned)std::min<int64_t>(tiles, cus)), block(kWaves * 64);
  hipLaunchKernelGGL(k_mx_a4, grid, block, kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace fp4

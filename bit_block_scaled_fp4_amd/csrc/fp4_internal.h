// Internal declarations shared by the HIP sources of libfp4 (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fp4 {

// Tiled device layout: 8-row groups x 1024-element K chunks (include/fp4.h).
constexpr int kGroupRows = 8;
constexpr int kChunkK = 1024;
constexpr int kTilePacked = 4096;  // 8 rows x 32 lanes x 16 B
constexpr int kTileScale = 512;    // 32 lanes x 8 rows x 2 blocks
constexpr int kMaxProj = 8;

__host__ __device__ inline int64_t groups_of(int64_t N) { return (N + kGroupRows - 1) / kGroupRows; }
__host__ __device__ inline int64_t chunks_of(int64_t K) { return (K + kChunkK - 1) / kChunkK; }

struct ProjDesc {
  const uint8_t* packed;
  const uint8_t* scales;
  const float* gscale;
  float* y;
  int64_t ldy;
  int32_t N;
  int32_t tile_begin;  // first workgroup of this projection in the fused grid (set by launch_gemv)
};

struct GemvArgs {
  const uint16_t* x;  // bf16 [M][K]
  int32_t M;
  int32_t K;
  int32_t C;      // chunks of 1024
  int32_t nproj;
  int32_t total_tiles;  // workgroups in the grid (set by launch_gemv)
  int32_t gw;           // row groups per workgroup (set by launch_gemv)
  int32_t cu;           // half-wave units per row group (set by launch_gemv)
  ProjDesc proj[kMaxProj];
};

hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, bool tiled, uint8_t* packed,
                           uint8_t* scales, float* gscale, hipStream_t s);
hipError_t launch_retile(const uint8_t* packed, const uint8_t* scales, int64_t N, int64_t K,
                         uint8_t* packed_t, uint8_t* scales_t, hipStream_t s);
// Fills the grid fields (tile_begin, total_tiles, gw, cu) of a copy of `a`
// and launches. gw/cu > 0 and rows (8 or 4 rows per unit) override the
// automatic choice (for tuning).
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s, int gw = 0, int cu = 0, int rows = 0);
// Small-M product on bf16 MFMA (M padded to 16 per M-tile; 16 or 32 rows
// per pass, more rows loop passes). nt: 16-row N-subtiles per wave (1 or 2);
// split: waves per workgroup (0 = automatic).
hipError_t launch_gemv_mfma(const GemvArgs& a, hipStream_t s, int nt = 2, int split = 0);
hipError_t launch_prefill(float* y, const uint16_t* x, const uint8_t* packed, const uint8_t* scales,
                          const float* gscale, int64_t M, int64_t N, int64_t K, hipStream_t s);

}  // namespace fp4

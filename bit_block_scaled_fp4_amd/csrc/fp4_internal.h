// Internal declarations shared by the HIP sources of libfp4 (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fp4 {

// Tiled device layout (include/fp4.h): 8-row groups x 1024-element K chunks;
// tile (g, c) is kTileBytes at (g*C + c)*kTileBytes and holds the group's
// codes for the chunk (row r at r*512, 16 bytes per 32-element lane piece)
// followed by their E4M3 block scales.
constexpr int kGroupRows = 8;
constexpr int kChunkK = 1024;
constexpr int kTileCodes = 4096;   // 8 rows x 32 pieces x 16 B
constexpr int kTileScales = 512;   // 8 rows x 64 blocks
constexpr int kTileBytes = kTileCodes + kTileScales;
constexpr int kMaxProj = 8;

__host__ __device__ inline int64_t groups_of(int64_t N) { return (N + kGroupRows - 1) / kGroupRows; }
__host__ __device__ inline int64_t chunks_of(int64_t K) { return (K + kChunkK - 1) / kChunkK; }

// Byte offset inside a tile of the scale of (row r of the group, block b of
// the chunk): the scales of rows 2i + h sit in half h (256 bytes), 8 bytes
// per lane piece l = b / 2, ordered (i, b % 2). A 64-lane wave whose lane
// 32h + l reads piece l of rows h, 2 + h, 4 + h, 6 + h finds all 8 of its
// scale bytes at kTileCodes + 8 * lane.
__host__ __device__ inline int tile_scale_offset(int r, int b) {
  return kTileCodes + (r & 1) * 256 + (b >> 1) * 8 + (r >> 1) * 2 + (b & 1);
}

// MXFP4 (OCP MX: E8M0 scale per 32 elements, no tensor scale) tiles: the
// same 8-row x 1024-element codes, then 256 scale bytes; the scale of
// (row 2i + h of the group, block l of the chunk) at kTileCodes + 128h + 4l +
// i, so lane 32h + l of a wave finds the scales of its four rows as one
// 4-byte word at kTileCodes + 4 * lane.
constexpr int kMxTileScales = 256;
constexpr int kMxTileBytes = kTileCodes + kMxTileScales;
__host__ __device__ inline int mx_tile_scale_offset(int r, int l) { return kTileCodes + (r & 1) * 128 + l * 4 + (r >> 1); }

// Caller-owned scratch memory (include/fp4.h, "Workspaces"). The first
// kWsHeaderBytes hold counters, one per 128-byte line, that are zero before
// a call and that every kernel using them puts back to zero; the bytes after
// the header are scratch that a call overwrites freely.
constexpr size_t kWsHeaderBytes = 65536;
constexpr int kWsCounterWords = 32;                          // u32 words per counter line
constexpr int kWsCounters = (int)(kWsHeaderBytes / 128);     // 512
struct Workspace {
  uint8_t* p = nullptr;
  size_t bytes = 0;
  bool valid() const { return p != nullptr; }
  unsigned* counter(int i) const { return reinterpret_cast<unsigned*>(p) + (size_t)i * kWsCounterWords; }
  uint8_t* scratch() const { return p + kWsHeaderBytes; }
};

// Greedy choice folded into a product launch whose every workgroup covers
// all M activation rows (include/fp4.h, fp4_lm_head_greedy). Each workgroup
// stores its largest (value, index) key per row in keys[m * S + wg], part of
// the workspace header (zero between calls); the workgroup with the last
// index collects them, writes idx and zeroes them again (greedy.h).
struct GreedyArgs {
  int32_t* idx = nullptr;   // [M] (nullptr: no greedy epilogue)
  uint64_t* keys = nullptr; // [M][S], in the workspace header
  int32_t S = 0;            // workgroups of the launch
};
// Whether the M x S keys fit in the workspace header.
inline bool greedy_keys_fit(int64_t M, int64_t S) { return M * S * 8 <= (int64_t)kWsHeaderBytes; }

struct ProjDesc {
  const uint8_t* tiles;
  const float* gscale;
  float* y;
  int64_t ldy;
  int32_t N;
  int32_t wg_begin;  // first workgroup of this projection in the fused grid (set by the launcher)
};

struct GemvArgs {
  const uint16_t* x;  // bf16 [M][K]
  int32_t M;
  int32_t K;
  int32_t C;          // chunks of 1024
  int32_t nproj;
  int32_t wc;         // waves per row group (set by the launcher)
  int32_t gw;         // row groups per workgroup (set by the launcher)
  ProjDesc proj[kMaxProj];
  GreedyArgs greedy;  // optional epilogue of the vector-ALU kernel (one projection)
  // optional SwiGLU epilogue of the vector-ALU kernel (projections 0 = gate
  // and 1 = up, equal N): h[m][n] = bf16(silu(gate) * up), bf16 [M][ldh]
  uint16_t* h;
  int64_t ldh;
  // optional RMSNorm prologue of the vector-ALU kernel: every product reads
  // bf16(x[m][k] / sqrt(mean_k x[m][k]^2 + eps) * gain[k]) instead of x
  const uint16_t* gain;
  float eps;
  int32_t mx;         // MXFP4 tiles (no tensor scale; vector-ALU kernel only)
};

hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, bool tiled, uint8_t* packed,
                           uint8_t* scales, float* gscale, hipStream_t s);
// The same rule for FP8 E4M3 codes times one fp32 scale (*w_scale, device).
hipError_t launch_quantize_fp8(const uint8_t* W, const float* w_scale, int64_t N, int64_t K, bool tiled,
                               uint8_t* packed, uint8_t* scales, float* gscale, hipStream_t s);
// MXFP4 quantisation of bf16 W (K % 32 == 0), one pass.
hipError_t launch_quantize_mx(const uint16_t* W, int64_t N, int64_t K, int mode, uint8_t* packed, uint8_t* scales,
                              hipStream_t s);
hipError_t launch_retile(const uint8_t* packed, const uint8_t* scales, int64_t N, int64_t K, uint8_t* tiles,
                         hipStream_t s);
// Vector-ALU product for M <= 4 activation rows (larger M: an error; those
// go to launch_gemv_mma). Positive gw (row groups per workgroup) and wc
// (waves per row group) override the automatic geometry (tuning).
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s, int gw = 0, int wc = 0);

// Both operands MXFP4 on the block-scaled FP4 matrix cores (prefill_a4.hip):
// y [M][N] from activation codes [M][K/2] and scales [M][K/32] and MX tiles.
hipError_t launch_mx_a4(float* y, const uint8_t* xq_codes, const uint8_t* xq_scales, const uint8_t* w_tiles, int64_t M,
                        int64_t N, int64_t K, hipStream_t s);
// Workgroups launch_gemv would launch for `a` (geometry as chosen there).
int64_t gemv_workgroups(const GemvArgs& a);
// The SwiGLU launch of the vector-ALU kernel (a.h set, two projections).
hipError_t launch_gemv_swiglu(const GemvArgs& a, hipStream_t s);
// Fallbacks for the matrix-core rows (neighbours.hip): RMS-normalised rows
// out = bf16(x * rsqrt(mean(x^2) + eps) * gain), bf16 [M][K]; and
// h = bf16(silu(g) * u) from fp32 g, u [M][N] (row stride N) into h [M][ldh].
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t K, uint16_t* out,
                          hipStream_t s);
hipError_t launch_swiglu(const float* g, const float* u, int64_t M, int64_t N, uint16_t* h, int64_t ldh,
                         hipStream_t s);
// Small-M product on bf16 MFMA, split over K chunks (16 activation rows per
// pass, more rows loop passes). With more than one chunk the chunk partial
// sums meet in `partials` (gemv_mma_partial_bytes of scratch) and are added
// in chunk order: inside the launch by the last-arriving workgroup of each
// pair block when `counters` (the workspace header: zero on entry, left
// zero) has room for the pair blocks, else by a second kernel. Without
// `partials` they are added atomically into y after a fill kernel zeroes it
// (the summation order then varies between calls).
hipError_t launch_gemv_mma(const GemvArgs& a, float* partials, unsigned* counters, hipStream_t s,
                           int ppw = 0);   // ppw > 0: pairs per workgroup (tuning)
// Bytes of partial sums launch_gemv_mma keeps for `a` (0 when it keeps none).
size_t gemv_mma_partial_bytes(const GemvArgs& a);

// Matrix-core product for prefill-sized M over 1..kMaxProj weight tensors
// that read the same x (one launch). bn > 0 forces the output tile width
// (128, 192 or 256; tuning), else it is chosen from the shapes; splits > 0
// forces the K split of the last round's tiles (1: none; tuning). A split
// uses per-device workspaces allocated on first need and kept.
struct PrefillProjDesc {
  const uint8_t* tiles;
  const float* gscale;
  float* y;
  int64_t ldy;
  int64_t N;
};
// Without a workspace the last round's tiles are never split.
hipError_t launch_prefill(const PrefillProjDesc* projs, int nproj, const uint16_t* x, int64_t M, int64_t K,
                          const Workspace& ws, hipStream_t s, int bn = 0, int splits = 0, bool mx = false);   // mx: MXFP4 tiles
// Workspace bytes a split of the last round's tiles needs (upper bound over
// tile widths and splits; 0 when no split can happen).
size_t prefill_ws_bytes(const PrefillProjDesc* projs, int nproj, int64_t M, int64_t K);

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();

// Greedy choice per row of fp32 y [M][N] (row stride ldy): idx[m] = the first
// index of the largest value. With a workspace, rows longer than one
// workgroup's segment are split over workgroups whose keys meet there;
// without one, one workgroup reads each whole row.
hipError_t launch_argmax(int32_t* idx, const float* y, int64_t M, int64_t N, int64_t ldy, const Workspace& ws,
                         hipStream_t s);
size_t argmax_ws_bytes(int64_t M, int64_t N);

}  // namespace fp4

// NVFP4 x bf16 product for prefill-sized M on the matrix cores.
//
// Prefill pushes hundreds or thousands of prompt tokens through each layer
// at once, so the product is a real dense contraction and compute-bound
// (page "imp" README, the prefill paragraph; page "1. The big picture",
// "Two phases with very different costs"). It runs on gfx950 bf16 MFMA:
// weights are decoded to bf16 values E2M1 * E4M3 (at most 6 significant
// bits inside bf16 range: exact) and the tensor scale multiplies the fp32
// result once in the epilogue.
//
// Tiling. A 256-thread workgroup computes a 256 (tokens) x BN (outputs)
// tile, BN = 128, 192 or 256. For BN = 128 and 256 the four waves split the
// columns (1 x 4 grid: each wave owns all 256 rows x BN/4 columns as 8 x NJ
// v_mfma_f32_32x32x16_bf16 tiles, so each decoded weight operand feeds 8
// MFMAs); for BN = 192 they form a 2 x 2 grid (128 x 96 each, 4 x 3 tiles).
// K advances in steps of 64, each split in four 16-deep MFMA slices.
//
// Data movement. Every global read is a direct-to-LDS buffer load (16 bytes
// per lane, no registers, coalesced 128-byte row segments):
//   - activations: two 32 KB stages, one step each, loaded a step ahead;
//   - packed weight codes: two stages of BN rows x 128 bytes, a window of
//     four steps each (one 128-byte piece run of every row of the tiled
//     layout), loaded during the first steps of the window before;
//   - block scales: two stages holding the tiled layout's scale bytes of the
//     same windows.
// Each wave then reads its MFMA operands from LDS: activations as bf16
// fragments, weights as one 16-byte code piece per lane per step that it
// decodes to bf16 slice by slice while the previous slice's MFMAs run.
// Keeping the weights packed in LDS cuts their LDS traffic fourfold against
// decoded bf16 tiles. The dot product is taken over a permuted K order, the
// same for both operands: lane half h of slice s covers K offsets
// 32h + 8s .. 32h + 8s + 7 of the step, so a lane's weight codes for a step
// are one 16-byte piece of one row.
//
// LDS rows (activations: 64 bf16; weights: 8 code pieces) are eight 16-byte
// slots, slot j ^ swz(r) holding chunk j of row r, so reads and the DMA
// writes never meet in a bank. Each step ends with the wave's DMA wait and
// one barrier.
//
// Order. Workgroups go round-robin over the 8 XCDs; tile t = (XCD, rank)
// is mapped so that one XCD works through all output tiles of one 256-row
// activation slab (2.6 MB at K = 5120, kept in that XCD's 4 MB L2) while
// every XCD streams the weights.
//
// Last round. When the last round of tiles over the compute units would
// leave most of them idle, those tiles run in a second launch, each split
// into S <= 4 ranges of whole windows along K on separate workgroups; the
// pieces exchange fp32 partial sums through the caller's workspace (its
// header holds one arrival counter per split tile) and the last piece of a
// tile adds them in piece order (so the result does not depend on which
// piece finishes last) and writes y. Without a workspace nothing is split.
//
// Bounds: the buffer loads read zeros for activation rows past M, columns
// past K, weight row groups past N and steps past the end, without touching
// memory; the epilogue's buffer stores drop rows past M and columns past N.
#include <algorithm>
#include <atomic>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int BM = 256, BK = 64;
constexpr int kWin = 4;                  // steps per weight window (256 K = 8 pieces of a row)
constexpr int kAStage = BM * BK * 2;     // 32 KB of activations per stage

// MX: MXFP4 tiles, whose window holds 64 scale bytes per 8-row group (one
// E8M0 per piece) instead of 128, moved 16 groups per DMA instruction (the
// stage rounded up to whole instructions).
template <int BN, bool MX = false>
struct Lds {
  static constexpr int kBStage = BN * 128;        // codes of one window
  static constexpr int kSStage = MX ? (BN / 8 + 15) / 16 * 1024 : BN / 8 * 128;   // scale bytes of one window
  static constexpr int kA = 0, kB = 2 * kAStage, kS = kB + 2 * kBStage;
  static constexpr int kBytes = kS + 2 * kSStage;
};

// Chunk slot of chunk j in row r: j ^ swz(r). swz is a bijection on every 8
// consecutive rows, and on the even (odd) rows of every 16, so 16-byte reads
// by 8 or 16 lanes of consecutive rows never meet in a bank.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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

// Direct-to-LDS load of 16 bytes per lane: lane L's bytes land at
// lds + 16 L (lds wave-uniform). Written as assembly because the compiler
// would otherwise wait for it before every LDS access; completion is
// awaited explicitly with dma_wait before the barrier that publishes it.
// M0 (reserved, so not listed as clobbered) is written by these statements
// only: nothing else in this kernel uses it.
__device__ __forceinline__ void dma16(const i32x4_t& rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// Two E2M1 codes (byte `sel` of w) times the block scale as packed bf16: one
// v_cvt_pk_bf16_f32, exact (<= 6 significant bits, inside bf16 range).
__device__ __forceinline__ uint32_t dec2(uint32_t w, int sel, float s) {
  const f32x2_t e = fp4x2_f32(w, sel);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{e[0] * s, e[1] * s}, bf16x2_t));
}

// Two E2M1 codes (byte `sel` of w) times 2^(c - 127) as packed bf16, in one
// v_cvt_scalef32_pk_bf16_fp4: the conversion applies the exponent field of
// its fp32 scale operand, here c << 23. Checked on MI355X against the fp32
// product path for every code byte and every c: bit-identical for c <= 254,
// subnormal results included; c = 255 (a NaN scale, which no quantiser here
// writes) gives a NaN of the other sign.
__device__ __forceinline__ uint32_t dec2_e8m0(uint32_t w, int sel, float s) {
  switch (sel) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  }
}

// Eight codes (word `slice` of a 16-byte piece) as a bf16x8 MFMA operand;
// `sc` holds the piece's two E4M3 block scales (slices 0, 1 use byte 0,
// slices 2, 3 byte 1) or, MX, its one E8M0 scale (byte 0; e2m1 * 2^(c-127)
// is exact in bf16 for the scales a quantiser produces from bf16 weights).
template <bool MX>
__device__ __forceinline__ bf16x8_t decode8(const uint4& piece, uint32_t sc, int slice) {
  const uint32_t w = word(piece, slice);
  if (MX) {
    const float s = __uint_as_float((sc & 0xFFu) << 23);
    const uint4 o = make_uint4(dec2_e8m0(w, 0, s), dec2_e8m0(w, 1, s), dec2_e8m0(w, 2, s), dec2_e8m0(w, 3, s));
    return __builtin_bit_cast(bf16x8_t, o);
  }
  const float s = slice < 2 ? __builtin_amdgcn_cvt_f32_fp8((int)sc, 0) : __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
  const uint4 o = make_uint4(dec2(w, 0, s), dec2(w, 1, s), dec2(w, 2, s), dec2(w, 3, s));
  return __builtin_bit_cast(bf16x8_t, o);
}

// This lane's weights of one step: piece (lane / 32) of row (lane % 32) of
// each of the wave's NJ 32-column tiles, with the piece's two block scales.
template <int NJ>
struct Pieces {
  uint4 w[NJ];
  uint32_t sc[NJ];
};
// MFMA operands of one slice.
template <int MI, int NJ>
struct Frags {
  bf16x8_t a[MI], b[NJ];
};

// Deals the instructions of a scheduling region out around its NMFMA MFMAs:
// after MFMA i come up to kValuPerMfma VALU operations, then one LDS read
// (i < NDSR). A wave issues in order, so an MFMA queued behind a long run of
// decode arithmetic would leave the matrix core idle.
constexpr int kValuPerMfma = 3;   // swept 2..8 on MI355X: 3 best (1-2 % over 5)
template <int NMFMA, int NDSR>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // VALU
    if (i < NDSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// One launch covers one or more weight tensors that read the same
// activations (the gate and up halves of an MLP, or Q, K and V): tile t =
// (256-row slab, projection, BN-column tile), slab-major, so an XCD's run of
// tiles stays on one activation slab across all projections.
struct PrefillProj {
  const uint8_t* tiles;
  const float* gscale;
  float* y;
  int64_t ldy;
  int32_t N;
  int32_t nt_begin;   // first column tile of this projection within a slab
};
struct PrefillArgs {
  const uint16_t* x;
  float* part;         // split tiles: partial sums, kPartFloats<BN> per piece
  unsigned* cnt;       // split tiles: arrivals (kCntStride apart, the workspace header), zero between launches
  int32_t M, K, m_tiles, nt_total, nproj;
  int32_t dp_tiles;    // tiles computed whole by one workgroup: the first ones
  int32_t per_xcd;     // of those, per XCD
  int32_t splits;      // workgroups (K ranges) per remaining tile
  PrefillProj proj[kMaxProj];
};
constexpr int kMaxSplits = 4;
constexpr int kCntStride = kWsCounterWords;   // one 128-byte line per counter
template <int BN>
constexpr int kPartFloats = BM * BN;

// SPLIT = false: workgroup b takes whole tile b' (XCD-contiguous order) of
// the first dp_tiles; SPLIT = true: workgroup b takes K range b % S of tile
// dp_tiles + b / S.
template <int BN, bool SPLIT, bool MX = false>
__global__ __launch_bounds__(256, 1) void k_prefill(const PrefillArgs a) {
  constexpr int TB = MX ? kMxTileBytes : kTileBytes;
  // wave grid: WM x WN waves, each owning 256 / WM rows (MI 32-row MFMA
  // tiles) x BN / WN columns (NJ 32-column tiles); 1 x 4 where BN / 4 is a
  // multiple of 32, so each decoded weight operand feeds 8 MFMAs
  constexpr int WM = BN % 128 == 0 ? 1 : 2, WN = 4 / WM;
  constexpr int MI = 8 / WM;
  constexpr int NJ = BN / (32 * WN);   // 32-column MFMA tiles per wave
  constexpr int NG = BN / 8;           // 8-row weight groups per tile
  constexpr int NBI = NG / 4;          // code DMA instructions per wave per window
  constexpr int NSW = MX ? (NG + 15) / 16 : NG / 8;   // waves issuing one scale DMA per window
  using L = Lds<BN, MX>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int last_piece;
  const int id = blockIdx.x, S = a.splits;
  int lin, piece = 0;
  if (!SPLIT) {
    lin = (id & 7) * a.per_xcd + (id >> 3);
    if (lin >= a.dp_tiles) return;
  } else {
    lin = a.dp_tiles + id / S;
    piece = id - (id / S) * S;
  }
  constexpr bool split = SPLIT;
  const int mt = lin / a.nt_total, jn = lin - mt * a.nt_total;
  int pi = 0;
  while (pi + 1 < a.nproj && jn >= a.proj[pi + 1].nt_begin) ++pi;
  const PrefillProj& pj = a.proj[pi];
  const uint16_t* __restrict__ x = a.x;
  const uint8_t* __restrict__ tiles = pj.tiles;
  const int M = a.M, N = pj.N, K = a.K;
  const int64_t ldy = pj.ldy;
  const int m0 = mt * BM, n0 = (jn - pj.nt_begin) * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, lh = lane >> 5;
  const int C = (K + kChunkK - 1) / kChunkK;
  const int G = (N + 7) >> 3;
  const int KT = (K + BK - 1) / BK;
  // this workgroup's steps: whole windows, piece p of S taking windows
  // [p nwin / S, (p + 1) nwin / S)
  const int nwin = (KT + kWin - 1) / kWin;
  const int kt0 = split ? piece * nwin / S * kWin : 0;
  const int kt1 = split ? min(KT, (piece + 1) * nwin / S * kWin) : KT;
  const uint32_t sbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;

  const int mrows = min(BM, M - m0);
  const int ngroups = min(NG, G - (n0 >> 3));
  const i32x4_t rx = rsrc4(x + (int64_t)m0 * K, (uint32_t)(mrows * K * 2));
  const i32x4_t rw = rsrc4(tiles + (int64_t)(n0 >> 3) * C * TB, (uint32_t)(ngroups * C * TB));
  const i32x4_t rnull = rsrc4(x, 0);

  // DMA lane roles. One instruction fills 8 LDS rows of 128 bytes: lane ->
  // row (lane / 8) of the 8, slot lane % 8, which holds chunk
  // (lane % 8) ^ swz(row); for 8-aligned row blocks swz(row) is
  // (lane / 8) ^ (block & 1).
  const int dr = lane >> 3, ds = lane & 7;
  const int achunk0 = ds ^ dr, achunk1 = ds ^ dr ^ 1;   // even / odd 8-row blocks
  // activations: instruction i of this wave fills rows 64 wave + 8i + dr
  const uint32_t a_row_off = (uint32_t)((wave * 64 + dr) * K * 2);
  auto dma_a = [&](int kt, int i0, int i1) {
    const int k0 = kt * BK;
    const i32x4_t& rs = kt < kt1 ? rx : rnull;
    // a chunk past K (ragged last step) gets bit 31 set: an offset past the resource
    const uint32_t oob0 = (uint32_t)((K - 1 - k0 - achunk0 * 8) >> 31) << 31;
    const uint32_t oob1 = (uint32_t)((K - 1 - k0 - achunk1 * 8) >> 31) << 31;
    const uint32_t lds = sbase + L::kA + (kt & 1) * kAStage + wave * 64 * 128;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int ch = (i & 1) ? achunk1 : achunk0;
      const uint32_t off = (a_row_off + (uint32_t)(i * 8 * K * 2) + (uint32_t)((k0 + ch * 8) * 2)) | ((i & 1) ? oob1 : oob0);
      dma16(rs, off, lds + i * 1024);
    }
  };
  // weight codes: instruction i of this wave fills group g = NBI wave + i
  // (rows 8g + dr); window `win` covers pieces 8 (win % 4) .. + 7 of chunk win / 4
  auto dma_b = [&](int win, int i0, int i1) {
    const bool live = win * kWin < kt1;
    const i32x4_t& rs = live ? rw : rnull;
    const int c = win >> 2, p0 = (win & 3) * 8;
    const uint32_t lds = sbase + L::kB + (win & 1) * L::kBStage;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int g = NBI * wave + i;
      const int piece = ds ^ dr ^ (g & 1);
      const uint32_t off = (uint32_t)((g * C + c) * TB + dr * 512 + (p0 + piece) * 16);
      dma16(rs, off, lds + g * 1024);
    }
  };
  // scales: wave w < NSW fills groups 8w .. 8w + 7, 128 bytes each: half
  // (lane / 4) % 2 of the tile's scale area, 64 bytes from piece p0 on.
  // MX: groups 16w .. 16w + 15, 64 bytes each: lane / 4 picks the group,
  // (lane / 2) % 2 the row parity h, lane % 2 which 16 of the 32 bytes of
  // pieces p0 .. p0 + 7 (their four rows' scales, 4 bytes per piece).
  auto dma_s = [&](int win) {
    if (wave >= NSW) return;
    const bool live = win * kWin < kt1;
    const i32x4_t& rs = live ? rw : rnull;
    const int c = win >> 2, p0 = (win & 3) * 8;
    uint32_t off;
    if (MX) {
      const int g = 16 * wave + (lane >> 2);
      off = (uint32_t)((g * C + c) * TB + kTileCodes + ((lane >> 1) & 1) * 128 + p0 * 4 + (lane & 1) * 16);
    } else {
      const int g = 8 * wave + dr;
      off = (uint32_t)((g * C + c) * TB + kTileCodes + ((lane >> 2) & 1) * 256 + p0 * 8 + (lane & 3) * 16);
    }
    dma16(rs, off, sbase + L::kS + (win & 1) * L::kSStage + wave * 1024);
  };

  // operand reads
  auto read_a = [&](int stage, int s, Frags<MI, NJ>& f) {
    const uint8_t* As = smem + L::kA + stage * kAStage;
    const int lchunk = 4 * lh + s;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm * (BM / WM) + i * 32 + l32;
      f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + r * 128 + ((lchunk ^ swz(r)) * 16));
    }
  };
  auto read_pieces = [&](int kt, Pieces<NJ>& p) {
    const int win = kt / kWin, q = 2 * (kt % kWin) + lh;   // piece within the window
    const uint8_t* Bs = smem + L::kB + (win & 1) * L::kBStage;
    const uint8_t* Ss = smem + L::kS + (win & 1) * L::kSStage;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = wn * (BN / WN) + j * 32 + l32;
      p.w[j] = *reinterpret_cast<const uint4*>(Bs + n * 128 + ((q ^ swz(n)) * 16));
      if (MX)
        p.sc[j] = Ss[(n >> 3) * 64 + (n & 1) * 32 + q * 4 + ((n & 7) >> 1)];
      else
        p.sc[j] = *reinterpret_cast<const uint16_t*>(Ss + (n >> 3) * 128 + (n & 1) * 64 + q * 8 + ((n & 7) >> 1) * 2);
    }
  };
  auto decode_b = [&](const Pieces<NJ>& p, int s, Frags<MI, NJ>& f) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b[j] = decode8<MX>(p.w[j], p.sc[j], s);
  };

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mma = [&](const Frags<MI, NJ>& f) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // prologue: step kt0's activations, its window's codes and scales
  dma_a(kt0, 0, 8);
  dma_b(kt0 / kWin, 0, NBI);
  dma_s(kt0 / kWin);
  dma_wait();
  __syncthreads();
  Frags<MI, NJ> f0, f1;
  Pieces<NJ> pc;
  read_pieces(kt0, pc);
  decode_b(pc, 0, f0);

  // Step kt (activation stage kt % 2, window kt / 4): it loads the
  // activations of step kt + 1 (two of the eight loads in each slice: the
  // stage was last read a step ago, before the last barrier) and, in the
  // first three steps of a window, the next window's codes (two halves,
  // issued at the step's start) and scales; runs its four slices,
  // alongside each reading the next slice's activation operands and decoding
  // its weight operands; in its last slice reads the weight pieces of step
  // kt + 1 (published by an earlier barrier) and decodes their slice 0. The
  // step ends with the DMA wait and the barrier that publishes its loads.
  for (int kt = kt0; kt < kt1; ++kt) {
    const int sa = kt & 1, sw = kt % kWin, win = kt / kWin;
    read_a(sa, 0, f0);
    dma_a(kt + 1, 0, 2);
    if (sw == 0) dma_b(win + 1, 0, NBI / 2);
    if (sw == 1) dma_b(win + 1, NBI / 2, NBI);
    if (sw == 2) dma_s(win + 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    read_a(sa, 1, f1);
    dma_a(kt + 1, 2, 4);
    decode_b(pc, 1, f1);
    interleave<MI * NJ, MI>();
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    read_a(sa, 2, f0);
    dma_a(kt + 1, 4, 6);
    decode_b(pc, 2, f0);
    interleave<MI * NJ, MI>();
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    read_a(sa, 3, f1);
    dma_a(kt + 1, 6, 8);
    decode_b(pc, 3, f1);
    interleave<MI * NJ, MI>();
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    read_pieces(kt + 1, pc);   // past the end: stale LDS, never used
    decode_b(pc, 0, f0);
    interleave<MI * NJ, 2 * NJ>();
    __builtin_amdgcn_sched_barrier(0);
    dma_wait();
    __syncthreads();
  }

  if constexpr (SPLIT) {
    // Every piece stores its partial sums with device-scope stores (sc1:
    // through to the memory side, so another XCD's L2 cannot serve an old
    // copy), waits for them, and counts itself in; the last of the tile's S
    // pieces reads the S partials back with device-scope loads and adds them
    // in piece order, so the sum does not depend on which piece came last.
    // Layout per piece: [wave][i][j][e / 4][lane][e % 4].
    const int st = lin - a.dp_tiles;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        a.part + (int64_t)st * S * kPartFloats<BN>, (short)0, S * kPartFloats<BN> * 4, kRsrcWord3);
    constexpr int kSc1 = 16;   // cache-policy bit: device scope
    auto part_off = [&](int p, int i, int j, int q) {
      return (uint32_t)(p * kPartFloats<BN> * 4 + ((((wave * MI + i) * NJ + j) * 4 + q) * 64 + lane) * 16);
    };
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rp, part_off(piece, i, j, q), 0, kSc1);
        }
    dma_wait();
    __syncthreads();
    if (tid == 0) {
      const unsigned n = __hip_atomic_fetch_add(a.cnt + (int64_t)st * kCntStride, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      last_piece = n == (unsigned)(S - 1);
      // all S pieces are in: back to zero for the next launch
      if (last_piece) __hip_atomic_store(a.cnt + (int64_t)st * kCntStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_piece) return;
    // y = gscale * (sum of the S partials in piece order), 4 rows of one
    // column per float4 (rows r0 + 8q .. + 3 of element group q)
    const float gs = MX ? 1.0f : *pj.gscale;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(pj.y + (int64_t)m0 * ldy, (short)0,
                                                                         (int)((int64_t)(mrows - 1) * ldy + N) * 4,
                                                                         kRsrcWord3);
#pragma unroll 8
    for (int gq = 0; gq < 4 * MI * NJ; ++gq) {
      const int i = gq / (4 * NJ), j = (gq >> 2) % NJ, q = gq & 3;
      f32x4_t t[kMaxSplits];
#pragma unroll
      for (int p = 0; p < kMaxSplits; ++p)   // pieces past S: past the resource, zeros without an access
        t[p] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, part_off(p, i, j, q), 0, kSc1));
      f32x4_t sum = t[0];
#pragma unroll
      for (int p = 1; p < kMaxSplits; ++p)
        if (p < S) sum += t[p];
      const int n = n0 + wn * (BN / WN) + j * 32 + l32;
      const uint32_t oobn = (uint32_t)((N - 1 - n) >> 31) << 31;
      const int r0 = wm * (BM / WM) + i * 32 + lh * 4 + q * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gs * sum[e]), ry,
                                              (uint32_t)(((r0 + e) * (int)ldy + n) * 4) | oobn, 0, 0);
    }
    return;
  }

  // epilogue: lane l of a 32x32 tile holds column l % 32 and rows
  // 8(e/4) + 4(l/32) + e%4 (e < 16). Buffer stores drop rows past M (past
  // the resource) and columns past N (bit 31 set in the offset).
  const float gs = MX ? 1.0f : *pj.gscale;
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(pj.y + (int64_t)m0 * ldy, (short)0,
                                                                       (int)((int64_t)(mrows - 1) * ldy + N) * 4,
                                                                       kRsrcWord3);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn * (BN / WN) + j * 32 + l32;
      const uint32_t oobn = (uint32_t)((N - 1 - n) >> 31) << 31;
      const int r0 = wm * (BM / WM) + i * 32 + lh * 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = r0 + (e >> 2) * 8 + (e & 3);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gs * acc[i][j][e]), ry,
                                              (uint32_t)((r * (int)ldy + n) * 4) | oobn, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // one tile's values live at a time
    }
}

}  // namespace

// The last round's tiles: with few of them, splitting each along K into S
// pieces keeps S times as many compute units busy (bounded by kMaxSplits
// and by the tile's windows).
static int auto_splits(int64_t total, int64_t nwin, int ncu) {
  if (ncu <= 0) return 1;
  const int64_t tail = total - (total - 1) / ncu * ncu;
  return (int)std::max<int64_t>(1, std::min<int64_t>({kMaxSplits, ncu / tail, nwin}));
}

// What launch_prefill runs: the tile width, the K split S of the last
// round's tiles and how many tiles that round holds (0: none split).
struct PrefillPlan {
  int bn = 0;
  int S = 1;
  int64_t tail = 0;
};

static int64_t tiles_of(const PrefillProjDesc* projs, int nproj, int64_t M, int bn) {
  int64_t nt = 0;
  for (int i = 0; i < nproj; ++i) nt += (projs[i].N + bn - 1) / bn;
  return (M + BM - 1) / BM * nt;
}

static int splits_of(int64_t total, int64_t nwin, int ncu, int splits, bool allow) {
  if (!allow) return 1;
  return splits > 0 ? (int)std::min<int64_t>({splits, kMaxSplits, nwin}) : auto_splits(total, nwin, ncu);
}

static PrefillPlan plan_prefill(const PrefillProjDesc* projs, int nproj, int64_t M, int64_t K, int bn, int splits,
                                bool allow_split) {
  PrefillPlan pl;
  const int64_t nwin = ((K + BK - 1) / BK + kWin - 1) / kWin;
  const int ncu = std::max(1, device_cu_count());
  if (bn <= 0) {
    // Tile width (and K split), from a cost model fitted on MI355X at
    // M = 2048, K = 5120: a full round of workgroups over the compute units
    // takes the tile time (relative: 128 wide 0.66, 192 wide 0.85, 256 wide
    // 1; wider tiles do more MFMA work per LDS and load byte); a last round
    // that is not full takes max(0.7, fill) of it (fewer busy units run at
    // a higher clock); split S ways along K it takes 1/S of a tile plus 0.3
    // (the partial sums' exchange). Ties go to the wider tile.
    const int widths[3] = {256, 192, 128};
    const int cost[3] = {100, 85, 66};
    int64_t best = -1;
    for (int w = 0; w < 3; ++w) {
      const int64_t total = tiles_of(projs, nproj, M, widths[w]), full = (total - 1) / ncu, tail = total - full * ncu;
      const int S = splits_of(total, nwin, ncu, splits, allow_split);
      const int64_t last = S > 1 ? cost[w] * 100 / S + cost[w] * 30
                                 : cost[w] * std::max<int64_t>(70, tail * 100 / ncu);
      const int64_t t = full * cost[w] * 100 + last;
      if (best < 0 || t < best) {
        best = t;
        bn = widths[w];
      }
    }
  }
  pl.bn = bn;
  const int64_t total = tiles_of(projs, nproj, M, bn);
  pl.S = splits_of(total, nwin, ncu, splits, allow_split);
  pl.tail = pl.S > 1 ? total - (total - 1) / ncu * ncu : 0;
  if (pl.tail > kWsCounters) {   // one header counter per split tile
    pl.S = 1;
    pl.tail = 0;
  }
  return pl;
}

template <int BN, bool MX>
static hipError_t launch_bn(PrefillArgs a, const PrefillProjDesc* projs, const PrefillPlan& pl, const Workspace& ws,
                            hipStream_t s) {
  using L = Lds<BN, MX>;
  // more than 64 KB of dynamic LDS must be allowed once per kernel and device
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> attr_set[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {   // racing first calls set the same value
    e = hipFuncSetAttribute((const void*)k_prefill<BN, false, MX>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            L::kBytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)k_prefill<BN, true, MX>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              L::kBytes);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  int64_t nt = 0;
  for (int i = 0; i < a.nproj; ++i) {
    a.proj[i].nt_begin = (int32_t)nt;
    nt += (projs[i].N + BN - 1) / BN;
  }
  const int64_t mt = (a.M + BM - 1) / BM;
  const int64_t total = mt * nt;
  if (total > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int64_t tail = pl.tail;
  a.dp_tiles = (int32_t)(total - tail);
  a.per_xcd = (int32_t)((a.dp_tiles + 7) / 8);
  a.splits = pl.S;
  a.m_tiles = (int32_t)mt;
  a.nt_total = (int32_t)nt;
  if (tail > 0) {
    a.part = reinterpret_cast<float*>(ws.scratch());
    a.cnt = ws.counter(0);
  }
  // whole tiles, then the K pieces of the rest (a second launch: the split
  // epilogue in the same kernel would cost the whole-tile path registers)
  if (a.dp_tiles > 0) {
    hipLaunchKernelGGL((k_prefill<BN, false, MX>), dim3((unsigned)(8 * a.per_xcd)), dim3(256), L::kBytes, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tail > 0) {
    hipLaunchKernelGGL((k_prefill<BN, true, MX>), dim3((unsigned)(tail * pl.S)), dim3(256), L::kBytes, s, a);
    e = hipGetLastError();
  }
  return e;
}

size_t prefill_ws_bytes(const PrefillProjDesc* projs, int nproj, int64_t M, int64_t K) {
  const PrefillPlan pl = plan_prefill(projs, nproj, M, K, 0, 0, true);
  if (pl.tail == 0) return 0;
  return kWsHeaderBytes + (size_t)(pl.tail * pl.S) * (size_t)(BM * pl.bn) * sizeof(float);
}

hipError_t launch_prefill(const PrefillProjDesc* projs, int nproj, const uint16_t* x, int64_t M, int64_t K,
                          const Workspace& ws, hipStream_t s, int bn, int splits, bool mx) {
  if (nproj < 1 || nproj > kMaxProj) return hipErrorInvalidValue;
  // buffer offsets are 32-bit: one 256-row slab of activations, of outputs
  // and of weights must each stay below 2 GB
  const int64_t C = chunks_of(K);
  if ((int64_t)BM * K * 2 >= (int64_t(1) << 31) || (int64_t)(256 / 8) * C * kTileBytes >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  PrefillArgs a{};
  a.x = x;
  a.M = (int32_t)M;
  a.K = (int32_t)K;
  a.nproj = nproj;
  for (int i = 0; i < nproj; ++i) {
    if ((int64_t)BM * projs[i].ldy * 4 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    a.proj[i].tiles = projs[i].tiles;
    a.proj[i].gscale = projs[i].gscale;
    a.proj[i].y = projs[i].y;
    a.proj[i].ldy = projs[i].ldy;
    a.proj[i].N = (int32_t)projs[i].N;
  }
  PrefillPlan pl = plan_prefill(projs, nproj, M, K, bn, splits, ws.valid());
  if (pl.tail > 0 &&
      ws.bytes < kWsHeaderBytes + (size_t)(pl.tail * pl.S) * (size_t)(BM * pl.bn) * sizeof(float)) {
    pl.S = 1;   // the workspace is too small for this split (tuning calls only: the API checks the size)
    pl.tail = 0;
  }
  if (mx) {
    switch (pl.bn) {
      case 128: return launch_bn<128, true>(a, projs, pl, ws, s);
      case 192: return launch_bn<192, true>(a, projs, pl, ws, s);
      case 256: return launch_bn<256, true>(a, projs, pl, ws, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (pl.bn) {
    case 128: return launch_bn<128, false>(a, projs, pl, ws, s);
    case 192: return launch_bn<192, false>(a, projs, pl, ws, s);
    case 256: return launch_bn<256, false>(a, projs, pl, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp4

// NVFP4 x bf16 product for small M (a handful of concurrent decode streams or
// speculative-verify tokens) on the matrix cores.
//
// Several activation rows share one pass over the weights, so the weights
// are still read once (page "1. The big picture", the batching and
// speculative-decoding bullets of "The most important number in this
// book"). On the vector ALUs every extra row costs another two-term dot
// product per weight pair, which makes that path ALU-bound from about four
// rows on; here the weights are decoded once to exact bf16 and multiplied on
// v_mfma_f32_16x16x32_bf16 with the activation rows as the A operand.
//
// Work split (split-K). Workgroup (b, c) owns K chunk c (1024 elements) and a
// block of 16-row weight pairs (two 8-row groups). It first copies the
// activation rows of its chunk into LDS; its waves then walk the pairs, each
// pair needing only weight loads. With one chunk the kernel writes y
// directly. Otherwise the chunk partials meet in one of two ways:
//   - in the caller's workspace [C][pairs][16 n][R][4 m] (R = ceil(rows /
//     4) row quads of the pass, so a pair's partials are one contiguous run
//     of whole cache lines), added in chunk order
//     with the tensor scale applied (deterministic): for passes of at most 8
//     rows by the last of a pair block's C workgroups to finish, inside the
//     launch (header counters of the workspace); for 16-row passes by a
//     second kernel;
//   - without a workspace, a fill kernel first zeroes y and every workgroup
//     adds its scaled partials into y with fp32 atomics (the order of the
//     chunk sums, and so the last bits of y, can vary between calls).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, q = l / 16):
//   A: row l % 16, k = 8q .. 8q+7;  B: column l % 16, k = 8q .. 8q+7;
//   D: column l % 16, rows 4q .. 4q+3.
// The k order inside one MFMA is free as long as A and B agree.
//
// Two kernels, by the rows of a pass:
// - k_gemv_mma8 (at most 8 rows): the 16 A rows are (activation row m,
//   block parity b), A[(m, b)][k] = x[m][k] where k lies in a block of parity
//   b, else 0. One MFMA then covers one 32-element piece (two blocks) of 16
//   weight rows and returns the two blocks' sums separately, so the E4M3
//   block scale (which has a mantissa) multiplies the fp32 result once per
//   block: the codes convert straight to unscaled bf16
//   (v_cvt_scalef32_pk_bf16_fp4 at scale 1, two per instruction). About 450
//   vector instructions per pair (SQ_INSTS_VALU on MI355X) against about
//   690 for the scaled decode of the 16-row kernel.
// - k_gemv_mma16 (9 to 16 rows): A rows are the 16 activation rows and each
//   weight is decoded with its block scale to exact bf16 (E2M1 * E4M3 has at
//   most 6 significant bits) before the MFMA; splitting blocks there would
//   double the MFMAs, which measured slower.
//
// Weight loads. In the operand layout one load instruction would touch 64
// bytes of each of 16 rows (a streaming read of that shape ran about 20 %
// slower than contiguous kilobytes on MI355X) and the block scales would take
// many 2-byte loads per pair. Instead a wave loads each tile of its pair as
// the M = 1 kernel does (four contiguous kilobytes, rows 2i and 2i + 1 per
// load, and the tile's 512 scale bytes at 8 bytes per lane) and moves them
// through a wave-private LDS region into the operand layout. Only the wave
// that wrote the region reads it, and a wave's LDS operations complete in
// order.
//
// LDS banks (measured on MI355X with replayed address patterns and the
// SQ_LDS_BANK_CONFLICT counter):
//   - 16-byte reads and writes of a half-wave are free of conflicts when
//     lanes l and l + 16 use the same 16-byte bank group (address bits 4..7)
//     or the same address, and the 16 lane positions use distinct groups (or
//     the same address);
//   - 8-byte reads and writes: 32 lanes a cycle over 64 four-byte banks, one
//     address read by several lanes is a broadcast;
//   - 4-byte accesses are free when the 64 lanes use 64 distinct banks;
//     4- and 2-byte reads that put several lanes on one dword cost about two
//     conflict cycles an instruction.
// Every LDS access of both kernels follows these rules (conflict counter 0).
#include <algorithm>

#include <atomic>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kMRows = 16;                // activation rows per pass (MFMA M)
constexpr int kPairRows = 16;             // weight rows per pair (MFMA N)
constexpr int kTrBytes = 8192 + 1024;    // per wave: one pair's codes and scales
constexpr int kSc1 = 16;                  // buffer cache-policy bit: device scope
constexpr int kCntStride = kWsCounterWords;   // one 128-byte header line per arrival counter

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ f32x2_t fp4x2_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // one v_cvt_pk_bf16_f32; exact: both values have <= 6 significant bits
  // and lie in bf16 range
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 8 elements (word j of a piece) times their block scale, as bf16 operands.
__device__ __forceinline__ bf16x8_t decode8(uint32_t w, float s) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t e = fp4x2_f32(w, i);
    o[i] = pack_bf16(e[0] * s, e[1] * s);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// Two E2M1 codes (byte sel of w) to two exact bf16, unscaled.
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  }
}

// E4M3 byte sel of w to fp32 (exact).
__device__ __forceinline__ float fp8_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

struct MmaArgs {
  const uint16_t* x;   // bf16 [M][K]
  float* ws;           // [C][npairs][16 n][r4][4 m] partials, r4 = row quads of the pass (C > 1; nullptr: atomic
                       // adds into y)
  unsigned* cnt;       // with ws: arrivals per pair block (kCntStride apart, the workspace header, zero
                       // between launches); nullptr: a second kernel adds the partials
  int M, K, C, m0;     // m0: first activation row of this pass
  int nproj;
  int npairs;          // pairs over all projections
  int pairs_per_wg;
  struct Proj {
    const uint8_t* tiles;
    const float* gscale;
    float* y;
    int64_t ldy;
    int32_t N;
    int32_t pair_begin;
  } proj[kMaxProj];
};

__device__ __forceinline__ int proj_of(const struct MmaArgs& a, int pair);

// Row quads of the pass (rows m0 .. min(m0 + 16, M) - 1, four per quad).
__device__ __forceinline__ int row_quads(const MmaArgs& a) { return (min(kMRows, a.M - a.m0) + 3) >> 2; }

// Epilogue of one pair: lane (q, n16) holds rows m0 + 4q + i (i < 4) of
// output column n16 of the pair in v[i]. C == 1: y = gscale * v; with a
// workspace: the unscaled chunk partial; else gscale * v added into y.
__device__ __forceinline__ void pair_out(const MmaArgs& a, int pair, int c, int q, int n16, const f32x4_t& v) {
  if (a.C == 1 || !a.ws) {
    const int p = proj_of(a, pair);
    const int n = 16 * (pair - a.proj[p].pair_begin) + n16;
    const float gs = *a.proj[p].gscale;
    if (n < a.proj[p].N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = a.m0 + 4 * q + i;
        if (m < a.M) {
          float* dst = a.proj[p].y + (int64_t)m * a.proj[p].ldy + n;
          if (a.C == 1)
            *dst = gs * v[i];
          else
            __hip_atomic_fetch_add(dst, gs * v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  } else {
    const int r4 = row_quads(a);
    if (q < r4) {   // rows past M are never read back
      // device-scope store (through to the memory side): the workgroup that
      // adds the partials may run on another XCD
      const __amdgpu_buffer_rsrc_t r = rsrc(a.ws + ((int64_t)c * a.npairs + pair) * 64 * r4, 256 * r4);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (n16 * r4 + q) * 16, 0, kSc1);
    }
  }
}

// Split K inside the launch. Every workgroup (b, c) stores its partials,
// waits for the stores and counts itself in on counter b; the last of the C
// arrivals resets the counter, reads the C partials of its pairs back with
// device-scope loads and writes y = gscale * (their sum in chunk order), so
// the result does not depend on the arrival order.
__device__ __forceinline__ void split_fixup(const MmaArgs& a, int pb, int pe) {
  __shared__ int last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* ctr = a.cnt + (int64_t)blockIdx.x * kCntStride;
    const unsigned n = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = n == (unsigned)(a.C - 1);
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  const int r4 = row_quads(a);
  const int items = (pe - pb) * 16 * r4;   // (pair, n16, m4)
  // One buffer resource over the pass's partials (the launcher keeps them,
  // and the offsets of up to 8 chunks past the last, below 2^31 bytes); an
  // offset past the last chunk reads zeros. A resource built per load (its
  // base differs by chunk and lane) cost about 4 us on the 8-row down 5120 x
  // 17408 at M = 4: 19.9 against 15.9 us.
  const int cstep = a.npairs * 256 * r4;   // bytes per chunk
  const __amdgpu_buffer_rsrc_t rw = rsrc(a.ws, a.C * cstep);
  for (int t = threadIdx.x; t < items; t += blockDim.x) {
    const int m4 = t % r4, pn = t / r4, pair = pb + (pn >> 4), n16 = pn & 15;
    const int p = proj_of(a, pair);
    const int n = 16 * (pair - a.proj[p].pair_begin) + n16;
    if (n >= a.proj[p].N) continue;
    const int off0 = pair * 256 * r4 + (n16 * r4 + m4) * 16;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < a.C; c0 += 8) {
      f32x4_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, off0 + (c0 + i) * cstep, 0, kSc1));
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
    const float gs = *a.proj[p].gscale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = a.m0 + 4 * m4 + i;
      if (m < a.M) a.proj[p].y[(int64_t)m * a.proj[p].ldy + n] = gs * sum[i];
    }
  }
}

// One pair's codes and scale bytes, as loaded: tile T, load i holds piece
// lane % 32 of row 2i + lane / 32; s[T] the tile's scale bytes at 8 * lane.
struct PairFrag {
  uint4 w[2][4];
  uint2 s[2];
};

__device__ __forceinline__ int proj_of(const MmaArgs& a, int pair) {
  int p = 0;
  while (p + 1 < a.nproj && pair >= a.proj[p + 1].pair_begin) ++p;
  return p;
}

// Loads pair `pair` of chunk c. A pair past the workgroup's range [pb, pe)
// gets a zero-byte resource: its loads return zeros without touching memory,
// so every wave runs the same loads.
__device__ __forceinline__ void load_pair(const MmaArgs& a, int pair, int pb, int pe, int c, int lane, PairFrag& f) {
  const int C = a.C;
  const bool v = pair < pe;
  const int p = proj_of(a, v ? pair : pb);
  const int lp = (v ? pair : pb) - a.proj[p].pair_begin;
  const int G = (a.proj[p].N + 7) >> 3;
  const int g0 = 2 * lp;
  const int bytes = !v ? 0 : (g0 + 1 < G ? (C + 1) * kTileBytes : kTileBytes);
  const __amdgpu_buffer_rsrc_t r = rsrc(a.proj[p].tiles + ((int64_t)g0 * C + c) * kTileBytes, bytes);
#pragma unroll
  for (int T = 0; T < 2; ++T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, T * C * kTileBytes + i * 1024 + lane * 16, 0, 2);
      f.w[T][i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const auto sv = __builtin_amdgcn_raw_buffer_load_b64(r, T * C * kTileBytes + kTileCodes + lane * 8, 0, 0);
    f.s[T] = make_uint2(sv[0], sv[1]);
  }
}

constexpr int kXsRow8 = 2048 + 16;   // k_gemv_mma8: staged activation row, padded for conflict-free A reads
constexpr int kZeroWin = 256;        // k_gemv_mma8: zeros read by the A lanes of the other block parity

// At most 8 activation rows (m0 .. m0+7) per launch; grid
// (ceil(npairs / pairs_per_wg), C), block kWaves waves.
__global__ __launch_bounds__(64 * kWaves) void k_gemv_mma8(const MmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[8 * kXsRow8 + kZeroWin];
  __shared__ __attribute__((aligned(16))) uint8_t tr[kWaves * kTrBytes];
  const int lane = threadIdx.x & 63, q = lane >> 4, n16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.y, K = a.K;
  const int pb = blockIdx.x * a.pairs_per_wg;
  const int pe = min(pb + a.pairs_per_wg, a.npairs);

  // Wave-private region in the operand layout. Pair row n (0..15: tile n / 8,
  // row n % 8) keeps its 512 code bytes at 512 n; word w of piece p sits at
  // byte ((w & 1) << 8) + ((((w >> 1) ^ e_n) & 1) << 7) + ((((p >> 2) ^ c_n)
  // & 7) << 4) + 4 (p & 3), e_n = (n & 1) ^ (n >> 3), c_n = (n >> 1) & 7, so
  // word w of four consecutive pieces is one 16-byte read. The reads meet the
  // 16-byte rule of LDS banks (lanes l and l + 16 of a half-wave in the same
  // 16-byte bank group of 256 bytes, or at the same address; the 16 lane
  // positions in distinct groups; measured on MI355X) and each b32 write
  // covers all 64 banks. Its 64 scale bytes sit at 8192 + 64 n, the scale of
  // block 2p + b in 16-byte group (2b + (p >> 4)) ^ s_n at byte p & 15,
  // s_n = ((n >> 1) ^ (n >> 3)) & 3.
  uint8_t* tw = tr + wave * kTrBytes;
  // Write addresses with the fields that depend on (T, i, w) left at zero: a
  // write XORs (w >> 1) ^ T into bit 7 (e_n = h ^ T) and i + 4T into bits 4..6
  // (c_n), then adds the row base 512 (8T + 2i) and (w & 1) << 8; the scales
  // XOR their group field likewise (s_n = (i ^ T) & 3).
  const int h = lane >> 5, l = lane & 31;
  const int wr_code = h * 512 + (h << 7) + ((l >> 2) << 4) + ((l & 3) << 2);
  const int wr_scale = 8192 + h * 64 + l;
  auto transpose_in = [&](const PairFrag& f) {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // row n = 8T + 2i + h, piece l
        const uint32_t wv[4] = {f.w[T][i].x, f.w[T][i].y, f.w[T][i].z, f.w[T][i].w};
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<uint32_t*>(tw + ((wr_code ^ ((((w >> 1) ^ T) << 7) | ((i + 4 * T) << 4))) +
                                             (8 * T + 2 * i) * 512 + ((w & 1) << 8))) = wv[w];
#pragma unroll
        for (int j = 0; j < 2; ++j) {   // scale of row n, block 2l + j: byte 2i + j
          const int byte = 2 * i + j;
          const uint32_t word = byte < 4 ? f.s[T].x : f.s[T].y;
          tw[(wr_scale ^ (((2 * j) ^ ((i ^ T) & 3)) << 4)) + (8 * T + 2 * i) * 64] = (uint8_t)(word >> (8 * (byte & 3)));
        }
      }
    }
  };
  // Lane (q, n) reads word q of the pieces of row n (elements 8q .. 8q+7 of
  // each, block parity q / 2) and the 32 scales of that parity.
  const int en = (n16 & 1) ^ (n16 >> 3), cn = (n16 >> 1) & 7, sn = ((n16 >> 1) ^ (n16 >> 3)) & 3;
  const int beta = q >> 1;
  const int rd_code = n16 * 512 + ((q & 1) << 8) + ((((q >> 1) ^ en) & 1) << 7) + (cn << 4);
  const int rd_scale0 = 8192 + n16 * 64 + (((2 * beta) ^ sn) << 4);
  const int rd_scale1 = 8192 + n16 * 64 + (((2 * beta + 1) ^ sn) << 4);
  // A lane (q, r) feeds MFMA row r = (activation row r % 8, parity r / 8): the
  // activations if its k range has that parity, else zeros. It reads unit u =
  // 16g + 4j + q of its row (see the staging below); the zero lanes read the
  // window at the group that continues their half-wave's row groups.
  const bool a_valid = (n16 >> 3) == beta;
  const int a_base = (a_valid ? (n16 & 7) * kXsRow8 + ((q & 1) << 10) : 8 * kXsRow8) + ((q >> 1) << 4);
  const int a_step2 = a_valid ? 256 : 0;   // per two piece groups (the window repeats every two)

  // activations of chunk c, rows m0 .. m0+7: row m at kXsRow8 * m, 16-byte
  // unit u (elements 8u .. 8u+7) at ((u & 1) << 10) + ((u >> 1) << 4), so the
  // units 8q and 8q + 8 of the A lanes q and q + 1 share a bank group; then
  // the zero window. Thread t stages unit u of row m with lanes l and l + 16
  // on units 2k and 2k + 1 (the same 16-byte rule for the writes). The
  // activation loads go out first and the first pair's weight loads after
  // them, so the staging writes wait for the activations only.
  constexpr int kXUnits8 = 8 * 128 / (64 * kWaves);
  uint4 xv[kXUnits8];
  {
    const int rows = min(8, a.M - a.m0);
#pragma unroll
    for (int s = 0; s < kXUnits8; ++s) {
      const int kk = wave + s * kWaves, L = lane;   // kk: uniform over the wave
      const int m = kk >> 1, u = 64 * (kk & 1) + 32 * (L >> 5) + 2 * (L & 15) + ((L >> 4) & 1);
      // rows past M: a zero-byte resource, zeros
      const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (int64_t)(a.m0 + min(m, rows - 1)) * K, m < rows ? K * 2 : 0);
      const u32x4_t r = __builtin_amdgcn_raw_buffer_load_b128(rx, (c * kChunkK + u * 8) * 2, 0, 0);   // past K: 0
      xv[s] = make_uint4(r[0], r[1], r[2], r[3]);
    }
  }
  PairFrag cur;
  load_pair(a, pb + wave, pb, pe, c, lane, cur);   // in flight while the activations are staged
#pragma unroll
  for (int s = 0; s < kXUnits8; ++s) {
    const int kk = wave + s * kWaves, L = lane;
    const int m = kk >> 1, u = 64 * (kk & 1) + 32 * (L >> 5) + 2 * (L & 15) + ((L >> 4) & 1);
    *reinterpret_cast<uint4*>(xs + m * kXsRow8 + ((u & 1) << 10) + ((u >> 1) << 4)) = xv[s];
  }
  if (threadIdx.x < kZeroWin / 16) *reinterpret_cast<uint4*>(xs + 8 * kXsRow8 + threadIdx.x * 16) = make_uint4(0, 0, 0, 0);
  __syncthreads();

  auto step = [&](int pair, const PairFrag& cf) {
    transpose_in(cf);
    const uint4 sv0 = *reinterpret_cast<const uint4*>(tw + rd_scale0);
    const uint4 sv1 = *reinterpret_cast<const uint4*>(tw + rd_scale1);
    const uint32_t sw[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};   // byte p: piece p
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_barrier(0);
      const uint4 cw = *reinterpret_cast<const uint4*>(tw + (rd_code ^ (g << 4)));
      const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
      const int ab = a_base + (g & 1) * 128 + (g >> 1) * a_step2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // piece p = 4g + j
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fp4x2_bf16(cws[j], e);
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xs + ab + 32 * j);
        const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float sc = fp8_f32(sw[g], j);   // scale of block 2p + q / 2
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, d[i], acc[i]);
      }
    }
    // lane (q, n) holds parity q / 2 of rows 4 (q % 2) + i; the lane 32 apart
    // holds the other parity of the same rows
    f32x4_t tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] = acc[i] + __shfl_xor(acc[i], 32);
    if (q < 2) pair_out(a, pair, c, q, n16, tot);   // rows 4q .. 4q+3
  };
  // Two register sets in turn, with no copy between them: a copy would wait
  // for every outstanding memory operation, the previous pair's partial
  // stores included, before the next loads go out. The next pair's loads
  // overlap this pair's arithmetic.
  PairFrag alt;
  for (int pair = pb + wave; pair < pe; pair += 2 * kWaves) {
    load_pair(a, pair + kWaves, pb, pe, c, lane, alt);
    step(pair, cur);
    if (pair + kWaves >= pe) break;
    load_pair(a, pair + 2 * kWaves, pb, pe, c, lane, cur);
    step(pair + kWaves, alt);
  }
  if (a.cnt && a.C > 1) split_fixup(a, pb, pe);
}

// 9 to 16 activation rows (m0 .. m0+15) per launch; grid and block as above.
__global__ __launch_bounds__(64 * kWaves) void k_gemv_mma16(const MmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kMRows * kChunkK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t tr[kWaves * kTrBytes];
  const int lane = threadIdx.x & 63, q = lane >> 4, n16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.y, K = a.K;
  const int pb = blockIdx.x * a.pairs_per_wg;
  const int pe = min(pb + a.pairs_per_wg, a.npairs);
  const int rr = n16 & 7;

  // Lane (q, n) takes the 16-byte piece P = 16 (q % 2) + 2t + q / 2 (t =
  // 0..7) of weight row n and feeds its elements 8j .. 8j+7 to MFMA (t, j);
  // the A lane (q, m) reads the matching activations x[m][32P + 8j ..]. In
  // each half-wave the lanes n and n + 16 thus read pieces P and P + 16 of
  // one row. Every LDS access below follows the 16-byte bank rule (lanes l
  // and l + 16 of a half-wave in one bank group or at one address, the 16
  // lane positions in distinct groups) or the 8-byte one (32 lanes a cycle,
  // 64 banks, one address broadcasts; 4- and 2-byte reads with several lanes
  // on one dword measured about two conflict cycles each):
  //   - codes: row n (0..15 over the pair) at 512 n, piece P at ((P / 16)
  //     << 8) + (((P % 16) ^ n) << 4): written from the loads as they come
  //     (lane (h, l) holds piece l), read as above;
  //   - activations: row m at 2048 m, 16-byte unit u at ((u / 64) << 10) +
  //     (((u % 64) ^ m) << 4);
  //   - scales: tile T's 512 bytes in 8-byte slots (row parity h, block
  //     pair l) at 8192 + 512 T + 256 h + 8 (l ^ (2T + h)), written 8
  //     bytes a lane as loaded; a lane reads its whole slot and keeps bytes
  //     2i and 2i + 1 (i = rr / 2: blocks 2P and 2P + 1 of its row).
  uint8_t* tw = tr + wave * kTrBytes;
  auto transpose_in = [&](const PairFrag& f) {
    const int h = lane >> 5, l = lane & 31;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 8 * T + 2 * i + h;
        *reinterpret_cast<uint4*>(tw + n * 512 + ((l >> 4) << 8) + (((l & 15) ^ n) << 4)) = f.w[T][i];
      }
      *reinterpret_cast<uint2*>(tw + 8192 + T * 512 + h * 256 + ((l ^ (2 * T + h)) << 3)) = f.s[T];
    }
  };
  auto xaddr = [](int m, int u) { return m * 2048 + ((u >> 6) << 10) + (((u & 63) ^ m) << 4); };
  // activations of chunk c, rows m0 .. m0+15: half-wave e (of 64) stages
  // row e / 4, units 16 (e % 4) + l % 16 and 64 more (lanes l and l + 16).
  // The activation loads go out before the first pair's weight loads, so the
  // staging writes wait for the activations only.
  constexpr int kXUnits16 = kMRows * 128 / (64 * kWaves);
  uint4 xv[kXUnits16];
  {
    const int rows = min(kMRows, a.M - a.m0);
#pragma unroll
    for (int s = 0; s < kXUnits16; ++s) {
      const int L = lane, e = ((wave + s * kWaves) << 1) + (L >> 5);
      const int m = (wave + s * kWaves) >> 1, u = (((L >> 4) & 1) << 6) + ((e & 3) << 4) + (L & 15);   // m = e / 4, uniform
      // rows past M: a zero-byte resource, zeros
      const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (int64_t)(a.m0 + min(m, rows - 1)) * K, m < rows ? K * 2 : 0);
      const u32x4_t r = __builtin_amdgcn_raw_buffer_load_b128(rx, (c * kChunkK + u * 8) * 2, 0, 0);   // past K: 0
      xv[s] = make_uint4(r[0], r[1], r[2], r[3]);
    }
  }
  PairFrag cur;
  load_pair(a, pb + wave, pb, pe, c, lane, cur);   // in flight while the activations are staged
#pragma unroll
  for (int s = 0; s < kXUnits16; ++s) {
    const int L = lane, e = ((wave + s * kWaves) << 1) + (L >> 5);
    const int m = (wave + s * kWaves) >> 1, u = (((L >> 4) & 1) << 6) + ((e & 3) << 4) + (L & 15);
    *reinterpret_cast<uint4*>(xs + xaddr(m, u)) = xv[s];
  }
  __syncthreads();

  auto step = [&](int pair, const PairFrag& cf) {
    // two accumulators (even and odd pieces) halve the dependent MFMA chain
    f32x4_t acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    transpose_in(cf);
    const int T = n16 >> 3;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // one piece at a time: keeps the compiler from hoisting every operand
      __builtin_amdgcn_sched_barrier(0);
      const int P = ((q & 1) << 4) + 2 * t + (q >> 1);
      const uint4 wv = *reinterpret_cast<const uint4*>(tw + n16 * 512 + ((P >> 4) << 8) + (((P & 15) ^ n16) << 4));
      const uint2 sv = *reinterpret_cast<const uint2*>(tw + 8192 + T * 512 + (rr & 1) * 256 + ((P ^ (2 * T + (rr & 1))) << 3));
      const uint32_t sc = (rr & 4 ? sv.y : sv.x) >> ((rr & 2) << 3);   // bytes 2i, 2i + 1 of the slot, i = rr / 2
      const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
      const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t b = decode8(word(wv, j), j < 2 ? s0 : s1);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xs + xaddr(n16, 4 * P + j));
        acc2[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b, acc2[t & 1], 0, 0, 0);
      }
    }
    const f32x4_t acc = acc2[0] + acc2[1];
    // lane (q, n16) holds D[m = 4q + i][n = n16]
    pair_out(a, pair, c, q, n16, acc);
  };
  // two register sets in turn, as in k_gemv_mma8
  PairFrag alt;
  for (int pair = pb + wave; pair < pe; pair += 2 * kWaves) {
    load_pair(a, pair + kWaves, pb, pe, c, lane, alt);
    step(pair, cur);
    if (pair + kWaves >= pe) break;
    load_pair(a, pair + 2 * kWaves, pb, pe, c, lane, cur);
    step(pair + kWaves, alt);
  }
  if (a.cnt && a.C > 1) split_fixup(a, pb, pe);
}

// y[m][n] = gscale * sum over chunks (in order) of the partials. A thread
// owns four rows (m, ..., m + 3) of one output column: one 16-byte partial
// per chunk, P chunks loaded together (indices past the last chunk are
// clamped to it and their values dropped), then added in chunk order. P is
// the smallest of 8, 16, 24, 32 that covers C (one round of loads up to 32
// chunks). 64-thread workgroups spread a small launch over the CUs (the
// 16-row down projection 5120 x 17408: 320 workgroups instead of 80).
// grid: npairs * 16 * ceil(rows / 4) threads, rows = min(16, M - m0).
template <int P>
__global__ __launch_bounds__(64) void k_reduce(const MmaArgs a) {
  const int r4 = row_quads(a);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (pair, n16, m4)
  if (t >= (int64_t)a.npairs * 16 * r4) return;
  const int m4 = (int)(t % r4);
  const int pn = (int)(t / r4), pair = pn >> 4, n16 = pn & 15;
  int p = 0;
  while (p + 1 < a.nproj && pair >= a.proj[p + 1].pair_begin) ++p;
  const int n = 16 * (pair - a.proj[p].pair_begin) + n16;
  if (n >= a.proj[p].N) return;
  const float gs = *a.proj[p].gscale;
  const int64_t cstride = (int64_t)a.npairs * 16 * r4;   // in f32x4
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.ws) + ((int64_t)pair * 16 + n16) * r4 + m4;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.C; c0 += P) {
    f32x4_t v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = src[(int64_t)min(c0 + i, a.C - 1) * cstride];
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (c0 + i < a.C) s += v[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = a.m0 + 4 * m4 + i;
    if (m < a.M) a.proj[p].y[(int64_t)m * a.proj[p].ldy + n] = gs * s[i];
  }
}

// Workgroups of the kernel resident per CU (LDS-bound: 3 for k_gemv_mma8,
// 2 for k_gemv_mma16 on MI355X), cached per device; 0 if unknown.
template <bool EIGHT>
int resident_per_cu() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, EIGHT ? k_gemv_mma8 : k_gemv_mma16, 64 * kWaves, 0) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Pairs per workgroup. The four waves of a workgroup take its pairs in
// turn, so a workgroup lasts about ceil(ppw / 4) pair steps, and the grid
// runs in ceil(workgroups / slots) rounds (slots: workgroups resident on the
// whole device). The choice minimises rounds x steps over ppw = 4 .. 32.
// Ties go to two steps per wave (ppw 8) for the 8-row kernel, else to the
// larger ppw. Sweeps on MI355X (graph-timed, rotating weights): at 16 rows
// gate_up 34816 x 5120 24 pairs (30.5 us against 32.6 with 8), down 5120 x
// 17408 12 (19.8 against 20.1), LM head 151936 x 1024 20 (25.5 against 28.1
// with 8); at 8 rows gate_up 8 (27.0 against 28.7 with 16), down 8 (18.5
// against 19.5 with 4), LM head 8 (23.4 against 23.8 with 16).
int pick_pairs_per_wg(int64_t pairs, int C, int64_t slots, bool eight) {
  if (slots <= 0) return C <= 8 ? 16 : 8;
  int best = 16;
  int64_t best_cost = -1;
  for (int p = 4; p <= 32; p += 4) {
    const int64_t wgs = (pairs + p - 1) / p * C;
    const int64_t cost = (wgs + slots - 1) / slots * (p / 4);
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && !(eight && best == 8))) {
      best_cost = cost;
      best = p;
    }
  }
  return best;
}

// y[m][n] = 0 for rows m0 .. m0 + rows - 1 of every projection (before the
// atomic adds of a multi-chunk pass without a workspace). grid.y: projection.
__global__ __launch_bounds__(256) void k_zero_rows(const MmaArgs a, int rows) {
  const auto& pj = a.proj[blockIdx.y];
  const int64_t n_all = (int64_t)rows * pj.N;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n_all; t += (int64_t)gridDim.x * 256) {
    const int64_t m = t / pj.N, n = t - m * pj.N;
    pj.y[(a.m0 + m) * pj.ldy + n] = 0.0f;
  }
}

MmaArgs mma_args(const GemvArgs& g) {
  MmaArgs a{};
  a.x = g.x;
  a.M = g.M;
  a.K = g.K;
  a.C = g.C;
  a.nproj = g.nproj;
  int64_t pairs = 0;
  for (int i = 0; i < g.nproj; ++i) {
    a.proj[i].tiles = g.proj[i].tiles;
    a.proj[i].gscale = g.proj[i].gscale;
    a.proj[i].y = g.proj[i].y;
    a.proj[i].ldy = g.proj[i].ldy;
    a.proj[i].N = g.proj[i].N;
    a.proj[i].pair_begin = (int32_t)pairs;
    pairs += (g.proj[i].N + kPairRows - 1) / kPairRows;
  }
  a.npairs = pairs > (int64_t(1) << 26) ? -1 : (int)pairs;
  return a;
}

int pairs_per_wg_for(const MmaArgs& a, bool eight) {
  const int64_t ncu = device_cu_count();
  return pick_pairs_per_wg(a.npairs, a.C, ncu * (eight ? resident_per_cu<true>() : resident_per_cu<false>()), eight);
}

}  // namespace

size_t gemv_mma_partial_bytes(const GemvArgs& g) {
  if (g.C <= 1) return 0;
  const MmaArgs a = mma_args(g);
  if (a.npairs < 0) return 0;
  return (size_t)a.C * (size_t)a.npairs * 256 * sizeof(float);
}

hipError_t launch_gemv_mma(const GemvArgs& g, float* partials, unsigned* counters, hipStream_t s, int ppw) {
  MmaArgs a = mma_args(g);
  if (a.npairs < 0) return hipErrorInvalidValue;
  const int64_t pairs = a.npairs;
  const bool use_ws = a.C > 1 && partials;
  if (use_ws) a.ws = partials;
  for (int m0 = 0; m0 < g.M; m0 += kMRows) {
    a.m0 = m0;
    const bool eight = g.M - m0 <= 8;
    a.pairs_per_wg = ppw > 0 ? ppw : pairs_per_wg_for(a, eight);
    const int64_t wgx = (pairs + a.pairs_per_wg - 1) / a.pairs_per_wg;
    const int rows = std::min(kMRows, g.M - m0);
    if (a.C > 1 && !use_ws) {
      int64_t most = 0;
      for (int i = 0; i < a.nproj; ++i) most = std::max<int64_t>(most, (int64_t)rows * a.proj[i].N);
      const int64_t blocks = std::min<int64_t>((most + 255) / 256, 4096);
      hipLaunchKernelGGL(k_zero_rows, dim3((unsigned)blocks, (unsigned)a.nproj), dim3(256), 0, s, a, rows);
    }
    // In-launch fixup for passes of at most 8 rows (its arrivals need one
    // header counter per pair block, and its loads address the pass's
    // partials with 32-bit offsets, up to 8 chunks past the last). MI355X,
    // graph-timed: fused gate_up 2 x 17408 x 5120 at M = 4 27.5 against 29.3
    // us with the second kernel, M = 8 29.4 against 30.3; at M = 16 the last
    // workgroups' sums of 16 rows form a tail (38.7 against 33.9 us), so
    // those passes keep the kernel.
    const bool small_ws = ((int64_t)a.C + 8) * pairs * 256 * ((rows + 3) / 4) < (int64_t(1) << 31);
    a.cnt = use_ws && eight && counters && wgx <= kWsCounters && small_ws ? counters : nullptr;
    const dim3 grid((unsigned)wgx, (unsigned)a.C), block(64 * kWaves);
    if (eight)
      hipLaunchKernelGGL(k_gemv_mma8, grid, block, 0, s, a);
    else
      hipLaunchKernelGGL(k_gemv_mma16, grid, block, 0, s, a);
    if (use_ws && !a.cnt) {
      const int64_t n = pairs * 16 * ((rows + 3) / 4);
      const dim3 rg((unsigned)((n + 63) / 64)), rb(64);
      if (a.C <= 8)
        hipLaunchKernelGGL(k_reduce<8>, rg, rb, 0, s, a);
      else if (a.C <= 16)
        hipLaunchKernelGGL(k_reduce<16>, rg, rb, 0, s, a);
      else if (a.C <= 24)
        hipLaunchKernelGGL(k_reduce<24>, rg, rb, 0, s, a);
      else
        hipLaunchKernelGGL(k_reduce<32>, rg, rb, 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp4

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
// tile, BN = 256 or 128; wave (wm, wn) of the 2 x 2 wave grid owns
// 128 x BN/2 as 4 x NJ v_mfma_f32_32x32x16_bf16 tiles. K advances in steps
// of 64, each split in four 16-deep MFMA slices.
//
// Operands. Activations go global -> registers -> LDS (two 32 KB stages,
// one barrier per step) -> MFMA operand registers. Weights skip LDS: each
// wave loads its own columns' packed codes straight from the tiled layout
// into registers and decodes the slice it is about to use while the MFMAs
// of the previous slice run. This keeps the LDS traffic (the bound of a
// bf16 GEMM at this tile size) to the activations alone. The dot product
// is taken over a permuted K order, the same for both operands: lane half h
// of slice s covers K offsets 32h + 8s .. 32h + 8s + 7 of the step, so a
// lane's weight codes for a whole step are one 16-byte piece of one row.
//
// Pipelining. Activation loads (L2 hits: one XCD shares a slab) are issued
// at the start of the step before their MFMAs and written into the other
// LDS stage in its second half; weight loads are issued in the middle of the
// step before last. The activation rows are
// 128 bytes, eight 16-byte chunks, chunk j of row r at slot j ^ swz(r), so
// that operand reads and stores never meet in a bank.
//
// Order. Workgroups go round-robin over the 8 XCDs; tile t = (XCD, rank)
// is mapped so that one XCD works through all output tiles of one 256-row
// activation slab (2.6 MB at K = 5120, kept in that XCD's 4 MB L2) while
// every XCD streams the weights.
//
// Loads use buffer resources: activation rows past M, activation columns
// past K and weight row groups past N read as zeros without touching memory;
// stores drop rows past M and columns past N the same way.
#include <algorithm>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int BM = 256, BK = 64;
constexpr int kStage = BM * BK * 2;      // 32 KB of activations per stage
constexpr int kSmem = 2 * kStage;

// 16-byte chunk slot of chunk j in row r of a stage: j ^ swz(r). Rows are
// 128 bytes; swz is a bijection on every 8 consecutive rows, and on the even
// (odd) rows of every 16, so the operand reads (8 or 16 lanes on 8 or 16
// consecutive rows) never meet in a bank.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ uint4 u4(u32x4_t v) { return make_uint4(v[0], v[1], v[2], v[3]); }

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

// Eight codes (word `slice` of a 16-byte piece) as a bf16x8 MFMA operand.
// `sc` is the aligned dword holding the piece's two block scales, in bytes
// 0, 1 (hi false) or 2, 3 (hi true); slices 0, 1 use the first scale, 2, 3
// the second. Byte selects keep every operation on the loaded dword inside
// the decode, so none is hoisted next to its load (which would wait there).
__device__ __forceinline__ bf16x8_t decode8(const uint4& piece, uint32_t sc, bool hi, int slice) {
  float s;
  if (slice < 2) {
    const float lo_s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0), hi_s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 2);
    s = hi ? hi_s : lo_s;
  } else {
    const float lo_s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 1), hi_s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 3);
    s = hi ? hi_s : lo_s;
  }
  const uint32_t w = word(piece, slice);
  const uint4 o = make_uint4(dec2(w, 0, s), dec2(w, 1, s), dec2(w, 2, s), dec2(w, 3, s));
  return __builtin_bit_cast(bf16x8_t, o);
}

// This thread's activations of one step: rows ra + 32i (i < 8), chunk ac.
struct ARegs {
  uint4 a[8];
};
// This lane's weights of one step: piece (lane / 32) of row (lane % 32) of
// each of the wave's NJ 32-column tiles, and the dword holding the piece's
// two block scales.
template <int NJ>
struct BRegs {
  uint4 w[NJ];
  uint32_t sc[NJ];
};
// MFMA operands of one slice.
template <int NJ>
struct Frags {
  bf16x8_t a[4], b[NJ];
};

// Deals the instructions of a scheduling region out around its NMFMA MFMAs:
// after MFMA i come up to kValuPerMfma VALU operations, then one LDS read
// (i < NDSR), one LDS write (i < NDSW) and one global load (i < NVMEM).
constexpr int kValuPerMfma = 5;
template <int NMFMA, int NDSR, int NDSW, int NVMEM>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // VALU
    if (i < NDSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i < NDSW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (i < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

template <int BN>
__global__ __launch_bounds__(256, 1) void k_prefill(float* __restrict__ y, const uint16_t* __restrict__ x,
                                                    const uint8_t* __restrict__ tiles,
                                                    const float* __restrict__ gscale, int M, int N, int K,
                                                    int m_tiles, int n_tiles, int per_xcd) {
  constexpr int NJ = BN / 64;   // 32-column MFMA tiles per wave
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int id = blockIdx.x;
  const int lin = (id & 7) * per_xcd + (id >> 3);   // XCD-contiguous tile index
  if (lin >= m_tiles * n_tiles) return;
  const int m0 = (lin / n_tiles) * BM, n0 = (lin % n_tiles) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int C = (K + kChunkK - 1) / kChunkK;
  const int G = (N + 7) >> 3;
  const int KT = (K + BK - 1) / BK;

  // activations: thread -> rows ra + 32i (i < 8), 16-byte chunk ac of the step
  const int ra = tid >> 3, ac = tid & 7;
  const int mrows = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + (int64_t)m0 * K, mrows * K * 2);
  // weights: lane -> row wn * BN/2 + 32j + l32 of the tile (j < NJ), piece lh
  const int g0 = n0 >> 3;
  const int ngroups = min(BN / 8, G - g0);
  const __amdgpu_buffer_rsrc_t rw = rsrc(tiles + (int64_t)g0 * C * kTileBytes, ngroups * C * kTileBytes);
  // the scale pair of row r sits at an offset = 2 (mod 4) when (r / 2) is odd
  const bool sc_hi = (tile_scale_offset(l32 & 7, 0) & 2) != 0;

  // Loads of steps past the end go through an empty resource (zeros, no
  // memory access), so every load is unconditional and the compiler can count
  // outstanding loads exactly.
  const __amdgpu_buffer_rsrc_t rnull = rsrc(x, 0);
  auto load_a = [&](int kt, ARegs& r) {
    const int k0 = kt * BK;
    const __amdgpu_buffer_rsrc_t rs = kt < KT ? rx : rnull;
    // a chunk past K (ragged last step) gets bit 31 set: an offset past the
    // resource (an arithmetic mask, not a select, which the compiler turns
    // into branches around the loads)
    const uint32_t oob = (uint32_t)((K - 1 - k0 - ac * 8) >> 31) << 31;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r.a[i] = u4(__builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(((ra + 32 * i) * K + k0 + ac * 8) * 2) | oob, 0, 0));
  };
  auto load_b = [&](int kt, BRegs<NJ>& r) {
    const int k0 = kt * BK;
    const int c = k0 / kChunkK, p = (k0 % kChunkK) / 32 + lh;
    const __amdgpu_buffer_rsrc_t rs = kt < KT ? rw : rnull;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nr = wn * (BN / 2) + j * 32 + l32;
      const int tb = ((nr >> 3) * C + c) * kTileBytes;
      r.w[j] = u4(__builtin_amdgcn_raw_buffer_load_b128(rs, tb + (nr & 7) * 512 + p * 16, 0, 0));
      r.sc[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (tb + tile_scale_offset(nr & 7, 2 * p)) & ~3, 0, 0);
    }
  };
  // quarter q (< 4) of writing a step's activations into an LDS stage
  auto store_a = [&](const ARegs& r, int stage, int q) {
    uint8_t* As = smem + stage * kStage;
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) {
      const int row = ra + 32 * i;
      *reinterpret_cast<uint4*>(As + row * 128 + ((ac ^ swz(row)) * 16)) = r.a[i];
    }
  };
  // slice s: lane half h covers K offsets 32h + 8s .. + 7 of the step, which
  // is chunk 4h + s of the activation row and word s of the weight piece
  auto read_a = [&](int stage, int s, Frags<NJ>& f) {
    const uint8_t* As = smem + stage * kStage;
    const int lchunk = 4 * lh + s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + l32;
      f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + r * 128 + ((lchunk ^ swz(r)) * 16));
    }
  };
  auto decode_b = [&](const BRegs<NJ>& r, int s, Frags<NJ>& f) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b[j] = decode8(r.w[j], r.sc[j], sc_hi, s);
  };

  f32x16_t acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mma = [&](const Frags<NJ>& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };

  // Step kt uses LDS stage kt % 2 and weight register set kt % 2. On entry
  // the weight operands of its slice 0 are decoded (in f0.b). It reads its
  // slice 0 activation operands and issues the activation loads of step
  // kt + 1 (one register set; they come from L2), then runs its four slices;
  // alongside the MFMAs of slice s it reads the activation operands of slice
  // s + 1 and decodes its weight operands, in slices 2 and 3 writes the step
  // kt + 1 activations into the other stage, and in slice 3 (its weight set
  // decoded) loads the weights of step kt + 2 and decodes slice 0 of step
  // kt + 1. One barrier per step.
  //
  // Scheduling: a wave issues in order, so an MFMA queued behind a long run
  // of decode arithmetic leaves the matrix core idle. Each slice is its own
  // scheduling region (sched_barrier) whose instructions are dealt out
  // around the MFMAs (sched_group_barrier): after every MFMA a few VALU
  // operations and at most one LDS or global memory instruction, which the
  // 32-cycle MFMA covers.
  Frags<NJ> f0, f1;
  ARegs an;
  auto step = [&](int kt, BRegs<NJ>& b_mine, const BRegs<NJ>& b_next, int stage) {
    read_a(stage, 0, f0);
    load_a(kt + 1, an);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    read_a(stage, 1, f1);
    decode_b(b_mine, 1, f1);
    interleave<4 * NJ, 4, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    read_a(stage, 2, f0);
    decode_b(b_mine, 2, f0);
    interleave<4 * NJ, 4, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    read_a(stage, 3, f1);
    decode_b(b_mine, 3, f1);
    store_a(an, stage ^ 1, 0);
    store_a(an, stage ^ 1, 1);
    interleave<4 * NJ, 4, 4, 0>();
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    load_b(kt + 2, b_mine);
    decode_b(b_next, 0, f0);
    store_a(an, stage ^ 1, 2);
    store_a(an, stage ^ 1, 3);
    interleave<4 * NJ, 0, 4, 2 * NJ>();
    __syncthreads();
  };

  // prologue: step 0's activations in stage 0, weights of steps 0 and 1 in
  // registers
  BRegs<NJ> b0, b1;
  load_a(0, an);
  load_b(0, b0);
  load_b(1, b1);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_a(an, 0, q);
  decode_b(b0, 0, f0);
  __syncthreads();

  // past the end the loads give zeros and go into a stage no step reads
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(kt, b0, b1, 0);
    step(kt + 1, b1, b0, 1);
  }
  if (kt < KT) step(kt, b0, b1, 0);   // odd step count: the last step sits in stage 0

  // epilogue: lane l of a 32x32 tile holds column l % 32 and rows
  // 8(e/4) + 4(l/32) + e%4 (e < 16). Buffer stores drop rows past M (past
  // the resource) and columns past N (bit 31 set in the offset).
  const float gs = *gscale;
  const __amdgpu_buffer_rsrc_t ry = rsrc(y + (int64_t)m0 * N, mrows * N * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn * (BN / 2) + j * 32 + l32;
      const uint32_t oobn = (uint32_t)((N - 1 - n) >> 31) << 31;
      const int r0 = wm * 128 + i * 32 + lh * 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = r0 + (e >> 2) * 8 + (e & 3);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gs * acc[i][j][e]), ry,
                                              (uint32_t)((r * N + n) * 4) | oobn, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // one tile's values live at a time
    }
}

}  // namespace

hipError_t launch_prefill(float* y, const uint16_t* x, const uint8_t* tiles, const float* gscale, int64_t M,
                          int64_t N, int64_t K, hipStream_t s) {
  // buffer offsets are 32-bit: one 256-row slab of activations, of outputs
  // and of weights must each stay below 2 GB
  const int64_t C = chunks_of(K);
  if ((int64_t)BM * K * 2 >= (int64_t(1) << 31) || (int64_t)BM * N * 4 >= (int64_t(1) << 31) ||
      (int64_t)(256 / 8) * C * kTileBytes >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  const int64_t mt = (M + BM - 1) / BM;
  // 256 x 256 tiles do twice the MFMA work per LDS and load byte of 256 x 128
  // tiles; take them unless their last round of workgroups over the 256
  // compute units is much emptier (the time is about rounds x tile time)
  const int64_t nt256 = (N + 255) / 256, nt128 = (N + 127) / 128;
  const int64_t rounds256 = (mt * nt256 + 255) / 256, rounds128 = (mt * nt128 + 255) / 256;
#ifdef PREFILL_WIDE_RULE
  const bool wide = PREFILL_WIDE_RULE;
#else
  const bool wide = 20 * rounds256 <= 13 * rounds128;
#endif
  const int64_t nt = wide ? nt256 : nt128;
  const int64_t total = mt * nt;
  if (total > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int64_t per_xcd = (total + 7) / 8;
  if (wide)
    hipLaunchKernelGGL(k_prefill<256>, dim3((unsigned)(8 * per_xcd)), dim3(256), kSmem, s, y, x, tiles, gscale,
                       (int)M, (int)N, (int)K, (int)mt, (int)nt, (int)per_xcd);
  else
    hipLaunchKernelGGL(k_prefill<128>, dim3((unsigned)(8 * per_xcd)), dim3(256), kSmem, s, y, x, tiles, gscale,
                       (int)M, (int)N, (int)K, (int)mt, (int)nt, (int)per_xcd);
  return hipGetLastError();
}

}  // namespace fp4

// NVFP4 quantisation (load time) and canonical -> tiled re-tiling.
//
// The engine shrinks every weight once when the model is loaded (page "How
// imp turns a model file into words", Part one) and keeps the transformed
// weights (page "imp" README, the weight-cache note). This file does both on
// the GPU. The quantised bytes are unique, so each fp32 step below is one
// IEEE operation rounded to nearest-even: divisions are correctly rounded
// (-fhip-fp32-correctly-rounded-divide-sqrt) and this file is compiled with
// -ffp-contract=off so that no multiply is fused into an add.
//
// Sources: bf16 weights, or a checkpoint released in FP8 (the imp README's
// quantiser builds NVFP4 weights from BF16 or FP8 releases): OCP E4M3 codes
// and one fp32 dequantisation scale per tensor, element value
// E4M3(code) * scale rounded once to fp32. The rule is the same for both.
//
// Launch sequence for one tensor, all on the caller's stream:
//   1. k_amax_init   slot := 0
//   2. k_amax        slot := max over W of the magnitude bits (atomic max;
//                    bf16 and E4M3 magnitudes order like their bit patterns,
//                    and rounding a product by a scale keeps that order)
//   3. k_encode      one thread per 16-element block: block scale, codes, pack
//   4. k_finalize    slot := amax / 2688  (the tensor scale gscale)
#include "fp4_internal.h"

namespace fp4 {
namespace {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 (>= 0) -> E4M3 code, nearest-even, saturating at 448 (code 0x7E).
// Normal results: round the 24-bit significand to 4 bits. Subnormal results
// (below 2^-6): the code is the integer nearest to s * 2^9 (ties to even),
// where 8 means the smallest normal, code 0x08.
__device__ __forceinline__ uint32_t e4m3_code(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  const uint32_t u = __float_as_uint(s);
  const int e = (int)(u >> 23) - 127;
  if (e >= -6) {
    const uint32_t sig = (u & 0x7FFFFFu) | 0x800000u;
    uint32_t q = sig >> 20;                 // 8..15
    const uint32_t rem = sig & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    uint32_t E = (uint32_t)(e + 7);
    if (q == 16u) { q = 8u; ++E; }
    return (E << 3) | (q - 8u);
  }
  return (uint32_t)__builtin_rintf(s * 512.0f);
}

// The two sources. Each gives the 16 fp32 values of a block and their
// largest magnitude, and turns the amax slot (largest magnitude bits) into
// the tensor amax.
struct SrcBf16 {
  const uint16_t* W;
  static constexpr int kPerVec = 8;   // elements per 16-byte load
  __device__ static uint32_t vec_max(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    return m;
  }
  __device__ float amax(uint32_t slot) const { return bf16_bits_to_float(slot); }
  // the 16 elements of the block at element offset off: values and largest magnitude
  __device__ float block(int64_t off, float (&w)[16]) const {
    const uint4* src = reinterpret_cast<const uint4*>(W + off);
    const uint4 a = src[0], c = src[1];
    const uint32_t d[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    uint32_t bm = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[2 * j] = bf16_bits_to_float(d[j] & 0xFFFFu);
      w[2 * j + 1] = bf16_bits_to_float(d[j] >> 16);
      bm = max(bm, max(d[j] & 0x7FFFu, (d[j] >> 16) & 0x7FFFu));
    }
    return bf16_bits_to_float(bm);
  }
};

struct SrcFp8 {
  const uint8_t* W;
  const float* scale;   // device fp32, the checkpoint's dequantisation multiplier
  static constexpr int kPerVec = 16;
  __device__ static uint32_t vec_max(const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) m = max(m, (w[j] >> (8 * b)) & 0x7Fu);
    return m;
  }
  // |RN(e * s)| = RN(|e| * |s|) grows with |e|: the largest code gives the amax
  __device__ float amax(uint32_t slot) const {
    return __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)slot, 0), fabsf(*scale));
  }
  __device__ float block(int64_t off, float (&w)[16]) const {
    const uint4 v = *reinterpret_cast<const uint4*>(W + off);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    const float s = *scale;
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[4 * j + 0] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)d[j], 0), s);
      w[4 * j + 1] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)d[j], 1), s);
      w[4 * j + 2] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)d[j], 2), s);
      w[4 * j + 3] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)d[j], 3), s);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(w[j]));
    return m;
  }
};

__global__ void k_amax_init(uint32_t* slot) { *slot = 0u; }

// Grid-stride over 16-byte vectors, four loads in flight per thread; the
// workgroup's maximum meets the others in ONE atomic per workgroup (an
// atomic per wave queued 16K atomics on the one word and dominated the pass).
template <class Src>
__global__ __launch_bounds__(256) void k_amax(const uint4* __restrict__ W, int64_t nvec, uint32_t* slot) {
  __shared__ uint32_t red[4];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const uint4 a = W[i], b = W[i + stride], c = W[i + 2 * stride], d = W[i + 3 * stride];
    m = max(m, max(max(Src::vec_max(a), Src::vec_max(b)), max(Src::vec_max(c), Src::vec_max(d))));
  }
  for (; i < nvec; i += stride) m = max(m, Src::vec_max(W[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m != 0u) atomicMax(slot, m);
  }
}

// Four E2M1 code bytes (8 elements, the even one in the low nibble) of the
// fp32 quotients v[0..7]. The rule: the magnitude code counts the decision
// thresholds |v| passes, the midpoints between the eight magnitudes, where
// the even code wins a tie (> at 0.25, 1.25, 2.5 and 5; >= at 0.75, 1.75 and
// 3.5), so |v| > 5 saturates to 6; the sign bit of v, zeros included, is
// bit 3. v_cvt_scalef32_pk_fp4_f32 with scale 1.0 computes exactly that: on
// MI355X it agreed with the threshold formula on all 2^32 - 2^24 non-NaN fp32
// inputs (an exhaustive check), at one instruction per two elements instead
// of about fifteen per element.
__device__ __forceinline__ uint32_t e2m1_codes8(const float* v) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
}

// One thread per 16-element block; a workgroup covers 256 blocks of one row
// (its row and segment come from the workgroup index, so no thread divides by
// the row length). For the tiled layout rows and blocks run over the padded
// space (G*8 rows x C*64 blocks) so padding is written as zeros.
// grid: rows * segs workgroups, segs = ceil(bpr / 256); block 256.
template <class Src>
__global__ __launch_bounds__(256) void k_encode(const Src src, int64_t N, int64_t K, int tiled,
                                                uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
                                                const uint32_t* __restrict__ slot) {
  const int64_t kb = K / 16;                          // blocks per row
  const int64_t C = chunks_of(K);
  const int64_t bpr = tiled ? C * 64 : kb;            // blocks per (padded) row
  const uint32_t segs = (uint32_t)((bpr + 255) / 256);
  const uint32_t wg = blockIdx.x;                     // uniform: scalar arithmetic
  const int64_t n = wg / segs;
  const int64_t b = (int64_t)(wg - (uint32_t)n * segs) * 256 + threadIdx.x;
  if (b >= bpr) return;

  uint32_t sc = 0, lo = 0, hi = 0;  // scale code, packed bytes 0..3 and 4..7
  const float amax = src.amax(*slot);
  if (n < N && b < kb && amax != 0.0f) {
    const float gscale = amax / 2688.0f;
    float w[16];
    const float bamax = src.block(n * K + b * 16, w);
    const float s = (bamax / 6.0f) / gscale;
    sc = e4m3_code(s);
    const float s_dec = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);   // OCP E4M3 decode
    if (s_dec != 0.0f) {
      const float d = __fmul_rn(s_dec, gscale);
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = w[j] / d;
      lo = e2m1_codes8(v);
      hi = e2m1_codes8(v + 8);
    }
  }
  if (!tiled) {
    *reinterpret_cast<uint2*>(packed + n * (K / 2) + b * 8) = make_uint2(lo, hi);
    scales[n * kb + b] = (uint8_t)sc;
  } else {
    // tiled: codes and scale go into the one tile buffer (`packed`)
    const int64_t g = n / kGroupRows, r = n % kGroupRows;
    const int64_t c = b / 64, l = (b % 64) / 2, j = b % 2;
    uint8_t* tile = packed + (g * C + c) * kTileBytes;
    *reinterpret_cast<uint2*>(tile + r * 512 + l * 16 + j * 8) = make_uint2(lo, hi);
    tile[tile_scale_offset((int)r, (int)(b % 64))] = (uint8_t)sc;
  }
}

// MXFP4 (OCP MX v1.0): one thread per 32-element block, one pass (no tensor
// scale). Shared exponent floor(log2(amax)) - 2 clamped to [-127, 127]: the
// bf16 magnitude's exponent field gives floor(log2) directly (a subnormal
// amax is below 2^-126, so its block clamps to -127). The elements are
// multiplied by 2^-shared (exact: a power of two, and |w| 2^-shared < 8)
// and rounded to E2M1 as in k_encode. A block with amax 0 keeps scale 0 and
// codes 0. Tiled layout: rows and blocks over the padded space; the tile is
// kMxTileBytes with the scale of (row 2i + h, block l) at
// kTileCodes + 128h + 4l + i. mode 0 row-major, 1 tiled, 2 the activation
// operand layout (row-major codes; the scale of (row n, block b) at
// ((b / 4) N + n) 4 + b % 4, K a multiple of 128).
// Threads run over the blocks of all rows in order (row = index / bpr), so
// no lane idles when a row has fewer than 256 blocks (K = 5120: 160).
// grid: ceil(rows * bpr / 256) workgroups; block 256.
__global__ __launch_bounds__(256) void k_mx_encode(const uint16_t* __restrict__ W, int64_t N, int64_t K, int mode,
                                                   uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t kb = K / 32;                          // blocks per row
  const int64_t C = chunks_of(K);
  const bool tiled = mode == 1;
  const int64_t bpr = tiled ? C * 32 : kb;            // blocks per (padded) row
  const int64_t rows = tiled ? groups_of(N) * kGroupRows : N;
  const int64_t gb = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gb >= rows * bpr) return;
  int64_t n, b;
  if (rows * bpr <= (int64_t)UINT32_MAX) {   // 32-bit division where it suffices
    const uint32_t q = (uint32_t)gb / (uint32_t)bpr;
    n = q;
    b = (int64_t)((uint32_t)gb - q * (uint32_t)bpr);
  } else {
    n = gb / bpr;
    b = gb - n * bpr;
  }

  uint32_t sc = 0, q[4] = {0u, 0u, 0u, 0u};
  if (n < N && b < kb) {
    const uint4* src = reinterpret_cast<const uint4*>(W + n * K + b * 32);
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      d[4 * i] = v.x;
      d[4 * i + 1] = v.y;
      d[4 * i + 2] = v.z;
      d[4 * i + 3] = v.w;
    }
    uint32_t bm = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) bm = max(bm, max(d[j] & 0x7FFFu, (d[j] >> 16) & 0x7FFFu));
    if (bm != 0u) {
      const int ef = (int)(bm >> 7);                 // exponent field of the bf16 amax
      const int shared = max(-127, min(127, (ef == 0 ? -127 : ef - 127) - 2));
      sc = (uint32_t)(shared + 127);
      const float inv = __uint_as_float((uint32_t)(127 - shared) << 23);   // 2^-shared
      float v[32];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[2 * j] = bf16_bits_to_float(d[j] & 0xFFFFu) * inv;
        v[2 * j + 1] = bf16_bits_to_float(d[j] >> 16) * inv;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = e2m1_codes8(v + 8 * i);
    }
  }
  if (!tiled) {
    *reinterpret_cast<uint4*>(packed + n * (K / 2) + b * 16) = make_uint4(q[0], q[1], q[2], q[3]);
    scales[mode == 2 ? ((b >> 2) * N + n) * 4 + (b & 3) : n * kb + b] = (uint8_t)sc;
  } else {
    const int64_t g = n / kGroupRows, r = n % kGroupRows;
    const int64_t c = b / 32, l = b % 32;
    uint8_t* tile = packed + (g * C + c) * kMxTileBytes;
    *reinterpret_cast<uint4*>(tile + r * 512 + l * 16) = make_uint4(q[0], q[1], q[2], q[3]);
    tile[mx_tile_scale_offset((int)r, (int)l)] = (uint8_t)sc;
  }
}

template <class Src>
__global__ void k_finalize(const Src src, uint32_t* slot) {
  const float amax = src.amax(*slot);
  *reinterpret_cast<float*>(slot) = amax / 2688.0f;   // 0 stays 0
}

// One thread per 16-byte lane piece of a tile's codes (rows r, pieces l);
// the threads with r < 2 also write that row parity's 8 scale bytes of
// piece l (rows r, r + 2, r + 4, r + 6).
__global__ __launch_bounds__(256) void k_retile(const uint8_t* __restrict__ packed,
                                                const uint8_t* __restrict__ scales, int64_t N,
                                                int64_t K, uint8_t* __restrict__ tiles) {
  const int64_t G = groups_of(N), C = chunks_of(K);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= G * C * 256) return;
  const int64_t tile = t / 256, rl = t % 256;
  const int r = (int)(rl / 32), l = (int)(rl % 32);
  const int64_t g = tile / C, c = tile % C;
  const int64_t row = g * kGroupRows + r;
  const int64_t rb = K / 2;                 // canonical bytes per row
  const int64_t kbyte = c * 512 + l * 16;   // first byte of this piece in the row
  uint2 a = make_uint2(0, 0), b = make_uint2(0, 0);
  if (row < N) {
    const uint8_t* src = packed + row * rb + kbyte;   // 8-byte aligned (rb % 8 == 0)
    if (kbyte + 8 <= rb) a = *reinterpret_cast<const uint2*>(src);
    if (kbyte + 16 <= rb) b = *reinterpret_cast<const uint2*>(src + 8);
  }
  uint8_t* dst = tiles + tile * kTileBytes;
  *reinterpret_cast<uint4*>(dst + r * 512 + l * 16) = make_uint4(a.x, a.y, b.x, b.y);
  if (r < 2) {
    const int64_t kb = K / 16;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row2 = g * kGroupRows + 2 * i + r;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t blk = c * 64 + l * 2 + j;
        const uint32_t v = (row2 < N && blk < kb) ? scales[row2 * kb + blk] : 0u;
        const int pos = i * 2 + j;
        w[pos / 4] |= v << (8 * (pos % 4));
      }
    }
    *reinterpret_cast<uint2*>(dst + tile_scale_offset(r, 2 * l)) = make_uint2(w[0], w[1]);
  }
}

}  // namespace

template <class Src>
static hipError_t launch_quantize_src(const Src& src, const void* W, int64_t N, int64_t K, bool tiled,
                                      uint8_t* packed, uint8_t* scales, float* gscale, hipStream_t s) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(k_amax_init, dim3(1), dim3(1), 0, s, slot);
  const int64_t nvec = N * K / Src::kPerVec;
  const int64_t want = (nvec + 255) / 256;
  const int grid_amax = (int)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL((k_amax<Src>), dim3(grid_amax), dim3(256), 0, s, reinterpret_cast<const uint4*>(W), nvec,
                     slot);
  const int64_t rows = tiled ? groups_of(N) * kGroupRows : N;
  const int64_t bpr = tiled ? chunks_of(K) * 64 : K / 16;
  const int64_t wgs = rows * ((bpr + 255) / 256);   // one thread per block
  if (wgs > UINT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_encode<Src>), dim3((unsigned)wgs), dim3(256), 0, s, src, N, K,
                     tiled ? 1 : 0, packed, scales, slot);
  hipLaunchKernelGGL((k_finalize<Src>), dim3(1), dim3(1), 0, s, src, slot);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, bool tiled, uint8_t* packed,
                           uint8_t* scales, float* gscale, hipStream_t s) {
  return launch_quantize_src(SrcBf16{W}, W, N, K, tiled, packed, scales, gscale, s);
}

hipError_t launch_quantize_fp8(const uint8_t* W, const float* w_scale, int64_t N, int64_t K, bool tiled,
                               uint8_t* packed, uint8_t* scales, float* gscale, hipStream_t s) {
  return launch_quantize_src(SrcFp8{W, w_scale}, W, N, K, tiled, packed, scales, gscale, s);
}

hipError_t launch_quantize_mx(const uint16_t* W, int64_t N, int64_t K, int mode, uint8_t* packed, uint8_t* scales,
                              hipStream_t s) {
  const bool tiled = mode == 1;
  const int64_t rows = tiled ? groups_of(N) * kGroupRows : N;
  const int64_t bpr = tiled ? chunks_of(K) * 32 : K / 32;
  const int64_t wgs = (rows * bpr + 255) / 256;
  if (wgs > UINT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mx_encode, dim3((unsigned)wgs), dim3(256), 0, s, W, N, K, mode, packed, scales);
  return hipGetLastError();
}

hipError_t launch_retile(const uint8_t* packed, const uint8_t* scales, int64_t N, int64_t K, uint8_t* tiles,
                         hipStream_t s) {
  const int64_t n = groups_of(N) * chunks_of(K) * 256;
  hipLaunchKernelGGL(k_retile, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, packed, scales, N, K, tiles);
  return hipGetLastError();
}

}  // namespace fp4

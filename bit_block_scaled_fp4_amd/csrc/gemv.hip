// NVFP4 x bf16 matrix-vector (and small-M) product on the vector ALUs.
//
// Decode reads every weight once per token and does about two flops per
// weight, so it is bound by HBM bandwidth (page "imp" README, the decode
// paragraph; page "1. The big picture", "The most important number in this
// book"). The kernel streams the tiled layout, decodes in registers, and
// never expands weights to 16 bits in memory.
//
// Work split. A wave owns whole tiles (8 rows x 1024 K elements, codes and
// block scales together, 4608 bytes). Load q of a tile reads rows 2q and
// 2q + 1 as one contiguous kilobyte, so lane 32h + l holds piece l (32 K
// elements) of rows h, 2 + h, 4 + h, 6 + h, and both halves of the wave use
// the same 32 activations per lane. A workgroup owns `gw` row groups and
// all of K: `wc` waves per group, wave j taking chunks j, j + wc, ... one
// per round. Every load of a round is issued before its arithmetic, the
// chunk partial sums of a row are added in LDS in wave order, and the tensor
// scale is applied once per output. Results
// are deterministic and no scratch memory or cross-workgroup
// synchronisation is used.
//
// Loads go through buffer resources: a resource of zero bytes (an absent
// chunk or row group) or an offset past the end of x (the ragged last chunk)
// returns zeros without touching memory, so every wave issues the same
// unconditional loads and the compiler's wait counts stay exact.
//
// Arithmetic per 16-element block and activation row: 8 conversions of two
// E2M1 codes to two exact bf16 (v_cvt_scalef32_pk_bf16_fp4, scale 1), 8
// two-term dot products with fp32 accumulation (v_dot2_f32_bf16) and one
// multiply-add by the E4M3 block scale (decoded by v_cvt_f32_fp8, OCP
// E4M3). The code conversions are shared by the activation rows of a pass.
#include <algorithm>

#include "fp4_internal.h"
#include "greedy.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr int kMaxWaves = 16;
// Passes of at least this many rows share the activation loads between the
// half-waves. MI355X, graph-timed, same box, two alternating passes: at 4
// rows fused gate_up 2 x 17408 x 5120 29.4 against 30.7 us and the LM head
// 27.1 against 28.2 us; at 1 and 2 rows the down projection was 0.3-0.5 us
// slower with sharing and the other shapes equal.
#ifndef FP4_SHARE_X_MIN_ROWS
#define FP4_SHARE_X_MIN_ROWS 4
#endif

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// 16 bytes at `off`; aux 2 marks the weight stream non-temporal (read once).
template <int AUX>
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int X>
__device__ __forceinline__ float swz_xor(float v) {
  // ds_swizzle bit mode within 32 lanes: source lane = lane ^ X.
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (X << 10)));
}

// Sum four per-lane values over the 32 lanes of a half-wave. Each step
// halves the number of live values, so the total of value R = hl >> 3 ends
// in the 8 lanes with hl >> 3 == R (7 swizzles instead of 20).
__device__ __forceinline__ float reduce4(const float (&a)[4], int hl) {
  const bool b4 = hl & 16, b3 = hl & 8;
  float v2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = b4 ? a[i] : a[i + 2];
    const float keep = b4 ? a[i + 2] : a[i];
    v2[i] = keep + swz_xor<16>(send);
  }
  float v = (b3 ? v2[1] : v2[0]) + swz_xor<8>(b3 ? v2[0] : v2[1]);
  v += swz_xor<4>(v);
  v += swz_xor<2>(v);
  v += swz_xor<1>(v);
  return v;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Byte `sel` of w holds two E2M1 codes; returns them as two exact bf16
// values (low nibble in the low half). `sel` folds to a constant.
__device__ __forceinline__ bf16x2_t fp4x2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  }
}

// Byte `sel` of w holds two E2M1 codes; returns them times 2^(c - 127) as
// two bf16, where `s` carries c in its exponent field (c << 23): the
// conversion applies only that field. Bit-identical on MI355X to the fp32
// product for every code byte and every c <= 254, subnormal results
// included (c = 255, a NaN scale, gives a NaN of the other sign).
__device__ __forceinline__ bf16x2_t fp4x2_e8m0(uint32_t w, int sel, float s) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  }
}

// E4M3 (OCP) byte `sel` of w -> fp32.
__device__ __forceinline__ float e4m3(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// Two 16-element blocks of one row: sum of s0 * (first 16 products) and
// s1 * (last 16 products) added to acc; d holds the 32 decoded weights.
__device__ __forceinline__ float dot_block2(const bf16x2_t (&d)[16], const uint4 (&x)[4], float s0, float s1,
                                            float acc) {
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    p0 = __builtin_amdgcn_fdot2_f32_bf16(d[e], __builtin_bit_cast(bf16x2_t, word(x[e >> 2], e & 3)), p0, false);
#pragma unroll
  for (int e = 8; e < 16; ++e)
    p1 = __builtin_amdgcn_fdot2_f32_bf16(d[e], __builtin_bit_cast(bf16x2_t, word(x[e >> 2], e & 3)), p1, false);
  return fmaf(s1, p1, fmaf(s0, p0, acc));
}

// One round of a wave: one tile (4 x 16 code bytes and 8 scale bytes per
// lane) and, per activation row, the lane's 32 activations of the chunk.
template <int MT>
struct Round {
  uint4 w[4];
  uint2 s;
  uint4 x[MT][4];
};

// What the kernel does around the products.
enum Mode { kPlain = 0, kGreedy = 1, kSwiglu = 2, kRms = 3 };

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 8 bf16 activations times r and the 8 matching bf16 gains, rounded back to
// bf16 (two fp32 multiplies, one rounding to nearest even per element).
__device__ __forceinline__ uint4 norm8(const uint4& x, const uint4& g, float r) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t xw = word(x, i), gw = word(g, i);
    const float x0 = __uint_as_float(xw << 16), x1 = __uint_as_float(xw & 0xffff0000u);
    const float g0 = __uint_as_float(gw << 16), g1 = __uint_as_float(gw & 0xffff0000u);
    const f32x2_t v = {x0 * r * g0, x1 * r * g1};
    o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 1 / sqrt(mean_k x[row][k]^2 + eps) for the rows m0 .. m0 + MT - 1 (< M), in
// fp32, computed by the whole workgroup into rinv[]; `tmp` is LDS of
// kMaxWaves * MT floats.
template <int MT>
__device__ __forceinline__ void row_rms(const GemvArgs& a, int m0, float* rinv, float* tmp) {
  const int K = a.K, M = a.M;
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  float ss[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    ss[mi] = 0.0f;
    const int row = min(m0 + mi, M - 1);
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (int64_t)row * K, K * 2);
    for (int u = threadIdx.x; u < K / 8; u += blockDim.x) {
      const uint4 v = ld16<0>(rx, u * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = word(v, i);
        const float f0 = __uint_as_float(w << 16), f1 = __uint_as_float(w & 0xffff0000u);
        ss[mi] = fmaf(f0, f0, ss[mi]);
        ss[mi] = fmaf(f1, f1, ss[mi]);
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss[mi] += __shfl_xor(ss[mi], d);
    if (lane == 0) tmp[wave * MT + mi] = ss[mi];
  }
  __syncthreads();
  if ((int)threadIdx.x < MT) {
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += tmp[w * MT + threadIdx.x];
    rinv[threadIdx.x] = 1.0f / sqrtf(t / (float)K + a.eps);
  }
  __syncthreads();
}

// grid: workgroups over all projections; block: gw * wc waves (at most 16).
// MODE kGreedy (one projection, M <= MT): the launch ends with the greedy
// choice over each row of y (greedy.h). kSwiglu (projections gate and up):
// a workgroup's first gw * wc waves take its row groups of gate, the others
// the same row groups of up, and the epilogue writes h = bf16(silu(gate) *
// up) instead of y. kRms (M <= MT): every workgroup first computes each
// row's 1 / sqrt(mean(x^2) + eps) and the products read bf16(x * that *
// gain). Each mode is its own instantiation, so the plain product keeps its
// registers. MX (kPlain only): MXFP4 tiles (kMxTileBytes; one E8M0 scale per
// 32-element piece, the four of a lane's rows in one word at kTileCodes +
// 4 * lane; no tensor scale).
template <int MT, int MODE, bool MX = false>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemv(const GemvArgs a) {
  constexpr int TB = MX ? kMxTileBytes : kTileBytes;
  __shared__ float part[kMaxWaves][MT][8];
  __shared__ uint64_t red[MODE == kGreedy ? kMaxWaves * MT : 1];
  __shared__ float rinv[MODE == kRms ? MT : 1];
  __shared__ int flag;
  uint64_t keys[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) keys[mi] = 0;
  const int lane = threadIdx.x & 63, hl = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C = a.C, K = a.K, M = a.M, Wc = a.wc, Gw = a.gw;

  int p = 0, gi, wc;
  if (MODE == kSwiglu) {
    p = wave / (Gw * Wc);
    const int rest = wave - p * Gw * Wc;
    gi = rest / Wc;
    wc = rest - gi * Wc;
  } else {
    while (p + 1 < a.nproj && (int)blockIdx.x >= a.proj[p + 1].wg_begin) ++p;
    gi = wave / Wc;
    wc = wave - gi * Wc;
  }
  const ProjDesc& pd = a.proj[p];
  const int N = pd.N, G = (N + 7) >> 3;
  const int g = ((int)blockIdx.x - pd.wg_begin) * Gw + gi;
  const bool gvalid = g < G;
  const float gs = MX ? 1.0f : *pd.gscale;

  for (int m0 = 0; m0 < M; m0 += MT) {
    if (MODE == kRms) row_rms<MT>(a, m0, rinv, &part[0][0][0]);
    float acc[MT][4];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mi][i] = 0.0f;

    for (int c = wc; c < C; c += Wc) {
      Round<MT> f;
      {
        const bool v = gvalid;
        const __amdgpu_buffer_rsrc_t r = rsrc(pd.tiles + (v ? ((int64_t)g * C + c) * TB : 0), v ? TB : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) f.w[q] = ld16<2>(r, q * 1024 + lane * 16);
        if (MX) {
          f.s = make_uint2(__builtin_amdgcn_raw_buffer_load_b32(r, kTileCodes + lane * 4, 0, 0), 0u);
        } else {
          const u32x2_t sv = __builtin_amdgcn_raw_buffer_load_b64(r, kTileCodes + lane * 8, 0, 0);
          f.s = make_uint2(sv[0], sv[1]);
        }
      }
      const int off = (c * kChunkK + hl * 32) * 2;   // past K (ragged last chunk): zeros
      // Both half-waves need the same 32 activations per lane. With kShareX
      // each half loads two of the four 16-byte units (half h: units 2h,
      // 2h + 1) and a lane swap hands each lane the other half's pair.
      constexpr bool kShareX = MT >= FP4_SHARE_X_MIN_ROWS;
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const int row = min(m0 + mi, M - 1);
        const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (int64_t)row * K, K * 2);
        if (kShareX) {
#pragma unroll
          for (int q = 0; q < 2; ++q) f.x[mi][q] = ld16<0>(rx, off + (2 * h + q) * 16);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) f.x[mi][q] = ld16<0>(rx, off + q * 16);
        }
      }
      uint4 gn[4];
      if (MODE == kRms) {
        const __amdgpu_buffer_rsrc_t rg = rsrc(a.gain, K * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) gn[q] = ld16<0>(rg, off + q * 16);
      }
      // keep every load of the round ahead of the arithmetic
      __builtin_amdgcn_sched_barrier(0);
      if (kShareX) {
        // permlane32_swap(v, v) returns the low half-wave's v in every lane as
        // its first result and the high half's as its second (checked on
        // MI355X): units 0, 1 come from half 0, units 2, 3 from half 1
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
          uint32_t lo[8], hi[8];
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            const uint32_t v = word(f.x[mi][d >> 2], d & 3);
            const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            lo[d] = r[0];
            hi[d] = r[1];
          }
          f.x[mi][0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
          f.x[mi][1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
          f.x[mi][2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          f.x[mi][3] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        }
      }
      if (MODE == kRms) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
#pragma unroll
          for (int q = 0; q < 4; ++q) f.x[mi][q] = norm8(f.x[mi][q], gn[q], rinv[mi]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (MX) {
          // row 2i + h, its one E8M0 block scale (byte i) applied by the
          // conversion itself: exact bf16 weights, no scale multiply
          const float sc = __uint_as_float(((f.s.x >> (8 * i)) & 0xFFu) << 23);
          bf16x2_t d[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) d[e] = fp4x2_e8m0(word(f.w[i], e >> 2), e & 3, sc);
#pragma unroll
          for (int mi = 0; mi < MT; ++mi) acc[mi][i] = dot_block2(d, f.x[mi], 1.0f, 1.0f, acc[mi][i]);
          continue;
        }
        // row 2i + h: its two block scales are bytes 2(i&1), 2(i&1)+1 of
        // word i >> 1
        const uint32_t sw = i < 2 ? f.s.x : f.s.y;
        const float s0 = e4m3(sw, (i & 1) * 2);
        const float s1 = e4m3(sw, (i & 1) * 2 + 1);
        bf16x2_t d[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) d[e] = fp4x2(word(f.w[i], e >> 2), e & 3);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) acc[mi][i] = dot_block2(d, f.x[mi], s0, s1, acc[mi][i]);
      }
    }

    // lane (h, hl) holds rows 2i + h; the half-wave total of row 2(hl >> 3) + h
    // ends in the lanes with hl % 8 == 0
    const int rr = 2 * (hl >> 3) + h;
    const bool holder = (hl & 7) == 0;
    if (Wc == 1 && MODE != kSwiglu) {
      const int n = 8 * g + rr;
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const float t = reduce4(acc[mi], hl);
        if (holder && gvalid && n < N && m0 + mi < M) {
          const float v = gs * t;
          pd.y[(int64_t)(m0 + mi) * pd.ldy + n] = v;
          if (MODE == kGreedy) keys[mi] = umax64(keys[mi], greedy_key(v, n));
        }
      }
    } else {
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const float t = reduce4(acc[mi], hl);
        if (holder) part[wave][mi][rr] = t;
      }
      __syncthreads();
      if ((int)threadIdx.x < Gw * MT * 8) {
        const int gg = threadIdx.x / (MT * 8), mi = (threadIdx.x / 8) % MT, r = threadIdx.x % 8;
        float s = 0.0f;
        for (int w = 0; w < Wc; ++w) s += part[gg * Wc + w][mi][r];   // chunk order
        const int n = 8 * (((int)blockIdx.x - pd.wg_begin) * Gw + gg) + r;
        if (MODE == kSwiglu) {
          float su = 0.0f;
          for (int w = 0; w < Wc; ++w) su += part[Gw * Wc + gg * Wc + w][mi][r];
          const float vg = *a.proj[0].gscale * s, vu = *a.proj[1].gscale * su;
          if (n < N && m0 + mi < M)
            a.h[(int64_t)(m0 + mi) * a.ldh + n] = bf16_rne(vg / (1.0f + __expf(-vg)) * vu);
        } else if (n < N && m0 + mi < M) {
          const float v = gs * s;
          pd.y[(int64_t)(m0 + mi) * pd.ldy + n] = v;
          if (MODE == kGreedy) {
#pragma unroll
            for (int j = 0; j < MT; ++j)
              if (j == mi) keys[j] = umax64(keys[j], greedy_key(v, n));
          }
        }
      }
      __syncthreads();
    }
  }
  if (MODE == kGreedy) greedy_finish<MT>(a.greedy, keys, M, red, &flag);
}

}  // namespace

// Launch geometry, from sweeps on MI355X (graph-timed, rotating weights):
// one tile per wave per round, rounds issued one after the other (a second
// tile in flight per wave measured no faster). Short K packs about four
// waves per workgroup.
//   M > 1: wc = ceil(C / 3) below 8 chunks; from 8 chunks on, one row
//     group of 8 waves per workgroup (two waves per SIMD; 7 or 9 leave the
//     SIMDs unevenly loaded): down 5120 x 17408 at M = 2 / 3 / 4 13.7 /
//     18.0 / 18.7 against 14.5 / 20.3 / 20.6 us with 6 waves, 16.6 / 22.1 /
//     22.3 with 9.
//   M = 1, at most 16 chunks: one round (wc = C), unless the launch has at
//     least 8 row groups per CU, where two rounds (wc = ceil(C / 2)) are
//     faster (gate_up 34816 x 5120: 17.6 against 18.0-18.7 us).
//   M = 1, more than 16 chunks: about one workgroup per CU, gw =
//     ceil(groups / CUs) row groups of about 9 / gw waves each, every wave
//     streaming its chunks (down 5120 x 17408: 10.9 against 11.8 us with 9
//     waves per group in two rounds; 8192 x 28672: 22.0 against 27.6 us).
//     Beyond 9 groups per CU the two-round layout below is used.
//   Otherwise wc = ceil(C / ceil(C / 16)); gw = max(1, 4 / wc).
//   Row groups per workgroup never exceed groups / CUs (small launches keep
//   every CU busy: Qwen3-0.6B-shaped QKV 4096 x 1024 at M = 1 3.15 against
//   3.44 us with four groups per workgroup; M = 2 3.51 against 3.94 us).
// Fills a.wc, a.gw and the projections' wg_begin; returns the workgroups.
template <int MT>
static int64_t plan_mt(GemvArgs& a, int gw, int wc) {
  const int rounds = (a.C + kMaxWaves - 1) / kMaxWaves;
  int64_t groups = 0;
  for (int i = 0; i < a.nproj; ++i) groups += groups_of(a.proj[i].N);
  const int ncu = device_cu_count();
  if (MT == 1 && gw <= 0 && wc <= 0) {
    if (ncu > 0 && a.C > kMaxWaves) {
      const int64_t per_cu = (groups + ncu - 1) / ncu;
      if (per_cu <= 9) {
        gw = (int)per_cu;
        wc = std::max(1, 9 / gw);
      }
    } else if (ncu > 0 && a.C >= 4 && groups >= 8 * (int64_t)ncu) {
      wc = (a.C + 1) / 2;
    }
  }
  int w = wc > 0 ? wc : (MT == 1 ? (a.C + rounds - 1) / rounds : a.C >= 8 ? 8 : (a.C + 2) / 3);
  a.wc = std::max(1, std::min(w, kMaxWaves));
  if (gw <= 0) {
    // about four waves per workgroup, but never so many row groups per
    // workgroup that the launch has fewer workgroups than CUs
    gw = std::max(1, 4 / a.wc);
    if (ncu > 0) gw = (int)std::max<int64_t>(1, std::min<int64_t>(gw, groups / ncu));
  }
  a.gw = std::max(1, std::min(gw, kMaxWaves / a.wc));
  int64_t wgs = 0;
  for (int i = 0; i < a.nproj; ++i) {
    a.proj[i].wg_begin = (int32_t)wgs;
    wgs += (groups_of(a.proj[i].N) + a.gw - 1) / a.gw;
  }
  return wgs;
}

template <int MT>
static hipError_t launch_mt(GemvArgs a, hipStream_t s, int gw, int wc) {
  const int64_t wgs = plan_mt<MT>(a, gw, wc);
  a.greedy.S = (int32_t)wgs;
  const dim3 grid((unsigned)wgs), block(64 * a.gw * a.wc);
  if (a.mx)
    hipLaunchKernelGGL((k_gemv<MT, kPlain, true>), grid, block, 0, s, a);
  else if (a.greedy.idx)
    hipLaunchKernelGGL((k_gemv<MT, kGreedy>), grid, block, 0, s, a);
  else if (a.gain)
    hipLaunchKernelGGL((k_gemv<MT, kRms>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_gemv<MT, kPlain>), grid, block, 0, s, a);
  return hipGetLastError();
}

// The gate and up products of a gated MLP with the SwiGLU epilogue: the
// geometry of the fused gate_up product (waves per row group as planned for
// both projections together), with each workgroup taking the same row
// groups of both, at most 16 waves in all.
template <int MT>
static hipError_t launch_swiglu_mt(GemvArgs a, hipStream_t s) {
  plan_mt<MT>(a, 0, 0);
  a.gw = std::max(1, std::min(a.gw, kMaxWaves / (2 * a.wc)));
  if (2 * a.gw * a.wc > kMaxWaves) return hipErrorInvalidValue;
  const int64_t wgs = (groups_of(a.proj[0].N) + a.gw - 1) / a.gw;
  a.proj[0].wg_begin = a.proj[1].wg_begin = 0;
  hipLaunchKernelGGL((k_gemv<MT, kSwiglu>), dim3((unsigned)wgs), dim3(64 * 2 * a.gw * a.wc), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv_swiglu(const GemvArgs& a, hipStream_t s) {
  if (a.nproj != 2 || a.proj[0].N != a.proj[1].N || !a.h) return hipErrorInvalidValue;
  if (a.M == 1) return launch_swiglu_mt<1>(a, s);
  if (a.M == 2) return launch_swiglu_mt<2>(a, s);
  if (a.M <= 4) return launch_swiglu_mt<4>(a, s);
  return hipErrorInvalidValue;
}

int64_t gemv_workgroups(const GemvArgs& a) {
  GemvArgs b = a;
  if (a.M == 1) return plan_mt<1>(b, 0, 0);
  if (a.M == 2) return plan_mt<2>(b, 0, 0);
  return plan_mt<4>(b, 0, 0);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t s, int gw, int wc) {
  if (a.M == 1) return launch_mt<1>(a, s, gw, wc);
  if (a.M == 2) return launch_mt<2>(a, s, gw, wc);
  if (a.M <= 4 || a.mx) return launch_mt<4>(a, s, gw, wc);   // MXFP4: passes of 4 rows
  return hipErrorInvalidValue;   // more NVFP4 rows go to the matrix-core kernel
}

}  // namespace fp4

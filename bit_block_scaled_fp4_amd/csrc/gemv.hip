// NVFP4 x bf16 matrix-vector (and small-M) product on the vector ALUs.
//
// Decode reads every weight once per token and does about two flops per
// weight, so it is bound by HBM bandwidth (page "imp" README, the decode
// paragraph; page "1. The big picture", "The most important number in this
// book"). The kernel therefore streams the tiled weight layout with 16-byte
// loads, decodes in registers, and never expands weights to 16 bits in memory.
//
// Work split. The unit of work is one 8-row group x one 1024-element chunk
// (one tile of the device layout: 4 KB of codes + 512 B of scales) and it
// belongs to one half-wave (32 lanes x 32 elements). A workgroup owns Gw
// whole row groups across all C chunks, i.e. Gw*C units on ceil(Gw*C/2)
// waves, so consecutive half-waves read consecutive tiles and consecutive
// workgroups read consecutive groups: at any moment the running waves sweep
// one compact window of memory, and the many small workgroups let the
// dispatcher balance the compute units. The chunk partial sums of a row are
// added in LDS in chunk order, so results are deterministic and no scratch
// memory or cross-workgroup synchronisation is needed. (Above 32 chunks a
// half-wave loops over chunks j, j+32, ...)
//
// Arithmetic per 16-element block and activation row:
//   8 x v_cvt_scalef32_pk_bf16_fp4 (two E2M1 codes -> two exact bf16, scale 1)
//   8 x v_dot2_f32_bf16 (two products + fp32 accumulate)
//   1 x fma with the E4M3 block scale (decoded by v_cvt_f32_fp8, OCP E4M3)
// and the tensor scale is applied once per output. The decode is shared by
// the MT activation rows of one pass.
#include <algorithm>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int X>
__device__ __forceinline__ float swz_xor(float v) {
  // ds_swizzle bit mode within 32 lanes: source lane = lane ^ X.
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (X << 10)));
}

// Sum eight per-lane values over the 32 lanes of a half-wave. Each step
// halves the number of live values (a transposing reduction), so the total
// for row R = hl >> 2 ends in lanes with hl >> 2 == R: 9 swizzles, not 40.
__device__ __forceinline__ float reduce8(const float (&a)[8], int hl) {
  const bool b4 = hl & 16, b3 = hl & 8, b2 = hl & 4;
  float v4[4], v2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float send = b4 ? a[i] : a[i + 4];
    const float keep = b4 ? a[i + 4] : a[i];
    v4[i] = keep + swz_xor<16>(send);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = b3 ? v4[i] : v4[i + 2];
    const float keep = b3 ? v4[i + 2] : v4[i];
    v2[i] = keep + swz_xor<8>(send);
  }
  float v = (b2 ? v2[1] : v2[0]) + swz_xor<4>(b2 ? v2[0] : v2[1]);
  v += swz_xor<2>(v);
  v += swz_xor<1>(v);
  return v;
}

// Byte `sel` of w holds two E2M1 codes; returns them as two exact bf16
// values (low nibble in the low half). `sel` folds to a constant once the
// calling loops are unrolled.
__device__ __forceinline__ bf16x2_t fp4x2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
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

// Same for four values: the total for row R = hl >> 3 ends in lanes with
// hl >> 3 == R.
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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One unit's operands for a lane: 16 B of each of its R rows (R = 8, or 4
// for half a row group), the scale bytes of those rows (2 per row) and 32
// activations per activation row.
template <int MT, int R>
struct Frag {
  uint4 w[R];
  uint32_t s[R / 2];
  uint4 x[MT][4];
};

__device__ __forceinline__ uint4 ld16_nt(const uint8_t* p) {
  // weights are read exactly once: stream them past the caches
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int MT, int R>
__device__ __forceinline__ void load_frag(Frag<MT, R>& f, const uint8_t* ptile, const uint8_t* stile,
                                          const uint16_t* x, int c, int hl, int m0, int M, int K) {
  // Scales use ordinary (cached) loads: with 4-row units the two halves of a
  // lane's 16 scale bytes belong to neighbouring workgroups, and the second
  // one should find the line in L2 rather than fetch it again.
  if constexpr (R == 8) {
    const uint4 sv = *reinterpret_cast<const uint4*>(stile);
    f.s[0] = sv.x; f.s[1] = sv.y; f.s[2] = sv.z; f.s[3] = sv.w;
  } else {
    const uint2 sv = *reinterpret_cast<const uint2*>(stile);
    f.s[0] = sv.x; f.s[1] = sv.y;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) f.w[r] = ld16_nt(ptile + r * 512);
  const int k0 = c * kChunkK + hl * 32;
  if ((c + 1) * kChunkK <= K) {
    // whole chunk (half-wave-uniform test): plain 16-byte loads
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int row = min(m0 + mi, M - 1);
      const uint4* xp = reinterpret_cast<const uint4*>(x + (int64_t)row * K + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) f.x[mi][q] = xp[q];
    }
  } else {
    // ragged last chunk: a lane's 32 activations are all, half (K % 32 == 16)
    // or none inside K. Addresses are clamped into the row and the values
    // outside K replaced by zero, so the loads stay unconditional.
    const int kv = K - k0;
    const int ka = kv > 0 ? k0 : 0, kb = kv >= 32 ? k0 + 16 : 0;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int row = min(m0 + mi, M - 1);
      const uint4* xa = reinterpret_cast<const uint4*>(x + (int64_t)row * K + ka);
      const uint4* xb = reinterpret_cast<const uint4*>(x + (int64_t)row * K + kb);
      const uint4 a0 = xa[0], a1 = xa[1], b0 = xb[0], b1 = xb[1];
      const uint4 z = make_uint4(0, 0, 0, 0);
      f.x[mi][0] = kv > 0 ? a0 : z;
      f.x[mi][1] = kv > 0 ? a1 : z;
      f.x[mi][2] = kv >= 32 ? b0 : z;
      f.x[mi][3] = kv >= 32 ? b1 : z;
    }
  }
}

template <int MT, int R>
__device__ __forceinline__ void compute_frag(float (&acc)[MT][R], const Frag<MT, R>& f) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    bf16x2_t d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = fp4x2(word(f.w[r], i >> 2), i & 3);
    const uint32_t sw = f.s[r >> 1];
    const float s0 = e4m3(sw, (r & 1) * 2);
    const float s1 = e4m3(sw, (r & 1) * 2 + 1);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p0 = __builtin_amdgcn_fdot2_f32_bf16(d[i], __builtin_bit_cast(bf16x2_t, word(f.x[mi][i >> 2], i & 3)), p0, false);
#pragma unroll
      for (int i = 8; i < 16; ++i)
        p1 = __builtin_amdgcn_fdot2_f32_bf16(d[i], __builtin_bit_cast(bf16x2_t, word(f.x[mi][i >> 2], i & 3)), p1, false);
      acc[mi][r] = fmaf(s1, p1, fmaf(s0, p0, acc[mi][r]));
    }
  }
}

// Half-wave units per workgroup: 32 (16 waves) for one or two activation
// rows, fewer for wider M tiles so that the registers of the activation
// fragment fit (the launch bound caps VGPRs at 512 / waves-per-SIMD).
template <int MT>
constexpr int max_units() { return MT == 1 ? 32 : (MT <= 4 ? 16 : 8); }

// Workgroup = Gw row units (R rows each) x all C chunks; half-wave j
// (0 <= j < Gw*Cu) takes row unit j / Cu and chunks (j % Cu) + Cu*i, ...
template <int MT, int R>
__global__ __launch_bounds__(32 * max_units<MT>()) void k_gemv(const GemvArgs a) {
  constexpr int kMaxUnits = max_units<MT>();
  __shared__ float red[kMaxUnits][MT][R];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, hl = lane & 31;
  const int j = 2 * wave + half;

  int p = 0;
  while (p + 1 < a.nproj && (int)blockIdx.x >= a.proj[p + 1].tile_begin) ++p;
  const int N = a.proj[p].N;
  const int G = (N + R - 1) / R;                         // row units of this projection
  const int C = a.C, K = a.K, M = a.M, Gw = a.gw;
  const int Cu = a.cu;                                   // half-wave units per row unit
  const int units = Gw * Cu;
  const int gi = j / Cu, c0 = j - gi * Cu;
  const int g = ((int)blockIdx.x - a.proj[p].tile_begin) * Gw + gi;
  const bool active = j < units && g < G;
  const int ga = active ? g : 0;
  // row unit ga = rows [R*ga, R*ga + R): 8-row group ga*R/8, first row (ga*R) % 8 inside it
  const int64_t tile0 = (int64_t)((ga * R) >> 3) * C + c0;
  const int r0 = (ga * R) & 7;
  const uint8_t* ptile = a.proj[p].packed + tile0 * kTilePacked + r0 * 512 + hl * 16;
  const uint8_t* stile = a.proj[p].scales + tile0 * kTileScale + hl * 16 + r0 * 2;
  const float gs = *a.proj[p].gscale;

  for (int m0 = 0; m0 < M; m0 += MT) {
    float acc[MT][R];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[mi][r] = 0.0f;
    if (active) {
      for (int c = c0; c < C; c += Cu) {
        Frag<MT, R> f;
        const int64_t dc = c - c0;
        load_frag<MT, R>(f, ptile + dc * kTilePacked, stile + dc * kTileScale, a.x, c, hl, m0, M, K);
        compute_frag<MT, R>(acc, f);
      }
    }
    float tot[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if constexpr (R == 8) tot[mi] = reduce8(acc[mi], hl);     // row hl >> 2 of this unit
      else tot[mi] = reduce4(acc[mi], hl);                      // row hl >> 3 of this unit
    }
    constexpr int kShift = R == 8 ? 2 : 3;
    const bool holder = (hl & ((1 << kShift) - 1)) == 0;
    const int rr = hl >> kShift;

    if (Cu == 1) {
      // every unit covers all of K: write directly
      const int n = R * g + rr;
      if (holder && active && n < N) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi)
          if (m0 + mi < M) a.proj[p].y[(int64_t)(m0 + mi) * a.proj[p].ldy + n] = gs * tot[mi];
      }
    } else {
      if (holder && j < units) {
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) red[j][mi][rr] = tot[mi];
      }
      __syncthreads();
      if ((int)threadIdx.x < Gw * MT * R) {
        const int gg = threadIdx.x / (MT * R), mi = (threadIdx.x / R) % MT, r = threadIdx.x % R;
        float s = 0.0f;
        for (int cc = 0; cc < Cu; ++cc) s += red[gg * Cu + cc][mi][r];   // chunk order
        const int n = R * (((int)blockIdx.x - a.proj[p].tile_begin) * Gw + gg) + r;
        if (n < N && m0 + mi < M) a.proj[p].y[(int64_t)(m0 + mi) * a.proj[p].ldy + n] = gs * s;
      }
      __syncthreads();
    }
  }
}

}  // namespace

// Launch geometry: R rows per unit, Cu half-wave units per row unit (each
// takes chunks c, c+Cu, ...), Gw row units per workgroup. Chosen from
// sweeps on MI355X (one 1024-chunk per unit is best while the workgroup
// stays small; long rows are split into ~6-chunk runs; a single chunk uses
// 4-row units, 8 per workgroup):
//   C == 1:      R = 4, Cu = 1, Gw = 8
//   2 <= C <= 7: R = 8, Cu = C, Gw = 1
//   C >= 8:      R = 4, Cu = ceil(C / 6), Gw = 1
struct Geometry { int rows, gw, cu; };

static Geometry pick_geometry(int C, int max_units) {
  Geometry g;
  if (C == 1) g = {4, 8, 1};
  else if (C <= 7) g = {8, 1, C};
  else g = {4, 1, (C + 5) / 6};
  g.cu = std::min(g.cu, max_units);
  g.gw = std::max(1, std::min(g.gw, max_units / g.cu));
  return g;
}

template <int MT, int R>
static hipError_t launch_mtr(GemvArgs a, hipStream_t s, int gw, int cu) {
  constexpr int kMaxUnits = max_units<MT>();
  a.cu = std::min(std::min(cu, a.C), kMaxUnits);
  a.gw = std::max(1, std::min(gw, kMaxUnits / a.cu));
  int64_t wgs = 0;
  for (int i = 0; i < a.nproj; ++i) {
    a.proj[i].tile_begin = (int32_t)wgs;
    wgs += ((a.proj[i].N + R - 1) / R + a.gw - 1) / a.gw;
  }
  a.total_tiles = (int32_t)wgs;
  const int waves = (a.gw * a.cu + 1) / 2;
  hipLaunchKernelGGL((k_gemv<MT, R>), dim3((unsigned)wgs), dim3(64 * waves), 0, s, a);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_mt(const GemvArgs& a, hipStream_t s, int gw, int cu, int rows) {
  const Geometry d = pick_geometry(a.C, max_units<MT>());
  if (rows <= 0) rows = d.rows;
  if (gw <= 0) gw = d.gw;
  if (cu <= 0) cu = d.cu;
  return rows == 4 ? launch_mtr<MT, 4>(a, s, gw, cu) : launch_mtr<MT, 8>(a, s, gw, cu);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t s, int gw, int cu, int rows) {
  if (a.M == 1) return launch_mt<1>(a, s, gw, cu, rows);
  if (a.M == 2) return launch_mt<2>(a, s, gw, cu, rows);
  if (a.M <= 4) return launch_mt<4>(a, s, gw, cu, rows);
  return launch_mt<8>(a, s, gw, cu, rows);
}

}  // namespace fp4

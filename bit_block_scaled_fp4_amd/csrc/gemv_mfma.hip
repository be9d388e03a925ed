// NVFP4 x bf16 product for small M (a handful of concurrent decode streams or
// speculative-verify tokens) on the matrix cores.
//
// Several activation rows share one pass over the weights, so the weights
// are still read once (page "1. The big picture", the batching and
// speculative-decoding bullets of "The most important number in this
// book"); the vector-ALU kernel would redo two products per weight for
// every activation row, which makes it ALU-bound from about four rows on.
// Here each weight is decoded once to bf16 (E2M1 * E4M3 has at most 6
// significant bits: exact) and fed to v_mfma_f32_16x16x32_bf16 with the
// activations (M padded to 16 per M-tile) as the A operand; the tensor
// scale is applied once in the epilogue.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, q = l / 16):
//   A: row l % 16, k = 8q .. 8q+7;  B: column l % 16, k = 8q .. 8q+7;
//   D: column l % 16, rows 4q .. 4q+3.
// The order of the 32 k inside one MFMA is free as long as A and B agree, so
// lane (q, n) loads row n's 16-byte piece p = 4t + q of a 1024-element chunk
// (t = 0..7, 32 elements = two scale blocks) and supplies its elements
// 8j..8j+7 to the j-th of four MFMAs; the A lane (q, m) loads the matching 32
// activations x[m][32p .. 32p+31]. One wave covers NT 16-row N-subtiles of
// one chunk, in two batches of four pieces whose loads are all in flight
// before the batch's arithmetic; S waves of a workgroup split the chunks of
// the same rows and add their partial tiles in LDS in a fixed order.
#include <algorithm>

#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 8;

__device__ __forceinline__ f32x2_t fp4x2_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // exact: both values have <= 6 significant bits and lie in bf16 range
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Four B operands (8 bf16 each) from one 16-byte piece: e2m1 * block scale.
__device__ __forceinline__ void decode_piece(bf16x8_t (&b)[4], const uint4& w, float s0, float s1) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float s = j < 2 ? s0 : s1;
    const uint32_t wd = word(w, j);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t e = fp4x2_f32(wd, i);
      o[i] = pack_bf16(e[0] * s, e[1] * s);
    }
    b[j] = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
  }
}

// grid: one workgroup per 16*NT-row tile (over all projections); S waves.
template <int NT, int MTL>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemv_mfma(const GemvArgs a) {
  extern __shared__ f32x4_t red_dyn[];                 // [S][NT][MTL][64] when S > 1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int q = lane >> 4, n16 = lane & 15;

  int p = 0;
  while (p + 1 < a.nproj && (int)blockIdx.x >= a.proj[p + 1].wg_begin) ++p;
  const int N = a.proj[p].N;
  const int G = (N + 7) >> 3;
  const int C = a.C, K = a.K, M = a.M;
  const int row0 = ((int)blockIdx.x - a.proj[p].wg_begin) * 16 * NT;
  const float gs = *a.proj[p].gscale;

  // this lane's weight row in each N-subtile: codes at prow + c*kTileBytes +
  // 16*piece, the piece's two block scales at srow + c*kTileBytes + 8*piece
  const uint8_t* prow[NT];
  const uint8_t* srow[NT];
  bool rvalid[NT];
#pragma unroll
  for (int s = 0; s < NT; ++s) {
    const int n = row0 + 16 * s + n16;
    const int g = n >> 3;
    rvalid[s] = g < G;
    const int gg = rvalid[s] ? g : 0;
    const uint8_t* tile0 = a.proj[p].tiles + (int64_t)gg * C * kTileBytes;
    prow[s] = tile0 + (n & 7) * 512;
    srow[s] = tile0 + tile_scale_offset(n & 7, 0);
  }

  for (int m0 = 0; m0 < M; m0 += 16 * MTL) {
    f32x4_t acc[NT][MTL];
#pragma unroll
    for (int s = 0; s < NT; ++s)
#pragma unroll
      for (int mt = 0; mt < MTL; ++mt) acc[s][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c = wave; c < C; c += S) {
      const bool full = (c + 1) * kChunkK <= K;
      // two batches of four pieces; every load of a batch is issued before
      // any of its arithmetic, so a chunk costs two memory round trips
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        uint4 wv[NT][4];
        uint32_t sv[NT][4];
        uint4 xv[MTL][4][4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int piece = 4 * (4 * hb + tt) + q;
#pragma unroll
          for (int s = 0; s < NT; ++s) {
            wv[s][tt] = *reinterpret_cast<const uint4*>(prow[s] + (int64_t)c * kTileBytes + piece * 16);
            sv[s][tt] = *reinterpret_cast<const uint16_t*>(srow[s] + (int64_t)c * kTileBytes + piece * 8);
          }
          const int k0 = c * kChunkK + 32 * piece;
          const int kv = K - k0;                     // <= 0, 16 or >= 32 (K % 16 == 0)
          const int ka = (full || kv > 0) ? k0 : 0, kb = (full || kv >= 32) ? k0 + 16 : 0;
#pragma unroll
          for (int mt = 0; mt < MTL; ++mt) {
            const int m = m0 + 16 * mt + n16;
            const int mr = m < M ? m : M - 1;
            const uint4* xp = reinterpret_cast<const uint4*>(a.x + (int64_t)mr * K + ka);
            const uint4* xq = reinterpret_cast<const uint4*>(a.x + (int64_t)mr * K + kb);
            xv[mt][tt][0] = xp[0];
            xv[mt][tt][1] = xp[1];
            xv[mt][tt][2] = xq[0];
            xv[mt][tt][3] = xq[1];
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int piece = 4 * (4 * hb + tt) + q;
          const int kv = K - (c * kChunkK + 32 * piece);
          bf16x8_t xa[MTL][4];
#pragma unroll
          for (int mt = 0; mt < MTL; ++mt) {
            const int m = m0 + 16 * mt + n16;
            const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              uint4 v = xv[mt][tt][j];
              if (m >= M || (!full && (j < 2 ? kv <= 0 : kv < 32))) v = z;
              xa[mt][j] = __builtin_bit_cast(bf16x8_t, v);
            }
          }
#pragma unroll
          for (int s = 0; s < NT; ++s) {
            const uint4 w = rvalid[s] ? wv[s][tt] : make_uint4(0, 0, 0, 0);
            const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sv[s][tt], 0);
            const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sv[s][tt], 1);
            bf16x8_t b[4];
            decode_piece(b, w, s0, s1);
#pragma unroll
            for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mt][j], b[j], acc[s][mt], 0, 0, 0);
          }
        }
      }
    }

    // lane (q, n16) holds rows m0 + 16 mt + 4q + i, column row0 + 16 s + n16
    if (S > 1) {
#pragma unroll
      for (int s = 0; s < NT; ++s)
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) red_dyn[((wave * NT + s) * MTL + mt) * 64 + lane] = acc[s][mt];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int s = 0; s < NT; ++s)
#pragma unroll
          for (int mt = 0; mt < MTL; ++mt) {
            f32x4_t t = red_dyn[(s * MTL + mt) * 64 + lane];
            for (int w = 1; w < S; ++w) t += red_dyn[((w * NT + s) * MTL + mt) * 64 + lane];   // wave order
            acc[s][mt] = t;
          }
      }
    }
    if (wave == 0) {
#pragma unroll
      for (int s = 0; s < NT; ++s) {
        const int n = row0 + 16 * s + n16;
        if (n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * mt + 4 * q + i;
            if (m < M) a.proj[p].y[(int64_t)m * a.proj[p].ldy + n] = gs * acc[s][mt][i];
          }
      }
    }
    if (S > 1) __syncthreads();
  }
}

template <int NT, int MTL>
hipError_t launch_nt(GemvArgs a, hipStream_t st, int split) {
  int64_t wgs = 0;
  for (int i = 0; i < a.nproj; ++i) {
    a.proj[i].wg_begin = (int32_t)wgs;
    wgs += (a.proj[i].N + 16 * NT - 1) / (16 * NT);
  }
  int S = split;
  if (S <= 0) {
    // enough waves to fill the machine, never more waves than chunks
    S = (int)std::min<int64_t>(kMaxWaves, std::max<int64_t>(1, (2048 + wgs - 1) / wgs));
    S = std::min(S, a.C);
    const int per = (a.C + S - 1) / S;
    S = (a.C + per - 1) / per;
  }
  S = std::max(1, std::min(S, std::min(kMaxWaves, a.C)));
  const size_t shm = S > 1 ? (size_t)S * NT * MTL * 64 * sizeof(f32x4_t) : 0;
  hipLaunchKernelGGL((k_gemv_mfma<NT, MTL>), dim3((unsigned)wgs), dim3(64 * S), shm, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(const GemvArgs& a, hipStream_t s, int nt, int split) {
  // 16 or 32 activation rows per pass (64 would spill); more rows loop passes
  const bool two = a.M > 16;
  if (nt == 1) return two ? launch_nt<1, 2>(a, s, split) : launch_nt<1, 1>(a, s, split);
  return two ? launch_nt<2, 2>(a, s, split) : launch_nt<2, 1>(a, s, split);
}

}  // namespace fp4

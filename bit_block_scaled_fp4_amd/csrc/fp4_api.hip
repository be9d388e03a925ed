// C ABI of libfp4 (declared and documented in include/fp4.h): argument
// checks on the host, then kernel launches on the caller's stream.
#include "../../include/fp4.h"

#include <cstdint>

#include "fp4_internal.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 28;
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxM = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_nk(int64_t N, int64_t K) {
  if (N < 1 || N > kMaxN || K < 16 || K > kMaxK || K % 16 != 0 || N * K > kMaxElems) return FP4_ERR_SHAPE;
  return FP4_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

}  // namespace

extern "C" {

const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "a required pointer is NULL";
    case FP4_ERR_SHAPE: return "size out of range or K not a multiple of 16";
    case FP4_ERR_ALIGN: return "pointer not aligned as required";
    case FP4_ERR_LAYOUT: return "unknown layout tag";
    case FP4_ERR_HIP: return "HIP launch failed";
    case FP4_ERR_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

int fp4_layout_bytes(int64_t N, int64_t K, int layout, size_t* packed_bytes, size_t* scale_bytes) {
  if (!packed_bytes || !scale_bytes) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (layout == FP4_LAYOUT_ROWMAJOR) {
    *packed_bytes = (size_t)(N * K / 2);
    *scale_bytes = (size_t)(N * K / 16);
  } else if (layout == FP4_LAYOUT_TILED) {
    const int64_t tiles = fp4::groups_of(N) * fp4::chunks_of(K);
    *packed_bytes = (size_t)(tiles * fp4::kTileBytes);   // codes and scales share each tile
    *scale_bytes = 0;
  } else {
    return FP4_ERR_LAYOUT;
  }
  return FP4_OK;
}

int fp4_quantize(const void* W_bf16, int64_t N, int64_t K, int layout, void* packed, void* scales,
                 float* gscale, void* stream) {
  if (layout != FP4_LAYOUT_ROWMAJOR && layout != FP4_LAYOUT_TILED) return FP4_ERR_LAYOUT;
  if (!W_bf16 || !packed || !gscale || (layout == FP4_LAYOUT_ROWMAJOR && !scales)) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (!aligned(W_bf16, 16) || !aligned(packed, layout == FP4_LAYOUT_TILED ? 16 : 8) || !aligned(gscale, 4))
    return FP4_ERR_ALIGN;
  return hip_status(fp4::launch_quantize(static_cast<const uint16_t*>(W_bf16), N, K, layout == FP4_LAYOUT_TILED,
                                         static_cast<uint8_t*>(packed), static_cast<uint8_t*>(scales), gscale,
                                         static_cast<hipStream_t>(stream)));
}

int fp4_quantize_fp8(const void* W_fp8, const float* w_scale, int64_t N, int64_t K, int layout, void* packed,
                     void* scales, float* gscale, void* stream) {
  if (layout != FP4_LAYOUT_ROWMAJOR && layout != FP4_LAYOUT_TILED) return FP4_ERR_LAYOUT;
  if (!W_fp8 || !w_scale || !packed || !gscale || (layout == FP4_LAYOUT_ROWMAJOR && !scales)) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (!aligned(W_fp8, 16) || !aligned(packed, layout == FP4_LAYOUT_TILED ? 16 : 8) || !aligned(gscale, 4) ||
      !aligned(w_scale, 4))
    return FP4_ERR_ALIGN;
  // gscale is scratch while the kernels run and w_scale is read by them
  if (static_cast<const void*>(w_scale) == static_cast<const void*>(gscale)) return FP4_ERR_UNSUPPORTED;
  return hip_status(fp4::launch_quantize_fp8(static_cast<const uint8_t*>(W_fp8), w_scale, N, K,
                                             layout == FP4_LAYOUT_TILED, static_cast<uint8_t*>(packed),
                                             static_cast<uint8_t*>(scales), gscale,
                                             static_cast<hipStream_t>(stream)));
}

int fp4_retile(const void* packed_rm, const void* scales_rm, int64_t N, int64_t K, void* packed_tiled,
               void* scales_tiled, void* stream) {
  (void)scales_tiled;   // the tiled layout keeps the scales inside `packed_tiled`
  if (!packed_rm || !scales_rm || !packed_tiled) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (!aligned(packed_rm, 8) || !aligned(packed_tiled, 16)) return FP4_ERR_ALIGN;
  return hip_status(fp4::launch_retile(static_cast<const uint8_t*>(packed_rm), static_cast<const uint8_t*>(scales_rm),
                                       N, K, static_cast<uint8_t*>(packed_tiled), static_cast<hipStream_t>(stream)));
}

// Whether 3 or 4 activation rows go to the matrix cores: at least 32 MiB
// of weights in at most 8 K chunks.
static bool gemv_mma_pays(int64_t groups, int64_t chunks) {
  return chunks <= 8 && groups * chunks * fp4::kTileBytes >= (int64_t(32) << 20);
}

int fp4_gemv_multi(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K, void* stream) {
  if (!projs || !x_bf16) return FP4_ERR_NULL;
  if (nproj < 1 || nproj > FP4_MAX_PROJ || M < 1 || M > kMaxM) return FP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16)) return FP4_ERR_ALIGN;
  fp4::GemvArgs a{};
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.M = (int32_t)M;
  a.K = (int32_t)K;
  a.C = (int32_t)fp4::chunks_of(K);
  a.nproj = nproj;
  int64_t groups = 0;
  for (int i = 0; i < nproj; ++i) {
    const fp4_proj& p = projs[i];
    if (!p.packed || !p.gscale || !p.y) return FP4_ERR_NULL;
    if (int st = check_nk(p.N, K)) return st;
    if (p.ldy < p.N || M * p.ldy > kMaxElems) return FP4_ERR_SHAPE;
    if (!aligned(p.packed, 16) || !aligned(p.y, 4) || !aligned(p.gscale, 4)) return FP4_ERR_ALIGN;
    a.proj[i].tiles = static_cast<const uint8_t*>(p.packed);
    a.proj[i].gscale = p.gscale;
    a.proj[i].y = p.y;
    a.proj[i].ldy = p.ldy;
    a.proj[i].N = (int32_t)p.N;
    groups += fp4::groups_of(p.N);
  }
  if (groups > (int64_t(1) << 30)) return FP4_ERR_SHAPE;
  // Few activation rows: the vector-ALU kernel (decode once, two products per
  // weight and row, no second launch). From five rows on, and from three on
  // large launches with few K chunks, the matrix cores: their 8-row kernel
  // costs about the same at 3 to 8 rows, and their split over K chunks adds
  // a reduce launch that a large launch with few chunks amortises. MI355X, 4
  // rows: fused gate_up 2 x 17408 x 5120 28.2 against 30.7 us, LM head
  // 151936 x 1024 24.3 against 29.8 us; down 5120 x 17408 (17 chunks) 22.8
  // against 21.3 us, so it stays on the vector ALUs.
  if (M <= 4 && !(M >= 3 && gemv_mma_pays(groups, a.C))) return hip_status(fp4::launch_gemv(a, static_cast<hipStream_t>(stream)));
  return hip_status(fp4::launch_gemv_mma(a, static_cast<hipStream_t>(stream)));
}

int fp4_gemv(float* y, const void* x_bf16, const void* packed, const void* scales, const float* gscale, int64_t M,
             int64_t N, int64_t K, void* stream) {
  if (!y || !x_bf16 || !packed || !gscale) return FP4_ERR_NULL;
  fp4_proj p{packed, scales, gscale, N, y, N};   // scales: unused with the tiled layout
  return fp4_gemv_multi(&p, 1, x_bf16, M, K, stream);
}

int fp4_gemm_prefill_multi(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K,
                           void* stream) {
  if (!projs || !x_bf16) return FP4_ERR_NULL;
  if (nproj < 1 || nproj > FP4_MAX_PROJ || M < 1 || M > kMaxM) return FP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16)) return FP4_ERR_ALIGN;
  // the kernel addresses one 256-row slab of x, of each y and of weight
  // tiles with 32-bit buffer offsets
  const int64_t slab = int64_t(1) << 31;
  if (int st = check_nk(8, K)) return st;
  if (256 * K * 2 >= slab || 32 * fp4::chunks_of(K) * fp4::kTileBytes >= slab) return FP4_ERR_SHAPE;
  fp4::PrefillProjDesc d[FP4_MAX_PROJ];
  for (int i = 0; i < nproj; ++i) {
    const fp4_proj& p = projs[i];
    if (!p.packed || !p.gscale || !p.y) return FP4_ERR_NULL;
    if (int st = check_nk(p.N, K)) return st;
    if (p.ldy < p.N || M * p.ldy > kMaxElems || 256 * p.ldy * 4 >= slab) return FP4_ERR_SHAPE;
    if (!aligned(p.packed, 16) || !aligned(p.y, 4) || !aligned(p.gscale, 4)) return FP4_ERR_ALIGN;
    d[i] = {static_cast<const uint8_t*>(p.packed), p.gscale, p.y, p.ldy, p.N};
  }
  return hip_status(fp4::launch_prefill(d, nproj, static_cast<const uint16_t*>(x_bf16), M, K,
                                        static_cast<hipStream_t>(stream)));
}

int fp4_gemm_prefill(float* y, const void* x_bf16, const void* packed, const void* scales, const float* gscale,
                     int64_t M, int64_t N, int64_t K, void* stream) {
  if (!y || !x_bf16 || !packed || !gscale) return FP4_ERR_NULL;
  fp4_proj p{packed, scales, gscale, N, y, N};   // scales: unused with the tiled layout
  return fp4_gemm_prefill_multi(&p, 1, x_bf16, M, K, stream);
}

int fp4_argmax_rows(int32_t* idx, const float* y, int64_t M, int64_t N, int64_t ldy, void* stream) {
  if (!idx || !y) return FP4_ERR_NULL;
  if (M < 1 || M > kMaxM || N < 1 || N > kMaxN || ldy < N || M * ldy > kMaxElems) return FP4_ERR_SHAPE;
  if (!aligned(y, 4) || !aligned(idx, 4)) return FP4_ERR_ALIGN;
  return hip_status(fp4::launch_argmax(idx, y, M, N, ldy, static_cast<hipStream_t>(stream)));
}

int fp4_lm_head_greedy(int32_t* idx, float* logits, const void* x_bf16, const void* packed, const void* scales,
                       const float* gscale, int64_t M, int64_t N, int64_t K, void* stream) {
  // every argument is checked before the first launch
  if (!idx || !logits || !x_bf16 || !packed || !gscale) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (M < 1 || M > kMaxM || M * N > kMaxElems) return FP4_ERR_SHAPE;
  if (!aligned(idx, 4) || !aligned(logits, 4) || !aligned(x_bf16, 16) || !aligned(packed, 16) ||
      !aligned(gscale, 4))
    return FP4_ERR_ALIGN;
  if (int st = fp4_gemv(logits, x_bf16, packed, scales, gscale, M, N, K, stream)) return st;
  return fp4_argmax_rows(idx, logits, M, N, N, stream);
}

}  // extern "C"

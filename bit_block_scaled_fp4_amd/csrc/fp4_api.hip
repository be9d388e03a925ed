// C ABI of libfp4 (declared and documented in include/fp4.h): argument
// checks on the host, then kernel launches on the caller's stream.
#include "../../include/fp4.h"

#include <algorithm>
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
    case FP4_ERR_WORKSPACE: return "workspace smaller than fp4_workspace_bytes reports";
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
  } else if (layout == FP4_LAYOUT_MX_ROWMAJOR || layout == FP4_LAYOUT_MX_TILED || layout == FP4_LAYOUT_MX_ACT) {
    if (K % (layout == FP4_LAYOUT_MX_ACT ? 128 : 32) != 0) return FP4_ERR_SHAPE;
    if (layout != FP4_LAYOUT_MX_TILED) {
      *packed_bytes = (size_t)(N * K / 2);
      *scale_bytes = (size_t)(N * K / 32);
    } else {
      *packed_bytes = (size_t)(fp4::groups_of(N) * fp4::chunks_of(K) * fp4::kMxTileBytes);
      *scale_bytes = 0;
    }
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

int fp4_quantize_mx(const void* W_bf16, int64_t N, int64_t K, int layout, void* packed, void* scales, void* stream) {
  if (layout != FP4_LAYOUT_MX_ROWMAJOR && layout != FP4_LAYOUT_MX_TILED && layout != FP4_LAYOUT_MX_ACT)
    return FP4_ERR_LAYOUT;
  if (!W_bf16 || !packed || (layout != FP4_LAYOUT_MX_TILED && !scales)) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (K % (layout == FP4_LAYOUT_MX_ACT ? 128 : 32) != 0) return FP4_ERR_SHAPE;
  if (!aligned(W_bf16, 16) || !aligned(packed, 16)) return FP4_ERR_ALIGN;
  return hip_status(fp4::launch_quantize_mx(static_cast<const uint16_t*>(W_bf16), N, K,
                                            layout == FP4_LAYOUT_MX_TILED ? 1 : layout == FP4_LAYOUT_MX_ACT ? 2 : 0,
                                            static_cast<uint8_t*>(packed), static_cast<uint8_t*>(scales),
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
// of weights.
static bool gemv_mma_pays(int64_t groups, int64_t chunks) {
  return groups * chunks * fp4::kTileBytes >= (int64_t(32) << 20);
}

// Few activation rows: the vector-ALU kernel (decode once, two products per
// weight and row). From five rows on, and from three on large launches, the
// matrix cores: their 8-row kernel costs about the same at 3 to 8 rows.
// MI355X, graph-timed with a workspace, vector ALUs against matrix cores at
// 3 / 4 rows: fused gate_up 2 x 17408 x 5120 at 4 rows 30.3 against 25.6
// us; down 5120 x 17408 19.4 / 18.9 against 16.5 / 16.5; 8192 x 28672 39.5
// / 37.3 against 34.2 / 34.0; 4096 x 14336 (33 MB) 14.0 / 13.1 against 12.5
// / 12.7; 28672 x 8192 46.0 / 44.2 against 32.1 / 32.0; 2048 x 65536 (64
// chunks) 26.0 / 23.8 against 23.8 / 23.9.
static bool gemv_on_valu(const fp4::GemvArgs& a) {
  int64_t groups = 0;
  for (int i = 0; i < a.nproj; ++i) groups += fp4::groups_of(a.proj[i].N);
  return a.M <= 4 && !(a.M >= 3 && gemv_mma_pays(groups, a.C));
}

// Checks the projections of a fused product and fills `a`.
static int gemv_args(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K, fp4::GemvArgs& a) {
  if (!projs || !x_bf16) return FP4_ERR_NULL;
  if (nproj < 1 || nproj > FP4_MAX_PROJ || M < 1 || M > kMaxM) return FP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16)) return FP4_ERR_ALIGN;
  a = fp4::GemvArgs{};
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
  return FP4_OK;
}

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Bytes of partial sums a product with these arguments keeps in scratch (0:
// none; the vector ALUs and one K chunk keep none).
static size_t gemv_partials(const fp4::GemvArgs& a) { return gemv_on_valu(a) ? 0 : fp4::gemv_mma_partial_bytes(a); }

// Workspace bytes a product with these arguments uses (0: none).
static size_t gemv_ws_need(const fp4::GemvArgs& a) {
  const size_t p = gemv_partials(a);
  return p ? fp4::kWsHeaderBytes + p : 0;
}

// A caller's workspace: NULL means none; otherwise 256-byte aligned and at
// least `need` bytes.
static int take_ws(void* workspace, size_t bytes, size_t need, fp4::Workspace& ws) {
  ws = fp4::Workspace{};
  if (!workspace) return FP4_OK;
  if (!aligned(workspace, 256)) return FP4_ERR_ALIGN;
  if (bytes < need) return FP4_ERR_WORKSPACE;
  ws.p = static_cast<uint8_t*>(workspace);
  ws.bytes = bytes;
  return FP4_OK;
}

// The product; `scratch` (may be null) holds its partial sums.
static int gemv_run(const fp4::GemvArgs& a, const fp4::Workspace& ws, uint8_t* scratch, hipStream_t s) {
  if (gemv_on_valu(a)) return hip_status(fp4::launch_gemv(a, s));
  return hip_status(fp4::launch_gemv_mma(a, reinterpret_cast<float*>(scratch), ws.valid() ? ws.counter(0) : nullptr, s));
}

static uint8_t* scratch_of(const fp4::Workspace& ws) { return ws.valid() ? ws.scratch() : nullptr; }

int fp4_gemv_multi_ws(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K, void* workspace,
                      size_t workspace_bytes, void* stream) {
  fp4::GemvArgs a;
  if (int st = gemv_args(projs, nproj, x_bf16, M, K, a)) return st;
  fp4::Workspace ws;
  if (int st = take_ws(workspace, workspace_bytes, gemv_ws_need(a), ws)) return st;
  return gemv_run(a, ws, scratch_of(ws), static_cast<hipStream_t>(stream));
}

int fp4_gemv_multi(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K, void* stream) {
  return fp4_gemv_multi_ws(projs, nproj, x_bf16, M, K, nullptr, 0, stream);
}

int fp4_gemv_ws(float* y, const void* x_bf16, const void* packed, const void* scales, const float* gscale, int64_t M,
                int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (!y || !x_bf16 || !packed || !gscale) return FP4_ERR_NULL;
  fp4_proj p{packed, scales, gscale, N, y, N};   // scales: unused with the tiled layout
  return fp4_gemv_multi_ws(&p, 1, x_bf16, M, K, workspace, workspace_bytes, stream);
}

int fp4_gemv(float* y, const void* x_bf16, const void* packed, const void* scales, const float* gscale, int64_t M,
             int64_t N, int64_t K, void* stream) {
  return fp4_gemv_ws(y, x_bf16, packed, scales, gscale, M, N, K, nullptr, 0, stream);
}

// Checks the projections of a fused prefill product and fills `d`.
static int prefill_args(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K,
                        fp4::PrefillProjDesc (&d)[FP4_MAX_PROJ]) {
  if (!projs || !x_bf16) return FP4_ERR_NULL;
  if (nproj < 1 || nproj > FP4_MAX_PROJ || M < 1 || M > kMaxM) return FP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16)) return FP4_ERR_ALIGN;
  // the kernel addresses one 256-row slab of x, of each y and of weight
  // tiles with 32-bit buffer offsets
  const int64_t slab = int64_t(1) << 31;
  if (int st = check_nk(8, K)) return st;
  if (256 * K * 2 >= slab || 32 * fp4::chunks_of(K) * fp4::kTileBytes >= slab) return FP4_ERR_SHAPE;
  for (int i = 0; i < nproj; ++i) {
    const fp4_proj& p = projs[i];
    if (!p.packed || !p.gscale || !p.y) return FP4_ERR_NULL;
    if (int st = check_nk(p.N, K)) return st;
    if (p.ldy < p.N || M * p.ldy > kMaxElems || 256 * p.ldy * 4 >= slab) return FP4_ERR_SHAPE;
    if (!aligned(p.packed, 16) || !aligned(p.y, 4) || !aligned(p.gscale, 4)) return FP4_ERR_ALIGN;
    d[i] = {static_cast<const uint8_t*>(p.packed), p.gscale, p.y, p.ldy, p.N};
  }
  return FP4_OK;
}

int fp4_gemm_prefill_multi_ws(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream) {
  fp4::PrefillProjDesc d[FP4_MAX_PROJ];
  if (int st = prefill_args(projs, nproj, x_bf16, M, K, d)) return st;
  fp4::Workspace ws;
  const size_t need = workspace ? fp4::prefill_ws_bytes(d, nproj, M, K) : 0;
  if (int st = take_ws(workspace, workspace_bytes, need, ws)) return st;
  return hip_status(fp4::launch_prefill(d, nproj, static_cast<const uint16_t*>(x_bf16), M, K, ws,
                                        static_cast<hipStream_t>(stream)));
}

int fp4_gemm_prefill_multi(const fp4_proj* projs, int nproj, const void* x_bf16, int64_t M, int64_t K,
                           void* stream) {
  return fp4_gemm_prefill_multi_ws(projs, nproj, x_bf16, M, K, nullptr, 0, stream);
}

int fp4_gemm_prefill_ws(float* y, const void* x_bf16, const void* packed, const void* scales, const float* gscale,
                        int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (!y || !x_bf16 || !packed || !gscale) return FP4_ERR_NULL;
  fp4_proj p{packed, scales, gscale, N, y, N};   // scales: unused with the tiled layout
  return fp4_gemm_prefill_multi_ws(&p, 1, x_bf16, M, K, workspace, workspace_bytes, stream);
}

int fp4_gemm_prefill(float* y, const void* x_bf16, const void* packed, const void* scales, const float* gscale,
                     int64_t M, int64_t N, int64_t K, void* stream) {
  return fp4_gemm_prefill_ws(y, x_bf16, packed, scales, gscale, M, N, K, nullptr, 0, stream);
}

static int argmax_check(const int32_t* idx, const float* y, int64_t M, int64_t N, int64_t ldy) {
  if (!idx || !y) return FP4_ERR_NULL;
  if (M < 1 || M > kMaxM || N < 1 || N > kMaxN || ldy < N || M * ldy > kMaxElems) return FP4_ERR_SHAPE;
  if (!aligned(y, 4) || !aligned(idx, 4)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

int fp4_argmax_rows(int32_t* idx, const float* y, int64_t M, int64_t N, int64_t ldy, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (int st = argmax_check(idx, y, M, N, ldy)) return st;
  fp4::Workspace ws;
  if (int st = take_ws(workspace, workspace_bytes, fp4::argmax_ws_bytes(M, N), ws)) return st;
  return hip_status(fp4::launch_argmax(idx, y, M, N, ldy, ws, static_cast<hipStream_t>(stream)));
}

// The greedy step's plan: the product launch itself ends with the choice
// (one launch) when a workspace is given, the product runs on the vector
// ALUs (its every workgroup covers all rows) and the workgroups' keys fit in
// the workspace header; otherwise the product, then fp4_argmax_rows' kernel.
// On the matrix cores the epilogue measured slower than the second launch
// (MI355X, LM head 151936 x 1024: M = 3 +7.2 against +5.4 us, M = 8 +8.6
// against +6.6 us; vector ALUs, M = 1: +4.4 against +5.9 us).
static bool greedy_fused(const fp4::GemvArgs& a) {
  if (!gemv_on_valu(a)) return false;
  return fp4::greedy_keys_fit(a.M, fp4::gemv_workgroups(a));
}

static size_t greedy_ws_need(const fp4::GemvArgs& a, int64_t N) {
  if (greedy_fused(a)) return fp4::kWsHeaderBytes;
  return std::max(gemv_ws_need(a), fp4::argmax_ws_bytes(a.M, N));
}

static int greedy_args(int32_t* idx, float* logits, const void* x_bf16, const void* packed, const float* gscale,
                       int64_t M, int64_t N, int64_t K, fp4::GemvArgs& a) {
  if (!idx || !logits || !x_bf16 || !packed || !gscale) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (M < 1 || M > kMaxM || M * N > kMaxElems) return FP4_ERR_SHAPE;
  if (!aligned(idx, 4) || !aligned(logits, 4) || !aligned(x_bf16, 16) || !aligned(packed, 16) ||
      !aligned(gscale, 4))
    return FP4_ERR_ALIGN;
  fp4_proj p{packed, nullptr, gscale, N, logits, N};
  return gemv_args(&p, 1, x_bf16, M, K, a);
}

int fp4_lm_head_greedy(int32_t* idx, float* logits, const void* x_bf16, const void* packed, const void* scales,
                       const float* gscale, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       void* stream) {
  (void)scales;   // unused with the tiled layout
  // every argument is checked before the first launch
  fp4::GemvArgs a;
  if (int st = greedy_args(idx, logits, x_bf16, packed, gscale, M, N, K, a)) return st;
  fp4::Workspace ws;
  if (int st = take_ws(workspace, workspace_bytes, workspace ? greedy_ws_need(a, N) : 0, ws)) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (ws.valid() && greedy_fused(a)) {
    a.greedy.idx = idx;
    a.greedy.keys = reinterpret_cast<uint64_t*>(ws.p);   // the header: zero between calls
    return gemv_run(a, ws, scratch_of(ws), s);
  }
  if (int st = gemv_run(a, ws, scratch_of(ws), s)) return st;
  return hip_status(fp4::launch_argmax(idx, logits, M, N, N, ws, s));
}

// RMS normalisation before the products: inside the vector-ALU launch for
// up to 2 rows (3-4 rows would spill there), else a norm kernel writing the
// normalised rows into the workspace, then the product on them.
static bool rms_fused(const fp4::GemvArgs& a) { return gemv_on_valu(a) && a.M <= 2; }

static size_t rms_ws_need(const fp4::GemvArgs& a) {
  if (rms_fused(a)) return 0;
  return fp4::kWsHeaderBytes + align256((size_t)a.M * (size_t)a.K * 2) + gemv_partials(a);
}

static int rms_check(const void* gain_bf16, float eps) {
  if (!gain_bf16) return FP4_ERR_NULL;
  if (!aligned(gain_bf16, 16)) return FP4_ERR_ALIGN;
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return FP4_ERR_SHAPE;   // finite, not negative, not NaN
  return FP4_OK;
}

int fp4_gemv_multi_rmsnorm(const fp4_proj* projs, int nproj, const void* x_bf16, const void* gain_bf16, float eps,
                           int64_t M, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  fp4::GemvArgs a;
  if (int st = gemv_args(projs, nproj, x_bf16, M, K, a)) return st;
  if (int st = rms_check(gain_bf16, eps)) return st;
  const size_t need = rms_ws_need(a);
  fp4::Workspace ws;
  if (int st = take_ws(workspace, workspace_bytes, need, ws)) return st;
  if (need > 0 && !ws.valid()) return FP4_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (rms_fused(a)) {
    a.gain = static_cast<const uint16_t*>(gain_bf16);
    a.eps = eps;
    return gemv_run(a, fp4::Workspace{}, nullptr, s);
  }
  uint16_t* xn = reinterpret_cast<uint16_t*>(ws.scratch());
  if (int st = hip_status(fp4::launch_rmsnorm(a.x, static_cast<const uint16_t*>(gain_bf16), eps, M, K, xn, s))) return st;
  a.x = xn;
  return gemv_run(a, ws, ws.scratch() + align256((size_t)M * (size_t)K * 2), s);
}

// The gated MLP's first half: one vector-ALU launch computing gate and up and
// writing h when the pair runs there, else the pair's product into fp32
// buffers in the workspace, then an elementwise kernel.
static int swiglu_args(void* h_bf16, int64_t ldh, const void* x_bf16, const void* gate_packed, const float* gate_gscale,
                       const void* up_packed, const float* up_gscale, int64_t M, int64_t N, int64_t K,
                       fp4::GemvArgs& a) {
  if (!h_bf16 || !gate_packed || !up_packed || !gate_gscale || !up_gscale) return FP4_ERR_NULL;
  if (ldh < N || M < 1 || M > kMaxM || M * ldh > kMaxElems) return FP4_ERR_SHAPE;
  if (!aligned(h_bf16, 2)) return FP4_ERR_ALIGN;
  static float stand_in __attribute__((aligned(16)));   // validated as y, never written
  fp4_proj p[2] = {{gate_packed, nullptr, gate_gscale, N, &stand_in, N}, {up_packed, nullptr, up_gscale, N, &stand_in, N}};
  if (int st = gemv_args(p, 2, x_bf16, M, K, a)) return st;
  a.h = static_cast<uint16_t*>(h_bf16);
  a.ldh = ldh;
  return FP4_OK;
}

static size_t swiglu_ws_need(const fp4::GemvArgs& a) {
  if (gemv_on_valu(a)) return 0;
  const size_t gu = align256((size_t)a.M * (size_t)a.proj[0].N * 4);
  return fp4::kWsHeaderBytes + 2 * gu + gemv_partials(a);
}

int fp4_gemv_swiglu(void* h_bf16, int64_t ldh, const void* x_bf16, const void* gate_packed, const float* gate_gscale,
                    const void* up_packed, const float* up_gscale, int64_t M, int64_t N, int64_t K, void* workspace,
                    size_t workspace_bytes, void* stream) {
  fp4::GemvArgs a;
  if (int st = swiglu_args(h_bf16, ldh, x_bf16, gate_packed, gate_gscale, up_packed, up_gscale, M, N, K, a)) return st;
  const size_t need = swiglu_ws_need(a);
  fp4::Workspace ws;
  if (int st = take_ws(workspace, workspace_bytes, need, ws)) return st;
  if (need > 0 && !ws.valid()) return FP4_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (gemv_on_valu(a)) return hip_status(fp4::launch_gemv_swiglu(a, s));
  const size_t gu = align256((size_t)M * (size_t)N * 4);
  float* g = reinterpret_cast<float*>(ws.scratch());
  float* u = reinterpret_cast<float*>(ws.scratch() + gu);
  a.proj[0].y = g;
  a.proj[1].y = u;
  a.proj[0].ldy = a.proj[1].ldy = N;
  a.h = nullptr;
  if (int st = gemv_run(a, ws, ws.scratch() + 2 * gu, s)) return st;
  return hip_status(fp4::launch_swiglu(g, u, M, N, static_cast<uint16_t*>(h_bf16), ldh, s));
}

// MXFP4 products: the same argument rules with the MX tiled layout, K % 32
// == 0 and no tensor scale.
static int mx_args(float* y, const void* x_bf16, const void* packed, int64_t M, int64_t N, int64_t K,
                   fp4::GemvArgs& a) {
  if (!y || !x_bf16 || !packed) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (K % 32 != 0 || M < 1 || M > kMaxM || M * N > kMaxElems) return FP4_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(packed, 16) || !aligned(y, 4)) return FP4_ERR_ALIGN;
  a = fp4::GemvArgs{};
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.M = (int32_t)M;
  a.K = (int32_t)K;
  a.C = (int32_t)fp4::chunks_of(K);
  a.nproj = 1;
  a.proj[0].tiles = static_cast<const uint8_t*>(packed);
  a.proj[0].y = y;
  a.proj[0].ldy = N;
  a.proj[0].N = (int32_t)N;
  a.mx = 1;
  return FP4_OK;
}

int fp4_gemv_mx(float* y, const void* x_bf16, const void* packed, int64_t M, int64_t N, int64_t K, void* stream) {
  fp4::GemvArgs a;
  if (int st = mx_args(y, x_bf16, packed, M, N, K, a)) return st;
  return hip_status(fp4::launch_gemv(a, static_cast<hipStream_t>(stream)));
}

int fp4_gemm_prefill_mx(float* y, const void* x_bf16, const void* packed, int64_t M, int64_t N, int64_t K,
                        void* stream) {
  fp4::GemvArgs a;
  if (int st = mx_args(y, x_bf16, packed, M, N, K, a)) return st;
  static const float one = 1.0f;   // the descriptor's scale pointer; the MX kernels read none
  fp4_proj p{packed, nullptr, &one, N, y, N};
  fp4::PrefillProjDesc d[FP4_MAX_PROJ];
  if (int st = prefill_args(&p, 1, x_bf16, M, K, d)) return st;
  return hip_status(fp4::launch_prefill(d, 1, static_cast<const uint16_t*>(x_bf16), M, K, fp4::Workspace{},
                                        static_cast<hipStream_t>(stream), 0, 0, true));
}

int fp4_gemm_mx_a4(float* y, const void* xq_packed, const void* xq_scales, const void* packed, int64_t M, int64_t N,
                   int64_t K, void* stream) {
  if (!y || !xq_packed || !xq_scales || !packed) return FP4_ERR_NULL;
  if (int st = check_nk(N, K)) return st;
  if (K % 128 != 0 || M < 1 || M > 65535 * 256 || M * N > kMaxElems || M * (K / 32) >= (int64_t(1) << 31))
    return FP4_ERR_SHAPE;
  if ((N + 7) / 8 * fp4::chunks_of(K) * fp4::kMxTileBytes >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;
  if (!aligned(xq_packed, 16) || !aligned(packed, 16) || !aligned(xq_scales, 4) || !aligned(y, 4)) return FP4_ERR_ALIGN;
  return hip_status(fp4::launch_mx_a4(y, static_cast<const uint8_t*>(xq_packed), static_cast<const uint8_t*>(xq_scales),
                                      static_cast<const uint8_t*>(packed), M, N, K, static_cast<hipStream_t>(stream)));
}

int fp4_workspace_bytes(int op, int64_t M, int64_t K, const int64_t* Ns, int nproj, size_t* bytes) {
  if (!bytes || !Ns) return FP4_ERR_NULL;
  if (nproj < 1 || nproj > FP4_MAX_PROJ || M < 1 || M > kMaxM) return FP4_ERR_SHAPE;
  *bytes = 0;
  // the planners read only shapes: stand-in pointers, never dereferenced
  static const uint8_t stand_in[16] __attribute__((aligned(16))) = {};
  void* const sp = const_cast<uint8_t*>(stand_in);
  fp4_proj p[FP4_MAX_PROJ];
  for (int i = 0; i < nproj; ++i) p[i] = fp4_proj{sp, nullptr, static_cast<float*>(sp), Ns[i], static_cast<float*>(sp), Ns[i]};
  switch (op) {
    case FP4_OP_GEMV: {
      fp4::GemvArgs a;
      if (int st = gemv_args(p, nproj, sp, M, K, a)) return st;
      *bytes = gemv_ws_need(a);
      return FP4_OK;
    }
    case FP4_OP_GEMM_PREFILL: {
      fp4::PrefillProjDesc d[FP4_MAX_PROJ];
      if (int st = prefill_args(p, nproj, sp, M, K, d)) return st;
      *bytes = fp4::prefill_ws_bytes(d, nproj, M, K);
      return FP4_OK;
    }
    case FP4_OP_ARGMAX_ROWS: {
      if (nproj != 1) return FP4_ERR_SHAPE;
      if (Ns[0] < 1 || Ns[0] > kMaxN || M * Ns[0] > kMaxElems) return FP4_ERR_SHAPE;
      *bytes = fp4::argmax_ws_bytes(M, Ns[0]);
      return FP4_OK;
    }
    case FP4_OP_GEMV_RMSNORM: {
      fp4::GemvArgs a;
      if (int st = gemv_args(p, nproj, sp, M, K, a)) return st;
      *bytes = rms_ws_need(a);
      return FP4_OK;
    }
    case FP4_OP_GEMV_SWIGLU: {
      if (nproj != 1) return FP4_ERR_SHAPE;
      fp4::GemvArgs a;
      if (int st = swiglu_args(sp, Ns[0], sp, sp, static_cast<float*>(sp), sp, static_cast<float*>(sp), M, Ns[0], K, a))
        return st;
      *bytes = swiglu_ws_need(a);
      return FP4_OK;
    }
    case FP4_OP_LM_HEAD_GREEDY: {
      if (nproj != 1) return FP4_ERR_SHAPE;
      fp4::GemvArgs a;
      int32_t* const ip = static_cast<int32_t*>(sp);
      if (int st = greedy_args(ip, static_cast<float*>(sp), sp, sp, static_cast<float*>(sp), M, Ns[0], K, a)) return st;
      *bytes = greedy_ws_need(a, Ns[0]);
      return FP4_OK;
    }
    default:
      return FP4_ERR_UNSUPPORTED;
  }
}

}  // extern "C"

/*
 * fp4.h: C ABI of the NVFP4 decode-path library for AMD Instinct MI355X
 * (gfx950). Built as libfp4.so from bit_block_scaled_fp4_amd/csrc/.
 *
 * What it computes. Decode in an LLM engine is bandwidth-bound: every weight
 * is read once per generated token and the arithmetic is trivial, so the
 * weights are kept in 4 bits and multiplied without first expanding them to
 * 16 bits (page "imp" README, the decode paragraph of the request
 * walkthrough; page "1. The big picture", section "The most important
 * number in this book", whose ceiling tokens/s <= bandwidth / bytes per token
 * is the roofline used to judge these kernels). Shrinking the weights at load
 * time is "the biggest single lever" for decode (page "How imp turns a model
 * file into words", Part one: loading the model).
 *
 * Format (NVFP4: four-bit values and two scales, as the engineering log's post
 * "NVFP4 at the bit level" describes it):
 *   - element: FP4 E2M1 (OCP MX v1.0), values {0,0.5,1,1.5,2,3,4,6} with sign,
 *     two per byte, the even K index in the low nibble;
 *   - block scale: one FP8 E4M3 (OCP "fn": max 448, no infinities) per 16
 *     consecutive K elements of a row;
 *   - tensor scale gscale: one fp32 decode multiplier per tensor.
 *   dequant(W)[n][k] = E2M1(q[n][k]) * E4M3(sc[n][k/16]) * gscale.
 *
 * Shapes. W is [N][K] (N output features, K input features), x is bf16
 * [M][K] row-major, y is fp32 [M][N] row-major (y[m*ldy + n]).
 * y[m][n] = sum_k dequant(W)[n][k] * x[m][k]. K must be a multiple of 16.
 *
 * Layouts of the quantised weights (see fp4_layout_bytes for sizes):
 *   FP4_LAYOUT_ROWMAJOR (canonical): packed [N][K/2] bytes, scales [N][K/16]
 *     bytes, both row-major.
 *   FP4_LAYOUT_TILED (device layout read by fp4_gemv, fp4_gemv_multi and
 *     fp4_gemm_prefill): ONE buffer, `packed`, holding codes and scales.
 *     Rows form groups of 8 (G = ceil(N/8)), K forms chunks of 1024
 *     (C = ceil(K/1024)); tile (g, c) is the 4608 bytes at (g*C + c)*4608:
 *       byte r*512 + l*16 + i          = canonical packed byte
 *                                        (row 8g+r, byte 512c + 16l + i),
 *       byte 4096 + h*256 + l*8 + 2i + j = scale of
 *                                        (row 8g + 2i + h, block 64c + 2l + j),
 *     for r < 8, l < 32, i < 16 (codes) or i < 4 (scales), h < 2, j < 2.
 *     Positions outside the tensor hold 0. A 64-lane wave thus reads rows
 *     2q and 2q+1 of a tile as one contiguous kilobyte (lane 32h + l gets
 *     piece l, two whole 16-element blocks, of row 2q + h) and finds the 8
 *     scale bytes it needs for its four rows at 4096 + 8*lane, so the block
 *     scales travel in the same stream as the codes. The `scales` arguments
 *     of the calls below are unused with this layout (pass NULL).
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device memory (e.g. a torch CUDA
 *     tensor's data_ptr()) on the current HIP device; the caller owns every
 *     buffer. The library allocates nothing and keeps no state between
 *     calls (it caches each device's compute-unit count, a device property).
 *   - Workspaces. Some products split work over workgroups whose partial
 *     results meet in scratch memory. That memory is a caller-owned device
 *     buffer, the workspace, passed to the *_ws forms and to the greedy
 *     calls; fp4_workspace_bytes gives the size a call needs. A workspace is
 *     256-byte aligned and filled with zeros once before its first use (e.g.
 *     hipMemset after allocating it). Its first 64 KiB are counters that
 *     every call leaves at zero when its kernels complete; the bytes after
 *     them are scratch that a call overwrites. One workspace can therefore
 *     serve any sequence of calls that run one after another (one stream, or
 *     a graph replayed on one stream); calls that may run at the same time
 *     need separate workspaces. A NULL workspace selects paths that need
 *     none (documented at each call), so the calls without a workspace
 *     argument never touch memory other than their arguments, and calls on
 *     different streams never share memory unless their arguments do.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only
 *     enqueue work: they never synchronise, and results are ready when the
 *     stream's work is. gscale is a device pointer, so quantise -> multiply
 *     is stream-ordered and can be captured in a HIP graph.
 *   - Arguments are checked on the host before any HIP call; on an error
 *     nothing is enqueued and the status says why. FP4_ERR_HIP means the
 *     launch itself failed. A fault inside a kernel surfaces at the
 *     caller's next synchronisation, as usual for HIP.
 *   - Alignment: x, W and tiled buffers must be 16-byte aligned (canonical
 *     packed data: 8-byte; canonical scales: none); y and gscale 4-byte
 *     aligned.
 *   - Size limits: 1 <= N <= 2^28, 16 <= K <= 2^24, 1 <= M <= 2^24.
 *   - Calls may be made from several host threads at once.
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define FP4_API __attribute__((visibility("default")))
#else
#define FP4_API
#endif

typedef enum {
    FP4_OK = 0,
    FP4_ERR_NULL = -1,        /* a required pointer is NULL */
    FP4_ERR_SHAPE = -2,       /* a size is out of range or K % 16 != 0 */
    FP4_ERR_ALIGN = -3,       /* a pointer is not aligned as required */
    FP4_ERR_LAYOUT = -4,      /* unknown layout tag */
    FP4_ERR_HIP = -5,         /* the HIP runtime rejected a launch */
    FP4_ERR_UNSUPPORTED = -6, /* valid request the library cannot serve */
    FP4_ERR_WORKSPACE = -7    /* workspace smaller than fp4_workspace_bytes reports */
} fp4_status;

typedef enum {
    FP4_LAYOUT_ROWMAJOR = 0,     /* NVFP4, canonical */
    FP4_LAYOUT_TILED = 1,        /* NVFP4, device tiles */
    FP4_LAYOUT_MX_ROWMAJOR = 2,  /* MXFP4, canonical: packed [N][K/2], E8M0 scales [N][K/32] */
    FP4_LAYOUT_MX_TILED = 3,     /* MXFP4, device tiles of 4352 bytes (below) */
    FP4_LAYOUT_MX_ACT = 4        /* MXFP4 activation operand of fp4_gemm_mx_a4 (below) */
} fp4_layout;

/* Human-readable text for a status code (static storage, never NULL). */
FP4_API const char *fp4_status_string(int status);

/* Bytes of the packed and scale arrays for an N x K weight in `layout`.
 * ROWMAJOR: N*K/2 and N*K/16. TILED: G*C*4608 and 0 (the scales live in
 * the tiles, see above). MX_ROWMAJOR and MX_ACT: N*K/2 and N*K/32; MX_TILED:
 * G*C*4352 and 0 (K % 32 == 0; MX_ACT K % 128 == 0). Host-only; enqueues
 * nothing. */
FP4_API int fp4_layout_bytes(int64_t N, int64_t K, int layout, size_t *packed_bytes, size_t *scale_bytes);

/* Quantise a bf16 weight W [N][K] (device) to NVFP4 in `layout`, writing
 * packed and scales (device, sized by fp4_layout_bytes; TILED writes codes
 * and scales into `packed` and ignores `scales`, which may be NULL) and the
 * tensor scale *gscale (device fp32). The rule, one fp32 IEEE operation per step:
 *   gscale = amax|W| / 2688 (= 448*6; 0 for an all-zero W);
 *   per block s = (block_amax / 6) / gscale, scale code = E4M3 nearest-even
 *   of s, saturating at 448;
 *   per element code = E2M1 nearest-even of w / (E4M3(code) * gscale),
 *   saturating at 6, sign from the sign bit (-0 for small negatives);
 *   a block whose scale code is 0 gets element codes 0.
 * The bytes are unique under this rule. W must hold finite values. Padding
 * positions of the tiled layout are written as 0. Uses *gscale as scratch
 * while it runs. (Load-time step of the engine tour's Part one: shrinking
 * every weight once, on the GPU.) */
FP4_API int fp4_quantize(const void *W_bf16, int64_t N, int64_t K, int layout, void *packed, void *scales,
                 float *gscale, void *stream);

/* MXFP4, the other block-scaled four-bit format in the imp README's
 * quantisation row, read as OCP Microscaling v1.0: the same E2M1 elements,
 * one E8M0 scale (an exponent, value 2^(c - 127)) per 32 consecutive
 * K-elements, no tensor scale. Quantise bf16 W [N][K] (K % 32 == 0) in one
 * pass: per block the shared exponent floor(log2(amax)) - 2 clamped to
 * [-127, 127], stored as code shared + 127; element code = E2M1 nearest-even
 * of w / 2^shared, saturating at 6, sign from the sign bit; a block with
 * amax 0 gets scale 0 and codes 0. layout MX_ROWMAJOR writes packed and
 * scales; MX_TILED writes the tiles into `packed` (scales unused): rows in
 * groups of 8, K in chunks of 1024, tile (g, c) the 4352 bytes at
 * (g*C + c)*4352, codes as in the NVFP4 tile, then byte 4096 + h*128 + l*4 + i
 * = scale of (row 8g + 2i + h, block 32c + l). MX_ACT (K % 128 == 0) writes
 * the codes as MX_ROWMAJOR and the scales grouped by 128-column step: the
 * scale of (row n, block b) at ((b / 4) * N + n) * 4 + b % 4, so one step's
 * scales of consecutive rows are contiguous. The bytes are unique. */
FP4_API int fp4_quantize_mx(const void *W_bf16, int64_t N, int64_t K, int layout, void *packed, void *scales,
                            void *stream);

/* y[M][N] = x * dequant(W)^T for MX_TILED weights W (dequant = E2M1 *
 * E8M0), fp32 accumulation, y overwritten. Every M runs on the vector-ALU
 * kernel (more than 4 rows in passes of 4 inside one launch). */
FP4_API int fp4_gemv_mx(float *y, const void *x_bf16, const void *packed, int64_t M, int64_t N, int64_t K,
                        void *stream);

/* The same product on the matrix cores for prefill-sized M (the prefill
 * kernel of fp4_gemm_prefill reading MX tiles: E2M1 * 2^(c - 127) decoded
 * exactly to bf16 MFMA operands). No K split of the last round of tiles. */
FP4_API int fp4_gemm_prefill_mx(float *y, const void *x_bf16, const void *packed, int64_t M, int64_t N, int64_t K,
                                void *stream);

/* Both operands MXFP4, on gfx950's block-scaled FP4 matrix cores (page
 * "github.com/kekzl/imp", the feature table: MXFP4 in the quantisation
 * row, a block-scaled GEMM in the engine row). y[M][N] (fp32, ldy = N,
 * overwritten) = dequant(xq) * dequant(W)^T, where xq holds the activation
 * rows x[M][K] quantised by fp4_quantize_mx with layout MX_ACT (codes
 * [M][K/2], E8M0 scales [K/128][M][4], device) and W is an MX_TILED
 * weight. Each product of two scaled E2M1 values is exact and the sums
 * are fp32, so y matches that definition closely; against the product with
 * bf16 activations (fp4_gemm_prefill_mx) it carries the activations' own
 * quantisation error (E2M1 keeps one mantissa bit), in exchange for the
 * matrix cores' FP4 rate. K % 128 == 0, M <= 16776960 and M*K/32 < 2^31
 * (FP4_ERR_SHAPE otherwise), the tiles below 2^31 bytes; xq_packed and packed 16-byte
 * aligned, xq_scales and y 4-byte aligned. No workspace, nothing
 * allocated. */
FP4_API int fp4_gemm_mx_a4(float *y, const void *xq_packed, const void *xq_scales, const void *packed, int64_t M,
                           int64_t N, int64_t K, void *stream);

/* The same quantisation for a checkpoint released in FP8 (the imp README:
 * its quantiser builds NVFP4 weights from BF16 or FP8 releases). W_fp8 is
 * [N][K] OCP E4M3 ("fn") codes, one byte per element (device, 16-byte
 * aligned); *w_scale (device fp32) is the tensor's dequantisation scale.
 * Element values are E4M3(code) * *w_scale, rounded once to fp32; from there
 * the rule, layouts, outputs and gscale are exactly those of fp4_quantize.
 * The NaN codes 0x7F and 0xFF are outside the domain (results unspecified),
 * like non-finite bf16 input; *w_scale must be finite. w_scale must not be
 * the gscale pointer (FP4_ERR_UNSUPPORTED): gscale is scratch while the
 * kernels run. */
FP4_API int fp4_quantize_fp8(const void *W_fp8, const float *w_scale, int64_t N, int64_t K, int layout,
                             void *packed, void *scales, float *gscale, void *stream);

/* Re-tile canonical (ROWMAJOR) packed/scales into the TILED layout, written
 * to `packed_tiled` (scales_tiled is unused and may be NULL). A pure byte
 * permutation plus zero padding; inputs and outputs must not overlap.
 * (The README's load-time weight transformation, cached across starts.) */
FP4_API int fp4_retile(const void *packed_rm, const void *scales_rm, int64_t N, int64_t K, void *packed_tiled,
               void *scales_tiled, void *stream);

/* y[M][N] = x[M][K] * dequant(W)^T for TILED weights, fp32 accumulation,
 * y overwritten (fp32, ldy = N). The decode-step matrix-vector product
 * (M = 1) and its small-M form, where several rows (concurrent streams,
 * or tokens being verified by speculative decoding) share one pass over
 * the weights (page "1. The big picture", the batching and speculative
 * decoding bullets of "The most important number in this book").
 * Any M >= 1 is accepted. `packed` holds the tiles; `scales` is unused.
 * Up to 4 rows run on the vector ALUs (3-4 rows of a launch reading at
 * least 32 MiB of weights aside), more on the matrix cores in passes of 16
 * rows.
 * The matrix-core path splits K into chunks of 1024 over workgroups; with
 * more than one chunk this call (no workspace) first zeroes y with a fill
 * kernel and adds the chunk sums into y with fp32 atomics, so the last
 * bits of y can differ between calls. fp4_gemv_ws adds them in chunk order
 * through a workspace instead (deterministic). */
FP4_API int fp4_gemv(float *y, const void *x_bf16, const void *packed, const void *scales, const float *gscale,
             int64_t M, int64_t N, int64_t K, void *stream);

/* fp4_gemv with a workspace (see Conventions; NULL = fp4_gemv). A chunked
 * matrix-core product keeps the chunk partial sums in the workspace and adds
 * them in chunk order (inside the launch for passes of at most 8 rows, in a
 * second kernel for 16-row passes): results are deterministic. */
FP4_API int fp4_gemv_ws(float *y, const void *x_bf16, const void *packed, const void *scales, const float *gscale,
                        int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream);

/* One projection of a fused launch: TILED weights (`packed`; `scales`
 * unused) with N rows and their own tensor scale, writing y[m*ldy + n]
 * (fp32, device) for n < N. */
typedef struct {
    const void *packed;
    const void *scales;
    const float *gscale;
    int64_t N;
    float *y;
    int64_t ldy;
} fp4_proj;

#define FP4_MAX_PROJ 8

/* Several projections that read the same x [M][K] (e.g. Q, K and V, or the
 * gate and up halves of an MLP) in ONE kernel launch: results equal
 * separate fp4_gemv calls. 1 <= nproj <= FP4_MAX_PROJ; `projs` is host
 * memory read before the call returns; ldy >= N for each. Cuts the number
 * of launches per token (page "imp" README: replaying one recorded launch
 * sequence instead of re-issuing hundreds of launches per token). */
FP4_API int fp4_gemv_multi(const fp4_proj *projs, int nproj, const void *x_bf16, int64_t M, int64_t K,
                   void *stream);

/* fp4_gemv_multi with a workspace, as fp4_gemv_ws. */
FP4_API int fp4_gemv_multi_ws(const fp4_proj *projs, int nproj, const void *x_bf16, int64_t M, int64_t K,
                              void *workspace, size_t workspace_bytes, void *stream);

/* The same product for prefill-sized M on the matrix cores: packed weight
 * codes are staged in LDS, dequantised exactly to bf16 (E2M1 x E4M3 fits
 * bf16) as MFMA operands and fed to bf16 MFMA with fp32 accumulation;
 * gscale is applied once in the fp32 epilogue. Prefill is compute-bound: thousands of prompt tokens go
 * through each layer at once (page "imp" README, the prefill paragraph;
 * page "1. The big picture", "Two phases with very different costs").
 * Any M >= 1 is accepted; y [M][N] fp32 overwritten. `packed` holds the
 * tiles; `scales` is unused. The first call on a device raises the kernels'
 * dynamic LDS limit (a launch attribute, no allocation). Output tiles are
 * 256 x 128, 192 or 256. FP4_ERR_SHAPE also covers shapes whose 256-row
 * slabs reach 2 GB (256*K*2 or 256*N*4 bytes, or 32 weight row groups: the
 * kernel uses 32-bit buffer offsets), i.e. K >= 4194304 or N >= 2097152. */
FP4_API int fp4_gemm_prefill(float *y, const void *x_bf16, const void *packed, const void *scales,
                     const float *gscale, int64_t M, int64_t N, int64_t K, void *stream);

/* fp4_gemm_prefill with a workspace (see Conventions; NULL =
 * fp4_gemm_prefill). When the last round of tiles over the compute units
 * would leave most of them idle, those tiles are split into up to 4 K
 * ranges on separate workgroups (a second launch) whose fp32 partial sums
 * meet in the workspace; the last piece of a tile adds them in K order,
 * whichever finishes last. Results are deterministic, but a split tile may
 * differ from an unsplit one in the last bits. */
FP4_API int fp4_gemm_prefill_ws(float *y, const void *x_bf16, const void *packed, const void *scales,
                                const float *gscale, int64_t M, int64_t N, int64_t K, void *workspace,
                                size_t workspace_bytes, void *stream);

/* fp4_gemm_prefill over several projections that read the same x [M][K]
 * (the gate and up halves of an MLP, or Q, K and V) in one pass over the
 * compute units: each y[m*ldy + n] (n < N) is written and nothing else,
 * with the results of separate fp4_gemm_prefill calls up to the rounding of
 * split tiles. The output tiles of all projections are spread over the
 * compute units together, so the last round of tiles is fuller than it is
 * for each projection alone. 1 <= nproj <= FP4_MAX_PROJ;
 * `projs` is host memory read before the call returns; ldy >= N, and a
 * 256-row slab of each y (256*ldy*4 bytes) stays below 2 GB. Other limits
 * and the first-call attribute are those of fp4_gemm_prefill. */
FP4_API int fp4_gemm_prefill_multi(const fp4_proj *projs, int nproj, const void *x_bf16, int64_t M, int64_t K,
                                   void *stream);

/* fp4_gemm_prefill_multi with a workspace, as fp4_gemm_prefill_ws. */
FP4_API int fp4_gemm_prefill_multi_ws(const fp4_proj *projs, int nproj, const void *x_bf16, int64_t M, int64_t K,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Greedy next-token choice: idx[m] = the first n with y[m][n] not below any
 * other element of row m, for fp32 y [M][N] (device, row stride ldy >= N);
 * a NaN ranks above every number (the first NaN wins) and -0 equals +0.
 * The last vector of a decode step times the vocabulary matrix gives one
 * logit per vocabulary entry and greedy decoding picks the most likely
 * (page "1. The big picture", steps 4 and 5). idx is int32 [M] (device).
 * With a workspace (see Conventions), rows longer than 4096 elements are
 * split over several workgroups whose partial results meet there; with
 * NULL, one workgroup reads each whole row (slower on long rows). The
 * result is deterministic either way. Limits: 1 <= N <= 2^28,
 * 1 <= M <= 2^24, M * ldy <= 2^40. */
FP4_API int fp4_argmax_rows(int32_t *idx, const float *y, int64_t M, int64_t N, int64_t ldy, void *workspace,
                            size_t workspace_bytes, void *stream);

/* The greedy decode step's last product and choice: logits [M][N] (fp32,
 * device, overwritten) = fp4_gemv(x, W) for the TILED vocabulary matrix W
 * [N][K], and idx [M] (int32, device) = the greedy choice of each row of
 * the logits, as fp4_argmax_rows takes it. With a workspace, when the
 * product runs on the vector ALUs (see fp4_gemv: up to 4 rows), the choice
 * is that launch's epilogue: every workgroup leaves its largest (value,
 * index) per row in the workspace header and the workgroup with the last
 * index waits for the others' keys (bounded; idx = -1 if they never came,
 * after which the workspace must be zeroed again), picks the index and
 * clears the keys: one launch in all. Otherwise the product, then
 * fp4_argmax_rows with the same workspace (on the matrix cores that second
 * launch measured faster than the epilogue). All arguments are checked
 * before the first launch. */
FP4_API int fp4_lm_head_greedy(int32_t *idx, float *logits, const void *x_bf16, const void *packed,
                               const void *scales, const float *gscale, int64_t M, int64_t N, int64_t K,
                               void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * fp4_gemv_multi_ws with the workspace taken from a fixed device array of
 * FP4_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends. Same arguments, results and limits as fp4_gemv_multi
 * otherwise (deterministic, like fp4_gemv_multi_ws). FP4_ERR_WORKSPACE if
 * the call needs more scratch than the array holds (fp4_workspace_bytes with
 * FP4_OP_GEMV tells; e.g. 17 K chunks x 4096 output rows of partial sums).
 * All calls on one GPU share the array: calls that may overlap in time on
 * one GPU race and must not be made. The first call on a device looks up
 * the array's device address (hipGetSymbolAddress); no call allocates. */
#define FP4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
FP4_API int fp4_gemv_multi_noalloc(const fp4_proj *projs, int nproj, const void *x_bf16, int64_t M, int64_t K,
                                   void *stream);

/* The attention block's products on the RMS-normalised stream: for each
 * projection, y[m][n] = sum_k dequant(W)[n][k] * xn[m][k] with
 *   xn[m][k] = bf16( x[m][k] / sqrt(mean_k x[m][k]^2 + eps) * gain[k] ),
 * the mean over the K elements of the row, in fp32, rounded once to bf16
 * (round to nearest even). A decode layer runs attention on its residual
 * stream (page "1. The big picture", step 3); for the Qwen3 family the
 * pages use as their example, Q, K and V read that stream RMS-normalised
 * (eps 1e-6 there). gain: bf16 [K] (device, 16-byte aligned); eps finite
 * and >= 0 (else FP4_ERR_SHAPE); projections and x as fp4_gemv_multi. Up
 * to 2 rows on the vector ALUs: one launch, every workgroup computing the
 * rows' sums of squares itself. Otherwise a norm kernel writes xn into the
 * workspace (required then: fp4_workspace_bytes with FP4_OP_GEMV_RMSNORM;
 * FP4_ERR_WORKSPACE without one), and the product reads it. */
FP4_API int fp4_gemv_multi_rmsnorm(const fp4_proj *projs, int nproj, const void *x_bf16, const void *gain_bf16,
                                   float eps, int64_t M, int64_t K, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* The first half of a gated MLP: h[m][n] = bf16( silu(g[m][n]) * u[m][n] )
 * with g = x * dequant(W_gate)^T, u = x * dequant(W_up)^T (each TILED
 * [N][K] with its own tensor scale), silu(z) = z / (1 + e^-z), in fp32,
 * rounded once to bf16 (nearest even); h is bf16 [M][ldh] (device, 2-byte
 * aligned, ldh >= N) and feeds the down projection. The pages' example
 * model family (Qwen3, page "1. The big picture") has this MLP; the gate,
 * up and down names are the workload's. When the pair runs on the vector
 * ALUs (see fp4_gemv) it is one launch: each workgroup computes the same
 * rows of gate and up and writes h. Otherwise the two products go to fp32
 * buffers in the workspace (required then: FP4_OP_GEMV_SWIGLU with
 * Ns[0] = N; FP4_ERR_WORKSPACE without one) and an elementwise kernel
 * writes h. */
FP4_API int fp4_gemv_swiglu(void *h_bf16, int64_t ldh, const void *x_bf16, const void *gate_packed,
                            const float *gate_gscale, const void *up_packed, const float *up_gscale, int64_t M,
                            int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream);

/* Which call a workspace size is asked for. */
typedef enum {
    FP4_OP_GEMV = 0,           /* fp4_gemv_ws, fp4_gemv_multi_ws */
    FP4_OP_GEMM_PREFILL = 1,   /* fp4_gemm_prefill_ws, fp4_gemm_prefill_multi_ws */
    FP4_OP_ARGMAX_ROWS = 2,    /* fp4_argmax_rows (K unused, Ns[0] = N) */
    FP4_OP_LM_HEAD_GREEDY = 3, /* fp4_lm_head_greedy (Ns[0] = N) */
    FP4_OP_GEMV_RMSNORM = 4,   /* fp4_gemv_multi_rmsnorm */
    FP4_OP_GEMV_SWIGLU = 5     /* fp4_gemv_swiglu (Ns[0] = N) */
} fp4_op;

/* *bytes = the workspace bytes a call of `op` with M activation rows, K
 * input features and nproj projections of Ns[i] output features needs on
 * the current device (0: the call uses none, any workspace or NULL will
 * do). Host only; enqueues nothing. The size depends on the launch plan,
 * which reads the device's compute-unit count. Returns FP4_ERR_SHAPE for
 * arguments the call itself would reject, FP4_ERR_UNSUPPORTED for an
 * unknown op. */
FP4_API int fp4_workspace_bytes(int op, int64_t M, int64_t K, const int64_t *Ns, int nproj, size_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */

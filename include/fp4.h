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
 *     buffer. Exceptions to "the library allocates nothing": fp4_gemv
 *     and fp4_gemv_multi on the matrix-core path (M >= 5; M = 3 or 4 when
 *     the call reads at least 32 MiB of weights and K <= 8192) with
 *     K > 1024 keep the per-chunk
 *     partial sums in a per-device workspace (C * ceil(N/16) * 1 KiB, C =
 *     ceil(K/1024), summed over the projections) that the library
 *     allocates with hipMalloc on the first call that needs it (or needs
 *     more) and keeps until the process ends; that first call must not be
 *     made while the stream is being captured into a graph. Calls on one
 *     device share the workspace, so such calls on different streams of the
 *     same device must not overlap in time. fp4_gemm_prefill,
 *     fp4_gemm_prefill_multi and fp4_argmax_rows keep workspaces of their
 *     own under the same rules (described at each call).
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
 *   - Calls may be made from several host threads; the workspaces are
 *     guarded by a lock while they are (re)allocated.
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
    FP4_ERR_UNSUPPORTED = -6  /* valid request the library cannot serve */
} fp4_status;

typedef enum { FP4_LAYOUT_ROWMAJOR = 0, FP4_LAYOUT_TILED = 1 } fp4_layout;

/* Human-readable text for a status code (static storage, never NULL). */
FP4_API const char *fp4_status_string(int status);

/* Bytes of the packed and scale arrays for an N x K weight in `layout`.
 * ROWMAJOR: N*K/2 and N*K/16. TILED: G*C*4608 and 0 (the scales live in
 * the tiles, see above). Host-only; enqueues nothing. */
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
 * Any M >= 1 is accepted. `packed` holds the tiles; `scales` is unused. */
FP4_API int fp4_gemv(float *y, const void *x_bf16, const void *packed, const void *scales, const float *gscale,
             int64_t M, int64_t N, int64_t K, void *stream);

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

/* The same product for prefill-sized M on the matrix cores: packed weight
 * codes are staged in LDS, dequantised exactly to bf16 (E2M1 x E4M3 fits
 * bf16) as MFMA operands and fed to bf16 MFMA with fp32 accumulation;
 * gscale is applied once in the fp32 epilogue. Prefill is compute-bound: thousands of prompt tokens go
 * through each layer at once (page "imp" README, the prefill paragraph;
 * page "1. The big picture", "Two phases with very different costs").
 * Any M >= 1 is accepted; y [M][N] fp32 overwritten. `packed` holds the
 * tiles; `scales` is unused. The first call on a device raises the kernels'
 * dynamic LDS limit (a launch attribute, no allocation). Output tiles are
 * 256 x 128, 192 or 256; when the last round of tiles over the compute
 * units would leave most of them idle, those tiles are split into up to 4
 * K ranges on separate workgroups (a second launch) whose fp32 partial sums
 * meet in a per-device workspace (1 KiB per tile column, per row of 256,
 * per K range: at most 64 MiB, plus 128 bytes per split tile), allocated
 * with hipMalloc on the first call that needs it (or needs more) and kept
 * until the process ends, under the rules of the fp4_gemv workspace above
 * (no graph capture during that first call; no overlapping calls on
 * different streams of one device). The partial sums are added in K order
 * whichever workgroup finishes last: results are deterministic, but a
 * split tile may differ from an unsplit one in the last bits. FP4_ERR_SHAPE also
 * covers shapes whose 256-row slabs reach 2 GB (256*K*2 or 256*N*4 bytes,
 * or 32 weight row groups: the kernel uses 32-bit buffer offsets), i.e.
 * K >= 4194304 or N >= 2097152. */
FP4_API int fp4_gemm_prefill(float *y, const void *x_bf16, const void *packed, const void *scales,
                     const float *gscale, int64_t M, int64_t N, int64_t K, void *stream);

/* fp4_gemm_prefill over several projections that read the same x [M][K]
 * (the gate and up halves of an MLP, or Q, K and V) in one pass over the
 * compute units: each y[m*ldy + n] (n < N) is written and nothing else,
 * with the results of separate fp4_gemm_prefill calls up to the rounding of
 * split tiles. The output tiles of all projections are spread over the
 * compute units together, so the last round of tiles is fuller than it is
 * for each projection alone. 1 <= nproj <= FP4_MAX_PROJ;
 * `projs` is host memory read before the call returns; ldy >= N, and a
 * 256-row slab of each y (256*ldy*4 bytes) stays below 2 GB. Other limits,
 * the first-call attribute and the workspace are those of
 * fp4_gemm_prefill. */
FP4_API int fp4_gemm_prefill_multi(const fp4_proj *projs, int nproj, const void *x_bf16, int64_t M, int64_t K,
                                   void *stream);

/* Greedy next-token choice: idx[m] = the first n with y[m][n] not below any
 * other element of row m, for fp32 y [M][N] (device, row stride ldy >= N);
 * a NaN ranks above every number (the first NaN wins) and -0 equals +0.
 * The last vector of a decode step times the vocabulary matrix gives one
 * logit per vocabulary entry and greedy decoding picks the most likely
 * (page "1. The big picture", steps 4 and 5). idx is int32 [M] (device).
 * Rows longer than 4096 elements are split over several workgroups whose
 * partial results meet in a per-device workspace (8 bytes per workgroup
 * plus 128 bytes per row), allocated with hipMalloc on the first call that
 * needs it (or needs more) and kept until the process ends, under the same
 * rules as the fp4_gemv workspace above: no graph capture during that first
 * call, and calls on different streams of one device must not overlap.
 * The result is deterministic. Limits: 1 <= N <= 2^28, 1 <= M <= 2^24,
 * M * ldy <= 2^40. */
FP4_API int fp4_argmax_rows(int32_t *idx, const float *y, int64_t M, int64_t N, int64_t ldy, void *stream);

/* The greedy decode step's last product and choice: logits [M][N] (fp32,
 * device, overwritten) = fp4_gemv(x, W) for the TILED vocabulary matrix W
 * [N][K], then idx = fp4_argmax_rows(logits). Two launches on `stream`
 * (plus fp4_gemv's own); all arguments are checked before the first. */
FP4_API int fp4_lm_head_greedy(int32_t *idx, float *logits, const void *x_bf16, const void *packed,
                               const void *scales, const float *gscale, int64_t M, int64_t N, int64_t K,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */

/*
 * NVFP4 oracle: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of what the NVFP4
 * decode path computes. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the GPU library never links or calls it, and
 * this file shares no code, header or table with the GPU sources.
 *
 * What is computed and where it comes from
 * ----------------------------------------
 * The engine the source pages describe stores weights as NVFP4 "so there is
 * less data to shuffle" (page "How imp turns a model file into words", Part
 * one: loading the model) and reads them "without unpacking them to 16 bits"
 * during the bandwidth-bound decode phase (page "imp" README, the decode
 * paragraph of the request walkthrough). The engineering log's post "NVFP4 at
 * the bit level" names the parts of the format: four-bit values and two
 * scales. The bit-level definition used here:
 *   - element: FP4 E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa
 *     bit; OCP Microscaling Formats v1.0), magnitudes {0,.5,1,1.5,2,3,4,6};
 *   - block scale: FP8 E4M3 "fn" (OCP 8-bit floating point: bias 7, no
 *     infinities, 0x7F/0xFF are NaN, max 448), one per 16 consecutive
 *     K-elements of a row;
 *   - tensor scale: one FP32 value, a decode multiplier.
 * Quantisation rule (fp32, one IEEE rounding per operation):
 *   gscale = amax|W| / (448*6);  per block: s = (block_amax / 6) / gscale,
 *   scale code = E4M3(s) rounded to nearest-even, saturating at 448;
 *   element code = E2M1(w / (E4M3(code)*gscale)) rounded to nearest-even.
 * Dequantised weight: E2M1(q) * E4M3(sc) * gscale.
 * Sources: bf16 weights, or a checkpoint released in FP8 (E4M3 codes and one
 * fp32 dequantisation scale per tensor; element value E4M3(code) * scale,
 * rounded once to fp32), which the imp README's quantiser also accepts.
 * Product: y[m][n] = sum_k dequant(W)[n][k] * x[m][k], here in fp64.
 *
 * Readings where the definition above leaves a choice (each is listed with
 * its reason in the project's design notes):
 *   - element order: even k in the low nibble of each byte;
 *   - canonical layout: packed [N][K/2], scales [N][K/16], row-major,
 *     K a multiple of 16 (blocks never straddle rows);
 *   - an all-zero tensor gives gscale = 0, and any block whose scale code
 *     is 0x00 gets element codes 0;
 *   - the sign of an element code is the sign bit of w/d, so small
 *     negative values encode as 0x8 (-0).
 *
 * Pins (tests run without a GPU): E2M1 values against the minifloat
 * bit-field formula; E4M3 decode against torch.float8_e4m3fn for all 256
 * codes; E4M3 encode against torch's round-to-nearest-even cast; E2M1 encode
 * against brute-force nearest search; quantiser round-trip invariants and a
 * hand-worked example; the product against numpy float64 matmul of the
 * dequantised matrix and exact power-of-two cases; the greedy choice against
 * the built-in max and numpy's argmax (ties, NaN, infinities, signed zeros);
 * the FP8 source against the bf16 path (power-of-two scales, exact in bf16)
 * and against fp32 values rounded by numpy (other scales), with torch's E4M3
 * decode, and the sign flip under a negated scale.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- decode */

/* E2M1 magnitudes for codes 0..7; bit 3 is the sign. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* E4M3 "fn": sign s, exponent e (4 bits, bias 7), mantissa m (3 bits).
 * e == 0: subnormal (m/8) * 2^(1-7);  otherwise (1 + m/8) * 2^(e-7);
 * e == 15 && m == 7: NaN. */
double orc_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

static double E4M3_TAB[256];
static double E2M1_TAB[16];
static pthread_once_t tab_once = PTHREAD_ONCE_INIT;

static void build_tables(void) {
    for (int c = 0; c < 256; ++c) E4M3_TAB[c] = orc_e4m3_value(c);
    for (int c = 0; c < 16; ++c) E2M1_TAB[c] = orc_e2m1_value(c);
}

static void tables(void) { pthread_once(&tab_once, build_tables); }

/* ---------------------------------------------------------------- encode */

/* Nearest finite E4M3 code to s >= 0, ties to the even code (even mantissa
 * bit), saturating: anything >= 448 (the largest finite value) gives 0x7E.
 * Positive codes 0x00..0x7E are increasing in value, so the two neighbours
 * of s are found by walking the table. */
uint8_t orc_e4m3_encode(float s_in) {
    tables();
    double s = (double)s_in;
    int neg = 0;
    if (s < 0 || (s == 0 && signbit(s))) { neg = 1; s = -s; }
    int c;
    if (!(s < E4M3_TAB[0x7E])) {
        c = 0x7E;
    } else {
        int lo = 0;
        while (E4M3_TAB[lo + 1] <= s) ++lo;       /* E4M3_TAB[lo] <= s < E4M3_TAB[lo+1] */
        double dlo = s - E4M3_TAB[lo], dhi = E4M3_TAB[lo + 1] - s;
        if (dlo < dhi)
            c = lo;
        else if (dhi < dlo)
            c = lo + 1;
        else
            c = (lo % 2 == 0) ? lo : lo + 1;
    }
    return (uint8_t)(c | (neg ? 0x80 : 0));
}

/* E2M1 code of v: the nearest of the eight magnitudes, ties to the even code
 * (even mantissa bit), magnitudes above 6 saturate to 6; the sign bit of the
 * code is the sign bit of v. Walks the midpoints between neighbours. */
uint8_t orc_e2m1_encode(float v) {
    double a = fabs((double)v);
    int code = 7;
    for (int i = 0; i < 7; ++i) {
        double mid = 0.5 * (E2M1_MAG[i] + E2M1_MAG[i + 1]);
        if (a < mid) { code = i; break; }
        if (a == mid) { code = (i % 2 == 0) ? i : i + 1; break; }
    }
    return (uint8_t)(code | (signbit(v) ? 8 : 0));
}

/* -------------------------------------------------------------- quantise */

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Where the values to quantise come from: bf16 bit patterns, FP8 E4M3 codes
 * times one fp32 dequantisation scale (a checkpoint released in FP8: the
 * imp README says its quantiser builds NVFP4 weights from BF16 or FP8
 * releases), or fp32 values as they are. Every kind yields one fp32 value per
 * element; the quantisation steps below do not depend on the kind. */
typedef struct {
    int kind;                 /* 0: bf16, 1: fp8 E4M3 codes * scale, 2: fp32 */
    const uint16_t *bf16;
    const uint8_t *fp8;
    float fp8_scale;
    const float *f32;
} src_t;

static float src_value(const src_t *src, int64_t i) {
    if (src->kind == 0) return bf16_to_f32(src->bf16[i]);
    if (src->kind == 1) {
        /* E4M3 decodes exactly to fp32; the product is one rounding */
        volatile float w = (float)E4M3_TAB[src->fp8[i]] * src->fp8_scale;
        return w;
    }
    return src->f32[i];
}

/* Quantise the [N][K] row-major values of `src` into the canonical layout.
 * Returns 0, or -1 if K is not a multiple of 16 or a size is negative.
 * Every arithmetic step is one fp32 operation, rounded to nearest-even
 * (this file is compiled with -ffp-contract=off and without fast-math). */
static int quantize_src(const src_t *src, int64_t N, int64_t K, uint8_t *packed, uint8_t *scales,
                        float *gscale_out) {
    tables();
    if (N < 0 || K < 0 || K % 16 != 0) return -1;
    /* 1. tensor amax (exact) */
    float amax = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) {
        float a = fabsf(src_value(src, i));
        if (a > amax) amax = a;
    }
    /* 2. tensor scale */
    if (amax == 0.0f) {
        *gscale_out = 0.0f;
        memset(packed, 0, (size_t)(N * K / 2));
        memset(scales, 0, (size_t)(N * K / 16));
        return 0;
    }
    volatile float gscale = amax / 2688.0f;      /* 448 * 6 */
    *gscale_out = gscale;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < K / 16; ++b) {
            float wb[16];
            for (int j = 0; j < 16; ++j) wb[j] = src_value(src, n * K + b * 16 + j);
            /* 3. block amax and scale */
            float bamax = 0.0f;
            for (int j = 0; j < 16; ++j) {
                float a = fabsf(wb[j]);
                if (a > bamax) bamax = a;
            }
            volatile float t = bamax / 6.0f;
            volatile float s = t / gscale;
            uint8_t sc = orc_e4m3_encode(s);
            float s_dec = (float)E4M3_TAB[sc];
            scales[n * (K / 16) + b] = sc;
            /* 4. elements */
            uint8_t codes[16];
            for (int j = 0; j < 16; ++j) {
                if (s_dec == 0.0f) {
                    codes[j] = 0;
                } else {
                    volatile float d = s_dec * gscale;
                    volatile float v = wb[j] / d;
                    codes[j] = orc_e2m1_encode(v);
                }
            }
            /* 5. pack, even k in the low nibble */
            for (int j = 0; j < 8; ++j)
                packed[n * (K / 2) + b * 8 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* W: bf16 bits [N][K]. */
int orc_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *packed, uint8_t *scales,
                 float *gscale_out) {
    src_t src = {0, W, NULL, 0.0f, NULL};
    return quantize_src(&src, N, K, packed, scales, gscale_out);
}

/* W: FP8 E4M3 codes [N][K], element value E4M3(code) * scale (fp32). The
 * NaN codes 0x7F and 0xFF are outside the domain, like non-finite bf16. */
int orc_quantize_fp8(const uint8_t *W, float scale, int64_t N, int64_t K, uint8_t *packed, uint8_t *scales,
                     float *gscale_out) {
    src_t src = {1, NULL, W, scale, NULL};
    return quantize_src(&src, N, K, packed, scales, gscale_out);
}

/* W: fp32 values [N][K] (finite). */
int orc_quantize_f32(const float *W, int64_t N, int64_t K, uint8_t *packed, uint8_t *scales,
                     float *gscale_out) {
    src_t src = {2, NULL, NULL, 0.0f, W};
    return quantize_src(&src, N, K, packed, scales, gscale_out);
}

/* Dequantised weights, fp64 [N][K]. */
void orc_dequant(const uint8_t *packed, const uint8_t *scales, float gscale, int64_t N, int64_t K,
                 double *out) {
    tables();
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[n * (K / 2) + k / 2];
            int q = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[n * K + k] = E2M1_TAB[q] * E4M3_TAB[scales[n * (K / 16) + k / 16]] * (double)gscale;
        }
}

/* --------------------------------------------------------------- product */

typedef struct {
    const uint16_t *x;        /* bf16 activations, or NULL ... */
    const double *xd;         /* ... fp64 activations */
    const uint8_t *packed, *scales;
    double gscale;
    int64_t M, N, K, n0, n1;
    double *y, *l1;
} gemv_job;

static void *gemv_rows(void *arg) {
    const gemv_job *j = (const gemv_job *)arg;
    const int64_t K = j->K;
    for (int64_t n = j->n0; n < j->n1; ++n) {
        const uint8_t *q = j->packed + n * (K / 2);
        const uint8_t *sc = j->scales + n * (K / 16);
        for (int64_t m = 0; m < j->M; ++m) {
            const uint16_t *xm = j->x ? j->x + m * K : NULL;
            const double *xdm = j->xd ? j->xd + m * K : NULL;
            double y = 0.0, l1 = 0.0;
            for (int64_t b = 0; b < K / 16; ++b) {
                double s = E4M3_TAB[sc[b]];
                double inner = 0.0;
                for (int64_t i = 0; i < 16; ++i) {
                    int64_t k = b * 16 + i;
                    uint8_t byte = q[k / 2];
                    double e = E2M1_TAB[(k % 2 == 0) ? (byte & 15) : (byte >> 4)];
                    double xv = xm ? (double)bf16_to_f32(xm[k]) : xdm[k];
                    inner += e * xv;
                    l1 += fabs(e * s * j->gscale * xv);
                }
                y += s * inner;
            }
            j->y[m * j->N + n] = j->gscale * y;
            if (j->l1) j->l1[m * j->N + n] = l1;
        }
    }
    return 0;
}

/* y[m][n] = gscale * sum_b E4M3(sc[n][b]) * sum_i E2M1(q[n][16b+i]) * x[m][16b+i]
 * in fp64, and l1[m][n] = sum_k |dequant(W)[n][k] * x[m][k]| (the scale of
 * the error bound). x is bf16 bits [M][K]; packed/scales canonical layout.
 * Rows n are split over `nthreads` threads; each sum runs in k order. */
static void gemv_any(const uint16_t *x, const double *xd, int64_t M, const uint8_t *packed,
                     const uint8_t *scales, float gscale, int64_t N, int64_t K, double *y, double *l1,
                     int nthreads) {
    tables();
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = (int)(N > 0 ? N : 1);
    pthread_t th[256];
    gemv_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        gemv_job j = {x, xd, packed, scales, (double)gscale, M, N, K, N * t / nthreads,
                      N * (t + 1) / nthreads, y, l1};
        jobs[t] = j;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], 0, gemv_rows, &jobs[t]);
    gemv_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], 0);
}

void orc_gemv(const uint16_t *x, int64_t M, const uint8_t *packed, const uint8_t *scales,
              float gscale, int64_t N, int64_t K, double *y, double *l1, int nthreads) {
    gemv_any(x, NULL, M, packed, scales, gscale, N, K, y, l1, nthreads);
}

/* The same product for fp64 activations x [M][K] (a normalised input, kept
 * exact): y and l1 as orc_gemv. */
void orc_gemv_f64(const double *x, int64_t M, const uint8_t *packed, const uint8_t *scales,
                  float gscale, int64_t N, int64_t K, double *y, double *l1, int nthreads) {
    gemv_any(NULL, x, M, packed, scales, gscale, N, K, y, l1, nthreads);
}

/* ----------------------------------------------------- fused neighbours */

/* The steps on either side of the product in a decode layer. Each layer
 * runs attention, then the MLP, each on the residual stream (page "1. The
 * big picture", step 3), for the Qwen3 family the pages use as their
 * example. Written out from these readings (the pages give no formulas):
 *   - the MLP is gated: h = silu(gate(x)) * up(x), then down(h), with
 *     silu(z) = z * sigmoid(z) = z / (1 + e^-z);
 *   - attention's Q, K and V products read the RMS-normalised stream:
 *     x_hat[k] = x[k] / sqrt(mean over k of x[k]^2 + eps) * gain[k].
 * Both in fp64 here. */

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* h[i] = silu(g[i]) * u[i] for n elements (g: the gate product, u: up). */
void orc_swiglu(const double *g, const double *u, int64_t n, double *h) {
    for (int64_t i = 0; i < n; ++i) h[i] = orc_silu(g[i]) * u[i];
}

/* out[m][k] = x[m][k] / sqrt(mean_k x[m][k]^2 + eps) * gain[k]; x [M][K]
 * and gain [K] are bf16 bits. */
void orc_rmsnorm(const uint16_t *x, const uint16_t *gain, int64_t M, int64_t K, double eps, double *out) {
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)bf16_to_f32(x[m * K + k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            out[m * K + k] = (double)bf16_to_f32(x[m * K + k]) * r * (double)bf16_to_f32(gain[k]);
    }
}

/* ---------------------------------------------------------------- MXFP4 */

/* The README's quantisation row lists MXFP4 beside NVFP4. Read here as the
 * OCP Microscaling v1.0 format of that name: the same E2M1 elements, one
 * shared scale per 32 consecutive K-elements of a row, encoded E8M0 (an
 * unsigned biased exponent, value 2^(c - 127), 0xFF NaN), no tensor scale.
 * Quantisation, the OCP conversion: per block, shared exponent
 * floor(log2(amax)) - 2 (2 = the exponent of E2M1's largest value, 6 =
 * 1.5 * 2^2), clamped to [-127, 127]; each element w / 2^shared rounded to
 * the nearest E2M1 value, ties to even, saturating at 6. Readings as for
 * NVFP4: a block with amax 0 gets scale code 0 and element codes 0; the sign
 * of an element code is the sign bit of w. Canonical layout: packed
 * [N][K/2] (even k in the low nibble), scales [N][K/32]; K % 32 == 0. */

double orc_e8m0_value(int code) {
    if ((code & 0xFF) == 0xFF) return NAN;
    return ldexp(1.0, (code & 0xFF) - 127);
}

/* W: bf16 bits [N][K]. Returns 0, or -1 for a bad shape. */
int orc_mx_quantize(const uint16_t *W, int64_t N, int64_t K, uint8_t *packed, uint8_t *scales) {
    if (N < 0 || K < 0 || K % 32 != 0) return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < K / 32; ++b) {
            double w[32], amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                w[j] = (double)bf16_to_f32(W[n * K + b * 32 + j]);
                if (fabs(w[j]) > amax) amax = fabs(w[j]);
            }
            uint8_t codes[32];
            if (amax == 0.0) {
                scales[n * (K / 32) + b] = 0;
                memset(codes, 0, sizeof codes);
            } else {
                int e;
                frexp(amax, &e);                     /* amax = f * 2^e, f in [0.5, 1): floor(log2) = e - 1 */
                int shared = (e - 1) - 2;
                if (shared < -127) shared = -127;
                if (shared > 127) shared = 127;
                scales[n * (K / 32) + b] = (uint8_t)(shared + 127);
                for (int j = 0; j < 32; ++j) {
                    double v = ldexp(w[j], -shared);  /* exact: a power-of-two scaling of a bf16 value */
                    codes[j] = orc_e2m1_encode((float)v);
                }
            }
            for (int j = 0; j < 16; ++j)
                packed[n * (K / 2) + b * 16 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* Dequantised MXFP4 weights, fp64 [N][K]. */
void orc_mx_dequant(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K, double *out) {
    tables();
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[n * (K / 2) + k / 2];
            int q = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[n * K + k] = E2M1_TAB[q] * orc_e8m0_value(scales[n * (K / 32) + k / 32]);
        }
}

/* y[m][n] = sum_b E8M0(sc[n][b]) * sum_{i<32} E2M1(q[n][32b+i]) * x[m][32b+i]
 * and l1[m][n] = sum_k |dequant(W)[n][k] * x[m][k]|, fp64, in k order. */
void orc_mx_gemv(const uint16_t *x, int64_t M, const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K,
                 double *y, double *l1) {
    tables();
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *q = packed + n * (K / 2);
        const uint8_t *sc = scales + n * (K / 32);
        for (int64_t m = 0; m < M; ++m) {
            const uint16_t *xm = x + m * K;
            double acc = 0.0, a1 = 0.0;
            for (int64_t b = 0; b < K / 32; ++b) {
                double s = orc_e8m0_value(sc[b]), inner = 0.0;
                for (int64_t i = 0; i < 32; ++i) {
                    int64_t k = b * 32 + i;
                    uint8_t byte = q[k / 2];
                    double e = E2M1_TAB[(k % 2 == 0) ? (byte & 15) : (byte >> 4)];
                    double xv = (double)bf16_to_f32(xm[k]);
                    inner += e * xv;
                    a1 += fabs(e * s * xv);
                }
                acc += s * inner;
            }
            y[m * N + n] = acc;
            if (l1) l1[m * N + n] = a1;
        }
    }
}

/* The GPU library's MXFP4 tiled layout: rows in groups of 8, K in chunks of
 * 1024; tile (g, c) is the 4352 bytes at (g*C + c)*4352:
 *   codes, bytes 0..4095: as the NVFP4 tile (row r's 32 pieces of 16 bytes
 *       at r*512 + l*16; piece l = elements 1024c + 32l .. + 31);
 *   scales, bytes 4096..4351: byte 4096 + h*128 + l*4 + i = scale of
 *       (row 8g + 2i + h, block 32c + l), h < 2, l < 32, i < 4.
 * Positions outside the tensor hold 0. */
void orc_mx_tile(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K, uint8_t *tiles) {
    int64_t G = (N + 7) / 8, C = (K + 1023) / 1024;
    for (int64_t g = 0; g < G; ++g)
        for (int64_t c = 0; c < C; ++c) {
            uint8_t *t = tiles + (g * C + c) * 4352;
            for (int r = 0; r < 8; ++r)
                for (int l = 0; l < 32; ++l) {
                    int64_t row = 8 * g + r;
                    for (int i = 0; i < 16; ++i) {
                        int64_t kb = (1024 * c + 32 * l) / 2 + i;
                        t[r * 512 + l * 16 + i] = (row < N && kb < K / 2) ? packed[row * (K / 2) + kb] : 0;
                    }
                }
            for (int h = 0; h < 2; ++h)
                for (int l = 0; l < 32; ++l)
                    for (int i = 0; i < 4; ++i) {
                        int64_t row = 8 * g + 2 * i + h, blk = 32 * c + l;
                        t[4096 + h * 128 + l * 4 + i] = (row < N && blk < K / 32) ? scales[row * (K / 32) + blk] : 0;
                    }
        }
}

/* --------------------------------------------------------- device layout */

/* The GPU library's tiled layout, written out as plain loops so that the
 * GPU re-tiling can be compared byte for byte. Rows form groups of 8
 * (G = ceil(N/8)); K forms chunks of 1024 (C = ceil(K/1024)); tile (g, c) is
 * the 4608 bytes at (g*C + c)*4608 of one buffer:
 *   codes, bytes 0..4095:  byte r*512 + l*16 + i          =  canonical packed byte
 *       (row 8g+r, byte (1024c + 32l)/2 + i)              r<8, l<32, i<16
 *   scales, bytes 4096..:  byte 4096 + h*256 + l*8 + 2i + j  =  canonical scale
 *       (row 8g + 2i + h, block 64c + 2l + j)             h<2, i<4, j<2
 * Positions outside the tensor (row >= N or k >= K) hold 0. */
void orc_tile(const uint8_t *packed, const uint8_t *scales, int64_t N, int64_t K, uint8_t *tiles) {
    int64_t G = (N + 7) / 8, C = (K + 1023) / 1024;
    for (int64_t g = 0; g < G; ++g)
        for (int64_t c = 0; c < C; ++c) {
            uint8_t *t = tiles + (g * C + c) * 4608;
            for (int r = 0; r < 8; ++r)
                for (int l = 0; l < 32; ++l) {
                    int64_t row = 8 * g + r;
                    for (int i = 0; i < 16; ++i) {
                        int64_t kb = (1024 * c + 32 * l) / 2 + i;      /* byte index in the row */
                        t[r * 512 + l * 16 + i] = (row < N && kb < K / 2) ? packed[row * (K / 2) + kb] : 0;
                    }
                }
            for (int h = 0; h < 2; ++h)
                for (int l = 0; l < 32; ++l)
                    for (int i = 0; i < 4; ++i)
                        for (int j = 0; j < 2; ++j) {
                            int64_t row = 8 * g + 2 * i + h, blk = 64 * c + 2 * l + j;
                            t[4096 + h * 256 + l * 8 + 2 * i + j] =
                                (row < N && blk < K / 16) ? scales[row * (K / 16) + blk] : 0;
                        }
        }
}

/* Element-wise versions of the two encoders, for sweeping many inputs. */
void orc_e4m3_encode_n(const float *s, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(s[i]);
}

void orc_e2m1_encode_n(const float *v, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(v[i]);
}

/* --------------------------------------------------------- greedy choice */

/* Greedy decoding takes, for the last position, the vocabulary entry with
 * the largest logit (page "1. The big picture", steps 4 and 5: the final
 * vector times the vocabulary matrix gives one score per entry; greedy
 * decoding always picks the most likely). Per row: the first index whose
 * value is not below any other; a NaN ranks above every number (the first
 * NaN wins) and -0 equals +0. */
static int ranks_above_f64(double a, double b) {
    if (isnan(b)) return 0;
    if (isnan(a)) return 1;
    return a > b;
}

static int ranks_above_f32(float a, float b) {
    if (isnan(b)) return 0;
    if (isnan(a)) return 1;
    return a > b;
}

void orc_argmax_rows_f64(const double *y, int64_t M, int64_t N, int64_t ldy, int32_t *idx) {
    for (int64_t m = 0; m < M; ++m) {
        const double *row = y + m * ldy;
        int64_t best = 0;
        for (int64_t n = 1; n < N; ++n)
            if (ranks_above_f64(row[n], row[best])) best = n;
        idx[m] = (int32_t)best;
    }
}

void orc_argmax_rows_f32(const float *y, int64_t M, int64_t N, int64_t ldy, int32_t *idx) {
    for (int64_t m = 0; m < M; ++m) {
        const float *row = y + m * ldy;
        int64_t best = 0;
        for (int64_t n = 1; n < N; ++n)
            if (ranks_above_f32(row[n], row[best])) best = n;
        idx[m] = (int32_t)best;
    }
}

/* Seeded bf16 input generator (C implementation of workloads/gen.py).
 *
 * Input generation only: no NVFP4 arithmetic lives here.
 * Element i of stream `seed` (counter form of SplitMix64, Steele/Lea/Flood,
 * OOPSLA 2014): u0 = U(2i), u1 = U(2i+1), z = sqrt(-2 ln(1-u0)) cos(2 pi u1)
 * (Box-Muller), v = sigma*z, optionally v *= outlier_scale when
 * U'(i) < outlier_p on the stream seed ^ OUTLIER_SALT, then
 * float64 -> float32 (RN) -> bfloat16 (RNE). Threads split the index range.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define OUTLIER_SALT 0x5DEECE66DULL

static inline uint64_t sm64(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1u) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline double u01(uint64_t seed, uint64_t i) {
    return (double)(sm64(seed, i) >> 11) * (1.0 / 9007199254740992.0);
}

static inline uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef struct {
    uint16_t *out;
    int64_t lo, hi, start;
    uint64_t seed;
    double sigma, p, scale;
} job_t;

static void *run(void *arg) {
    const job_t *j = (const job_t *)arg;
    const double two_pi = 2.0 * 3.141592653589793;
    for (int64_t i = j->lo; i < j->hi; ++i) {
        uint64_t idx = (uint64_t)(j->start + i);
        double u0 = u01(j->seed, 2u * idx), u1 = u01(j->seed, 2u * idx + 1u);
        double v = sqrt(-2.0 * log1p(-u0)) * cos(two_pi * u1) * j->sigma;
        if (j->p > 0.0 && u01(j->seed ^ OUTLIER_SALT, idx) < j->p) v *= j->scale;
        j->out[i] = to_bf16((float)v);
    }
    return 0;
}

/* Fill out[0..n) with elements start..start+n-1 of stream `seed`. */
void wl_gen_bf16(uint16_t *out, int64_t n, uint64_t seed, int64_t start, double sigma,
                 double outlier_p, double outlier_scale, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n < 65536) nthreads = 1;
    pthread_t th[64];
    job_t jobs[64];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].out = out;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
        jobs[t].start = start;
        jobs[t].seed = seed;
        jobs[t].sigma = sigma;
        jobs[t].p = outlier_p;
        jobs[t].scale = outlier_scale;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], 0, run, &jobs[t]);
    run(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], 0);
}

/* Raw SplitMix64 outputs, for cross-checking against the numpy version. */
void wl_splitmix64(uint64_t *out, int64_t n, uint64_t seed, int64_t start) {
    for (int64_t i = 0; i < n; ++i) out[i] = sm64(seed, (uint64_t)(start + i));
}

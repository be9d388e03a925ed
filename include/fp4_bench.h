/*
 * fp4_bench.h: measurement aid exported by libfp4.so next to the product
 * calls of fp4.h. It is not part of the decode path; the benchmark uses it
 * to measure the streaming-read ceiling that the decode kernels are compared
 * with (page "1. The big picture", section "The most important number in
 * this book": decode speed is at most bandwidth over bytes per token, and
 * real engines reach 60-90 % of that ceiling).
 */
#ifndef FP4_BENCH_H
#define FP4_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of device memory at `buf` once, with 16-byte loads, one
 * kilobyte per wave and load instruction, `unroll` (1, 2, 4 or 8) load
 * instructions in flight per wave; `workgroups` workgroups of `waves`
 * (1..16) waves. mode 0: the kilobyte blocks go round-robin over all waves;
 * mode 1: each wave reads one contiguous range. nontemporal != 0 marks the
 * loads as streaming (read once). `sink` (device, one uint32 per wave of
 * the grid) is written only in the practically impossible case that the
 * folded words equal a fixed constant; it keeps the loads live.
 * buf: 16-byte aligned; bytes: a nonzero multiple of 1024 below 2^31.
 * Enqueues one kernel on `stream` (a hipStream_t; NULL = default stream).
 * Returns 0, -1 (NULL pointer), -2 (argument out of range), -3 (alignment)
 * or -5 (the launch failed). */
int fp4_bench_stream_read(const void *buf, size_t bytes, int workgroups, int waves, int unroll, int mode,
                          int nontemporal, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4_BENCH_H */

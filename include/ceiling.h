/*
 * libtmm_ceiling.so: two measurement kernels that bound what any single launch of the
 * bandwidth-bound paths can reach on the device it runs on.  Not part of the GEMM's path;
 * bench.py runs them beside the decode GEMV so that its rate can be read against the measured
 * ceiling as well as against the published HBM bandwidth.
 *
 * The page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "Roofline", bounds a
 * memory-bound kernel by bytes moved over bandwidth; these kernels measure the two terms a
 * real launch adds to that: the fixed cost of a launch, and the rate at which one launch can
 * stream a given number of bytes it has not read before.
 *
 * Pointers are device pointers owned by the caller; nothing is allocated.  Calls are
 * asynchronous on `stream` (a hipStream_t; NULL: the default stream).  Return value: 0 on
 * success, 1 for an invalid argument (nothing is launched), 5 if the launch failed.
 */
#ifndef TMM_CEILING_H
#define TMM_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at `src` once with 16-byte non-temporal loads (the load the decode GEMV
 * streams its weights with), `grid` workgroups of `block` threads, each thread keeping 4
 * loads in flight.  The loaded values are folded into one word per wave, written to
 * sink[wave] only if it equals a value the data cannot produce in practice, so the stores
 * add no traffic; `sink` must hold grid * block / 64 floats.  bytes: a positive multiple of
 * 16 below 2^31; src: 16-byte aligned; grid >= 1; block a multiple of 64 in [64, 1024].
 */
int ceiling_stream_read(const void* src, int64_t bytes, float* sink, int grid, int block, void* stream);

/* Launch an empty kernel of `grid` workgroups of `block` threads (the launch floor). */
int ceiling_launch_floor(int grid, int block, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TMM_CEILING_H */

/*
 * rs_bench.h — measurement and self-check helpers beside the layout library
 * (librs_bench.so). Neither is a step of the layout transform.
 *
 * rs_bench_copy: a plain streaming copy of known traffic on gfx950, built the
 * way the transform kernels stream (16-byte vectors, nontemporal loads,
 * stores with nt and sc1 set, small short-lived workgroups). The benchmark
 * times it as the practical HBM
 * ceiling next to the 8 TB/s peak, and its counter readings calibrate the HBM
 * byte counters (it reads and writes exactly `bytes`).
 *
 * rs_bench_sqrt_check: checks, value by value, a device building block of the
 * library against the correctly rounded operation it stands for.
 *
 * rs_bench_store_check: drives the library's cache-policy store through each
 * of its paths, for a test to compare the buffer with the expected contents.
 */
#ifndef RS_BENCH_H
#define RS_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0, bytes) = src[0, bytes). dst and src: device, 16-byte aligned,
 * not overlapping; bytes: a multiple of 16, >= 0. Asynchronous on `stream`
 * (a hipStream_t passed as void*). Returns 0, -1 (bad argument: nothing is
 * launched) or -6 (launch error). */
int rs_bench_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* Self-check of the short correctly rounded square root that the 8-bit Adam
 * step uses for inputs in [2^-96, FLT_MAX]: every fp32 whose bit pattern lies
 * in [lo, hi] is compared, bit for bit, with the general correctly rounded
 * square root. Synchronous on the current device (allocates 16 bytes of
 * device memory for the counts). *mismatches receives the number of values
 * that differ and *first_mismatch the lowest such bit pattern (0xFFFFFFFF if
 * none). Returns 0, -1 (lo > hi or a null pointer: nothing is launched) or -6
 * (HIP error). */
int rs_bench_sqrt_check(uint32_t lo, uint32_t hi, uint64_t* mismatches, uint32_t* first_mismatch);

/* Self-check of the store the layout kernels use for nt-sc1 writes: a buffer
 * store addressed from the first active lane of the wave, or, when some lane's
 * address lies below that one or 2 GiB or more above it, a plain global store.
 * dst: device, 16-byte aligned, nvec 16-byte vectors (nvec a positive multiple
 * of 128, at most 2^30). Wave w (lanes l = 0..63, v = 64 w + l) writes the
 * vector {t, 0, v, 0xA5000000 | mode} (four uint32) at vector t of dst:
 *   mode 0: t = v (one buffer base per wave);
 *   mode 1: t = 64 w + 63 - l (lane 0 holds the highest address: global path);
 *   mode 2: t = 32 w + l for l < 32 and nvec/2 + 32 w + l - 32 otherwise (the
 *           two halves of the buffer: global path once a half is 2 GiB);
 *   mode 3: t = v for l % 3 != 0; the other lanes write nothing.
 * Asynchronous on `stream` (a hipStream_t passed as void*). Returns 0, -1 (bad
 * argument: nothing is launched) or -6 (launch error). */
int rs_bench_store_check(void* dst, int64_t nvec, int mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RS_BENCH_H */

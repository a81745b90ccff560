/*
 * rs_bench.h — measurement helper beside the layout library (librs_bench.so).
 *
 * Not a step of the layout transform: a plain streaming copy of known traffic
 * on gfx950, built the way the transform kernels stream (16-byte nontemporal
 * vectors, small short-lived workgroups). The benchmark times it as the
 * practical HBM ceiling next to the 8 TB/s peak, and its counter readings
 * calibrate the HBM byte counters (it reads and writes exactly `bytes`).
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

#ifdef __cplusplus
}
#endif

#endif /* RS_BENCH_H */

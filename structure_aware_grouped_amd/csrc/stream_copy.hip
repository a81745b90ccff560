// rs_bench_copy: a 16-byte streaming copy for gfx950, the practical HBM
// ceiling next to which the layout kernels are measured. Each 64-thread
// workgroup moves 1 KiB (one nontemporal 16-byte load and store per lane)
// and exits, which keeps many independent streams in flight across the HBM
// channels, as the unpack and pack kernels do. Launches use at most 2^24
// workgroups; beyond that each workgroup loops.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "rs_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 64;
constexpr int64_t kMaxGrid = int64_t(1) << 24;

__global__ __launch_bounds__(kThreads) void copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                           int64_t nvec) {
  for (int64_t b = blockIdx.x; b * kThreads < nvec; b += gridDim.x) {
    const int64_t i = b * kThreads + threadIdx.x;
    if (i < nvec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  }
}

}  // namespace

extern "C" int rs_bench_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return -1;
  if (bytes == 0) return 0;
  if (!dst || !src || (reinterpret_cast<uintptr_t>(dst) & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u)) return -1;
  const char* d = static_cast<const char*>(dst);
  const char* s = static_cast<const char*>(src);
  if (d < s + bytes && s < d + bytes) return -1;
  const int64_t nvec = bytes / 16;
  const int64_t groups = std::min<int64_t>((nvec + kThreads - 1) / kThreads, kMaxGrid);
  hipLaunchKernelGGL(copy16_kernel, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// rs_bench_copy: a 16-byte streaming copy for gfx950, the practical HBM
// ceiling next to which the layout kernels are measured. Each 64-thread
// workgroup moves 1 KiB (one 16-byte load and store per lane) and exits,
// which keeps many independent streams in flight across the HBM channels, as
// the unpack and pack kernels do. Loads are nontemporal; stores are buffer
// stores with nt and sc1 set (cache-policy immediate 18), the fastest store
// measured for a cold streamed copy on gfx950: 6.70 TB/s against 6.62 with
// nontemporal global stores. Launches use at most 2^24 workgroups; beyond
// that each workgroup loops.
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
    // the workgroup's 1 KiB of dst is the buffer (a raw descriptor: word 3
    // 0x00020000, 32-bit data format); lane t writes 16 bytes at 16t
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(dst + b * kThreads, 0, -1, 0x00020000);
    if (i < nvec)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_nontemporal_load(src + i), r,
                                             static_cast<int>(threadIdx.x) * 16, 0, 18);
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

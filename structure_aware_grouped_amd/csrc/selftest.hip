// rs_bench_sqrt_check: the short correctly rounded square root of the
// device helpers (sqrt_rn_short, used by the 8-bit Adam step where its input
// lies in [kSqrtShortMin, FLT_MAX]) against the general correctly rounded
// sequence, on every fp32 bit pattern of a range. A self-check beside the
// layout library, not a step of the layout transform.
#include "device_common.h"

#include "rs_bench.h"

namespace {

__global__ __launch_bounds__(256) void sqrt_check_kernel(uint32_t lo, uint32_t hi, unsigned long long* bad,
                                                         uint32_t* first) {
  const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  unsigned long long count = 0;
  uint32_t first_bad = 0xFFFFFFFFu;
  for (uint64_t u = lo + tid; u <= hi; u += stride) {
    const float x = __uint_as_float(static_cast<uint32_t>(u));
    if (__float_as_uint(rs::sqrt_rn_short(x)) != __float_as_uint(__builtin_sqrtf(x))) {
      ++count;
      first_bad = min(first_bad, static_cast<uint32_t>(u));
    }
  }
  if (count) {
    atomicAdd(bad, count);
    atomicMin(first, first_bad);
  }
}

}  // namespace

extern "C" int rs_bench_sqrt_check(uint32_t lo, uint32_t hi, uint64_t* mismatches, uint32_t* first_mismatch) {
  if (lo > hi || !mismatches || !first_mismatch) return -1;
  unsigned long long* d_bad = nullptr;
  uint32_t* d_first = nullptr;
  int rc = 0;
  if (hipMalloc(reinterpret_cast<void**>(&d_bad), sizeof(unsigned long long)) != hipSuccess ||
      hipMalloc(reinterpret_cast<void**>(&d_first), sizeof(uint32_t)) != hipSuccess) {
    rc = -6;
  } else {
    const unsigned long long zero = 0;
    const uint32_t none = 0xFFFFFFFFu;
    unsigned long long bad = 0;
    uint32_t first = none;
    if (hipMemcpy(d_bad, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d_first, &none, sizeof none, hipMemcpyHostToDevice) != hipSuccess) {
      rc = -6;
    } else {
      hipLaunchKernelGGL(sqrt_check_kernel, dim3(256 * 64), dim3(256), 0, nullptr, lo, hi, d_bad, d_first);
      if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
          hipMemcpy(&bad, d_bad, sizeof bad, hipMemcpyDeviceToHost) != hipSuccess ||
          hipMemcpy(&first, d_first, sizeof first, hipMemcpyDeviceToHost) != hipSuccess)
        rc = -6;
    }
    *mismatches = bad;
    *first_mismatch = first;
  }
  if (d_bad) (void)hipFree(d_bad);
  if (d_first) (void)hipFree(d_first);
  return rc;
}

// Self-checks of device building blocks of the layout library, beside it and
// not steps of the layout transform.
//
// rs_bench_sqrt_check: the short correctly rounded square root of the device
// helpers (sqrt_rn_short, used by the 8-bit Adam step where its input lies in
// [kSqrtShortMin, FLT_MAX]) against the general correctly rounded sequence,
// on every fp32 bit pattern of a range.
//
// rs_bench_store_check: the cache-policy store sts (nt and sc1 set) with lane
// to address maps that take each of its paths: the buffer store from the
// first active lane's address, and the global store when a lane lies below
// that address or 2 GiB or more above it.
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

// Wave w (64 threads) stores for each lane l the vector {t, 0, v, 0xA5000000 | mode}
// at vector t of dst, v = 64 w + l:
//   mode 0: t = v;  mode 1: t = 64 w + 63 - l (the first active lane has the
//   highest address);  mode 2: lanes 0-31 at 32 w + l, lanes 32-63 at
//   nvec / 2 + 32 w + l - 32 (two halves of the buffer);  mode 3: t = v, lanes
//   with l % 3 == 0 store nothing (lane 0 inactive).
__global__ __launch_bounds__(64) void store_check_kernel(rs::u32x4* dst, uint32_t nvec, int mode) {
  const uint32_t w = blockIdx.x, l = threadIdx.x, v = 64u * w + l;
  uint32_t t = v;
  if (mode == 1) t = 64u * w + 63u - l;
  if (mode == 2) t = l < 32u ? 32u * w + l : nvec / 2u + 32u * w + (l - 32u);
  if (mode == 3 && l % 3u == 0u) return;
  rs::sts<rs::kStoreNtSc1>(dst + t, rs::u32x4{t, 0u, v, 0xA5000000u | static_cast<uint32_t>(mode)});
}

}  // namespace

extern "C" int rs_bench_store_check(void* dst, int64_t nvec, int mode, void* stream) {
  if (!dst || (reinterpret_cast<uintptr_t>(dst) & 15u) || mode < 0 || mode > 3 || nvec <= 0 || nvec % 128 != 0 ||
      nvec > (int64_t(1) << 30))
    return -1;
  hipLaunchKernelGGL(store_check_kernel, dim3(static_cast<unsigned>(nvec / 64)), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<rs::u32x4*>(dst), static_cast<uint32_t>(nvec),
                     mode);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

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

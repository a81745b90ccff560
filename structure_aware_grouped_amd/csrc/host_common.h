// Host-side helpers shared by the entry points of the RaggedShard / DBuffer
// layout library: argument checks, launch error reporting, grid sizes and the
// per-plan pointer-table upload.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "device_common.h"
#include "rs_internal.h"

namespace rs {

// Grid of a launch: one workgroup per work item up to the plan's max_grid
// (kMaxGrid unless RS_MAX_GRID lowers it), beyond which every workgroup loops
// over items p, p + grid, ... (max_grid is a multiple of 8, so item p still
// runs on XCD p % 8).
inline dim3 grid_of(const rs_plan* p, int64_t n_items) {
  return dim3(static_cast<unsigned>(std::min<int64_t>(n_items, p->max_grid)));
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int check_call(const rs_plan* p, const char* who) {
  if (!p) return fail(RS_EINVAL, std::string(who) + ": null plan");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(RS_EHIP, std::string(who) + ": hipGetDevice failed");
  if (cur != p->device)
    return fail(RS_EINVAL, std::string(who) + ": current device " + std::to_string(cur) +
                               " differs from the plan's device " + std::to_string(p->device));
  return RS_OK;
}

inline int launched(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RS_EHIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
  return RS_OK;
}

// Upload a per-tensor pointer table on `stream` if it differs from the last one.
// Kernels read the table in device memory when they run, so a graph captured
// from these calls uses the table as it is at replay. A new table is therefore
// refused while `stream` is being captured: the caller makes one call with the
// same pointers before the capture, and the capture then holds kernels only.
inline int sync_table(rs_plan* p, PtrTable* tab, const void* const* ptrs, hipStream_t stream, const char* who) {
  const size_t bytes = sizeof(void*) * static_cast<size_t>(p->n);
  if (tab->valid && std::memcmp(tab->seen.data(), ptrs, bytes) == 0) return RS_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess)
    return fail(RS_EHIP, std::string(who) + ": hipStreamIsCapturing failed");
  if (cap != hipStreamCaptureStatusNone)
    return fail(RS_EINVAL, std::string(who) + ": tensor pointers differ from the plan's last call while the "
                               "stream is being captured; make one call with these pointers before the capture");
  if (tab->pending && hipEventSynchronize(tab->done) != hipSuccess)
    return fail(RS_EHIP, std::string(who) + ": waiting for the previous table upload failed");
  std::memcpy(tab->stage, ptrs, bytes);
  if (hipMemcpyAsync(tab->dev, tab->stage, bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(tab->done, stream) != hipSuccess) {
    tab->valid = false;
    return fail(RS_EHIP, std::string(who) + ": pointer table upload failed");
  }
  tab->pending = true;
  std::memcpy(tab->seen.data(), ptrs, bytes);
  tab->valid = true;
  return RS_OK;
}

inline int elem_bytes(int32_t dt) {
  switch (dt) {
    case RS_F32: return 4;
    case RS_BF16: return 2;
    case RS_E4M3: case RS_I8: case RS_U8: return 1;
    default: return 0;
  }
}

namespace {

// Code format of an rs_dtype (the device side's Fmt, which is local to each file).
[[maybe_unused]] int fmt_of(int32_t q_dt) {
  switch (q_dt) {
    case RS_E4M3: return FMT_E4M3;
    case RS_I8: return FMT_I8;
    case RS_U8: return FMT_U8;
    default: return -1;
  }
}

}  // namespace
}  // namespace rs

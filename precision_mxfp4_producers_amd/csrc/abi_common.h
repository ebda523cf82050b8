// Host-side argument checks and launch-error capture shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp4.h"

namespace mx {

extern thread_local int g_last_hip_error;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool mult32(int64_t v) { return v > 0 && (v % 32) == 0; }
inline bool mult32z(int64_t v) { return v >= 0 && (v % 32) == 0; }   // zero allowed (empty)

inline fp4_status launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FP4_EHIP;
  }
  return FP4_OK;
}

inline hipStream_t as_stream(hipStream_t s) { return s; }

}  // namespace mx

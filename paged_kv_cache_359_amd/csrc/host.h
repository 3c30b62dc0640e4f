// Host-side helpers of the C entry points: argument checks and launch status.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "pkv.h"

namespace pkv {

// Text of the last HIP error a call of this thread reported (see pkv_last_error).
extern thread_local char g_last_error[256];

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int dtype_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

inline bool valid_dtype(pkv_dtype dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }

// Clears an error left by earlier, unrelated runtime calls so that a launch is judged only
// by its own outcome.
inline void clear_stale_error() { (void)hipGetLastError(); }

inline pkv_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return PKV_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
  return PKV_ERR_HIP;
}

}  // namespace pkv

// zf_hip_status.h -- HIP status checks of the library's .hip files: a
// failing call's error code is remembered per thread (zf_hip_error_name).
#pragma once
#include <hip/hip_runtime.h>

#include "zf_internal.h"

namespace zf {
inline bool hip_ok(hipError_t e) {
  if (e != hipSuccess) last_hip_error = static_cast<int>(e);
  return e == hipSuccess;
}
}  // namespace zf

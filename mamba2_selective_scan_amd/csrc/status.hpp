// status.hpp -- the per-thread record of the last HIP error, shared by the
// library's translation units (ssm_scan_last_hip_error reads it).
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

extern thread_local hipError_t t_last_hip_error;

// Records `err` for ssm_scan_last_hip_error and returns `code`.
int hip_fail(hipError_t err, int code);

}  // namespace ssm

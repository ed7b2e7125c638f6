// hip_error.hpp - HIP runtime errors as C ABI status codes.
#pragma once
#include <hip/hip_runtime.h>

#include "error.hpp"

namespace moe {
// MOE_OK for hipSuccess, else MOE_EHIP with the runtime's text
int hip_status(hipError_t err, const char* what);
}  // namespace moe

#include <rocprofiler-sdk-roctx/roctx.h>

namespace moe {
// A roctx range around one C-ABI call that enqueues GPU work, named after
// the call: rocprofv3 --marker-trace shows where each call's kernels and
// copies come from (a no-op when no profiler is attached).
struct ApiRange {
  explicit ApiRange(const char* name) { roctxRangePushA(name); }
  ~ApiRange() { roctxRangePop(); }
  ApiRange(const ApiRange&) = delete;
  ApiRange& operator=(const ApiRange&) = delete;
};
}  // namespace moe

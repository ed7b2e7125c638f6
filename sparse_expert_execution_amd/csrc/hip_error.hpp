// hip_error.hpp - HIP runtime errors as C ABI status codes.
#pragma once
#include <hip/hip_runtime.h>

#include "error.hpp"

namespace moe {
// MOE_OK for hipSuccess, else MOE_EHIP with the runtime's text
int hip_status(hipError_t err, const char* what);
}  // namespace moe

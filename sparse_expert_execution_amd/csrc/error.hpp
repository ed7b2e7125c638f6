// error.hpp - thread-local error text shared by the C ABI translation units.
#pragma once
#include <hip/hip_runtime.h>

#include <string>

namespace moe {
extern thread_local std::string g_last_error;
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_status(hipError_t err, const char* what);
}  // namespace moe

// error.hpp - thread-local error text shared by the C ABI translation units
// (HIP-free: the host-only sources build without the HIP runtime).
#pragma once
#include <string>

#include "../../include/moe.h"

namespace moe {
extern thread_local std::string g_last_error;
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// descriptor checks and the expert block layout (host.cpp)
int check_desc(const moe_desc* d);
void layout(const moe_desc* d, size_t off[6], size_t* bytes);
}  // namespace moe

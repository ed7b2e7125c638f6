// host.cpp - HIP-free parts of the C ABI: error text, version, the q* split.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/moe.h"
#include "planner.hpp"

namespace moe {

thread_local std::string g_last_error;

int set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return moe::g_last_error.c_str(); }

int32_t moe_abi_version(void) { return 1; }

// q* (see include/moe.h): the fill count that balances PCIe fill time
// q / b_pcie against host-side time (m - q) / b_host; expert size cancels.
int32_t moe_qstar(int32_t m, double b_pcie, double b_host) {
  if (m < 0 || !(b_pcie > 0) || !(b_host > 0)) {
    moe::set_error(MOE_EINVAL, "qstar needs m >= 0 and positive rates");
    return -1;
  }
  int32_t best = 0;
  double best_t = 0;
  for (int32_t q = 0; q <= m; ++q) {
    const double tp = q / b_pcie, th = (m - q) / b_host;
    const double t = tp > th ? tp : th;
    if (q == 0 || t <= best_t) {
      best = q;
      best_t = t;
    }
  }
  return best;
}

}  // extern "C"

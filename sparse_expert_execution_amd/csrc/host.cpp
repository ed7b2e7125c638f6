// host.cpp - HIP-free parts of the C ABI: error text, version, descriptor
// checks, the expert block layout, the q* split.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/moe.h"
#include "error.hpp"
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

namespace moe {

namespace {
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

int check_desc(const moe_desc* d) {
  if (!d) return set_error(MOE_EINVAL, "desc is null");
  if (d->hidden <= 0 || d->inter <= 0 || d->hidden % 32 || d->inter % 32)
    return set_error(MOE_EINVAL, "hidden (%d) and inter (%d) must be positive multiples of 32",
                     d->hidden, d->inter);
  if (d->n_experts < 1 || d->n_experts > 1024)
    return set_error(MOE_EINVAL, "n_experts %d outside [1, 1024]", d->n_experts);
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 64)
    return set_error(MOE_EINVAL, "top_k %d outside [1, min(E, 64)]", d->top_k);
  if (d->wtype != MOE_WTYPE_BF16 && d->wtype != MOE_WTYPE_MXFP4 && d->wtype != MOE_WTYPE_NVFP4)
    return set_error(MOE_EUNSUPPORTED, "expert weight type %d not supported", d->wtype);
  if (d->router_wtype != MOE_WTYPE_BF16 && d->router_wtype != MOE_WTYPE_F32)
    return set_error(MOE_EUNSUPPORTED, "router weight type %d not supported", d->router_wtype);
  if (d->has_shared != 0 && d->has_shared != 1)
    return set_error(MOE_EINVAL, "has_shared must be 0 or 1");
  return MOE_OK;
}

void layout(const moe_desc* d, size_t off[6], size_t* bytes) {
  const size_t H = d->hidden, I = d->inter;
  if (d->wtype == MOE_WTYPE_BF16) {
    off[0] = 0;
    off[1] = I * H * 2;
    off[2] = 2 * I * H * 2;
    off[3] = off[4] = off[5] = 0;
    *bytes = align256(3 * I * H * 2);
  } else {
    const bool nv = d->wtype == MOE_WTYPE_NVFP4;
    const size_t cg = I * H / 2, sg = I * H / (nv ? 16 : 32);
    off[0] = 0;
    off[1] = cg;
    off[2] = cg + sg;
    off[3] = 2 * cg + sg;
    off[4] = 2 * cg + 2 * sg;
    off[5] = 3 * cg + 2 * sg;
    *bytes = align256(3 * cg + 3 * sg + (nv ? 16 : 0));   // NVFP4: three fp32 scales
  }
}

}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return moe::g_last_error.c_str(); }

int moe_expert_layout(const moe_desc* desc, size_t offsets[6], size_t* bytes) {
  int st = moe::check_desc(desc);
  if (st) return st;
  if (!offsets || !bytes) return moe::set_error(MOE_EINVAL, "null output pointer");
  moe::layout(desc, offsets, bytes);
  return MOE_OK;
}

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

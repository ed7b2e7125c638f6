// noalloc.hip - moe_route_decode for callers that cannot allocate: the decode
// workspace lives in a file-scope device array of fixed size instead of a
// caller-provided buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands in for the symbol): the device address of this GPU's
// copy comes from hipGetSymbolAddress once per device, with that device
// current, and only that address is used afterwards.  The first call on a
// device clears the array with a fill kernel on the caller's stream (the
// decode protocol needs a zero workspace once; every call leaves its counters
// at zero again).  Every call on a device shares its array, so calls that can
// overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"
#include "hip_error.hpp"

namespace moe {
namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;
  bool cleared = false;
};
std::mutex g_m;
DeviceScratch g_dev[kMaxDevices];

__global__ void clear_kernel(uint4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
}

// this device's copy of the array, cleared on `stream` the first time
int device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_status(err, "moe_route_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(MOE_EUNSUPPORTED, "moe_route_decode_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> g(g_m);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return hip_status(err != hipSuccess ? err : hipErrorInvalidSymbol,
                        "moe_route_decode_noalloc: hipGetSymbolAddress");
    d.ptr = p;
  }
  if (!d.cleared) {
    hipLaunchKernelGGL(clear_kernel, dim3(512), dim3(256), 0, stream,
                       static_cast<uint4*>(d.ptr), kScratchBytes / 16);
    err = hipGetLastError();
    if (err != hipSuccess) return hip_status(err, "moe_route_decode_noalloc: clear");
    d.cleared = true;
  }
  *out = d.ptr;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_decode_noalloc(const moe_desc* desc, const void* x,
                                        const void* w_router, int32_t T, int32_t* ids, float* w,
                                        const int32_t* slot_of_expert, const void* slot_pool,
                                        const void* shared_expert, float* y,
                                        int32_t* wait_status, void* stream) {
  moe::ApiRange range_("moe_route_decode_noalloc");
  if (T == 0) return moe_workspace_bytes(desc, 1, MOE_MODE_DECODE) ? MOE_OK : MOE_EINVAL;
  const size_t need = moe_workspace_bytes(desc, T, MOE_MODE_DECODE);
  if (need == 0) return MOE_EINVAL;   // bad descriptor or T: the text is set
  if (need > moe::kScratchBytes)
    return moe::set_error(MOE_EWORKSPACE,
                          "moe_route_decode_noalloc: T=%d with E=%d, k=%d, I=%d needs %zu bytes "
                          "of scratch; the static array holds %zu",
                          T, desc->n_experts, desc->top_k, desc->inter, need,
                          moe::kScratchBytes);
  void* ws = nullptr;
  int st = moe::device_scratch(static_cast<hipStream_t>(stream), &ws);
  if (st) return st;
  st = moe_route_decode(desc, x, w_router, T, ids, w, slot_of_expert, slot_pool, shared_expert,
                        y, ws, moe::kScratchBytes, stream);
  if (st) return st;
  if (wait_status) return moe_decode_status(ws, moe::kScratchBytes, wait_status, 1, stream);
  return MOE_OK;
}

// decode.hip - host-side glue of the one-kernel decode and of the standalone
// small-batch router (kernels in decode_impl.hpp).
#include "decode_impl.hpp"

namespace moe {
namespace dec {
hipError_t launch_bf16(DecArgs& a, hipStream_t st);
hipError_t launch_mxfp4(DecArgs& a, hipStream_t st);
hipError_t launch_nvfp4(DecArgs& a, hipStream_t st);
}  // namespace dec

using namespace dec;

namespace {
int elems_per_vector(int wtype) { return wtype == 1 ? 8 : 32; }
}  // namespace

bool decode_shape_supported(int wtype, int H, int I) {
  const int epv = elems_per_vector(wtype);
  if (H % epv || I % epv || I > kMaxI) return false;
  int lr, nv;
  return lx_cap((H / epv + 63) / 64) > 0 && down_map(I / epv, &lr, &nv);
}

bool route_small_supported(int router_f32, int H) { return H / (router_f32 ? 4 : 8) <= 64 * 16; }

hipError_t launch_route_small(const void* x, const void* w_router, int router_f32, int T, int H,
                              int E, int k, int renorm, float* z, unsigned* ticket, int32_t* ids,
                              float* w, hipStream_t st) {
  RouteArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.wr = w_router;
  a.T = T; a.H = H; a.E = E; a.k = k; a.renorm = renorm;
  a.z = z; a.ids = ids; a.w = w; a.ticket = ticket;
  return router_f32 ? launch_route_r<true>(a, st) : launch_route_r<false>(a, st);
}

int decode_max_tokens(int wtype, int H, int I) {
  const int t = max_tokens(H);
  const int m = wtype == 2 ? mf_max_tokens(H, I) : 0;
  return m > 0 && m < t ? m : t;
}

hipError_t launch_decode(const DecodeLaunch& f, hipStream_t st) {
  if (f.T < 1 || f.T > decode_max_tokens(f.wtype, f.H, f.I) || f.k > kMaxK || f.E > kMaxE)
    return hipErrorInvalidValue;
  DecArgs a;
  a.x = static_cast<const uint16_t*>(f.x);
  a.wr = f.w_router;
  a.router_f32 = f.router_f32;
  a.ids = f.ids;
  a.w = f.w;
  a.slot_of = f.slot_of;
  a.pool = static_cast<const uint8_t*>(f.pool);
  a.shared = static_cast<const uint8_t*>(f.shared);
  a.hdr = f.hdr;
  a.z = f.z;
  a.zstride = f.zstride;
  a.h = f.h;
  a.st = f.stamps;
  a.y = f.y;
  a.expert_bytes = f.expert_bytes;
  for (int i = 0; i < 6; ++i) a.off[i] = f.off[i];
  a.goff = f.goff;
  a.T = f.T; a.H = f.H; a.I = f.I; a.E = f.E; a.k = f.k; a.renorm = f.renorm;
  a.route = f.w_router ? 1 : 0;
  const int epv = elems_per_vector(f.wtype);
  a.lx = (f.H / epv + 63) / 64;
  if (!down_map(f.I / epv, &a.lr, &a.nv)) return hipErrorInvalidValue;
  a.G = 0;
  if (f.wtype == 1) return launch_bf16(a, st);
  return f.wtype == 3 ? launch_nvfp4(a, st) : launch_mxfp4(a, st);
}

}  // namespace moe

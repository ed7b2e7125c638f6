// decode.hip - host-side glue of the small-batch decode kernel and of the
// standalone router (kernels in decode_impl.hpp).
#include "decode_impl.hpp"

namespace moe {
namespace flow {
hipError_t launch_flow_bf16(FlowArgs& a, hipStream_t st);
hipError_t launch_flow_mxfp4(FlowArgs& a, hipStream_t st);
}  // namespace flow

using namespace flow;

size_t decode_plan_bytes() { return sizeof(Plan); }

bool decode_shape_supported(int wtype, int H, int I) {
  (void)I;
  return round_lg(H / (wtype == 1 ? 8 : 32)) > 0;
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

hipError_t launch_decode_flow(const FlowLaunch& f, hipStream_t st) {
  FlowArgs a;
  a.x = static_cast<const uint16_t*>(f.x);
  a.wr = f.w_router;
  a.router_f32 = f.router_f32;
  a.ids = f.ids;
  a.w = f.w;
  a.slot_of = f.slot_of;
  a.pool = static_cast<const uint8_t*>(f.pool);
  a.shared = static_cast<const uint8_t*>(f.shared);
  a.hdr = f.hdr;
  a.plan = static_cast<Plan*>(f.plan);
  a.z = f.z;
  a.h = f.h;
  a.y = f.y;
  a.expert_bytes = f.expert_bytes;
  for (int i = 0; i < 6; ++i) a.off[i] = f.off[i];
  a.T = f.T; a.H = f.H; a.I = f.I; a.E = f.E; a.k = f.k; a.renorm = f.renorm;
  a.NR = f.w_router ? (f.E + kFW - 1) / kFW : 1;
  return f.wtype == 1 ? launch_flow_bf16(a, st) : launch_flow_mxfp4(a, st);
}

}  // namespace moe

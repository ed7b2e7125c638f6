// decode_mxfp4.hip - the MXFP4-weight variants of the one-kernel decode
// (kernel in decode_impl.hpp); compiled apart so the two weight formats
// build in parallel.
#include "decode_impl.hpp"

namespace moe {
namespace flow {
namespace {

// ---------------------------------------------------------------------------
// flow launch: pick the compiled variant for (format, H, T, E)
// ---------------------------------------------------------------------------
template <int WT, int LG, int RGW, int TC, int M>
hipError_t launch_flow_t(const FlowArgs& a, hipStream_t st) {
  constexpr int PF = 4;
  hipLaunchKernelGGL((flow_kernel<WT, LG, RGW, 2, PF, TC, M>), dim3(a.NR + a.NGU + a.ND),
                     dim3(kFT), 0, st, a);
  return hipGetLastError();
}

template <int WT, int LG, int RGW, int TC>
hipError_t launch_flow_m(const FlowArgs& a, hipStream_t st) {
  if (a.E <= 128) return launch_flow_t<WT, LG, RGW, TC, 2>(a, st);
  if (a.E <= 256) return launch_flow_t<WT, LG, RGW, TC, 4>(a, st);
  return launch_flow_t<WT, LG, RGW, TC, 16>(a, st);
}

template <int WT, int LG, int RGW>
hipError_t launch_flow_c(const FlowArgs& a, hipStream_t st) {
  if (a.T <= 1) return launch_flow_m<WT, LG, RGW, 1>(a, st);
  if (a.T <= 4) return launch_flow_m<WT, LG, RGW, 4>(a, st);
  return launch_flow_m<WT, LG, RGW, 16>(a, st);
}

// gate/up rows per wave: about 16 (BF16) or 8 (MXFP4, whose decode needs more
// registers) sixteen-byte vectors of gate + up per lane
constexpr int rgw_for(int wt, int lg) {
  return wt == 1 ? (lg >= 8 ? 1 : (lg >= 3 ? 2 : (lg == 2 ? 4 : 8)))
                 : (lg >= 4 ? 1 : (lg >= 2 ? 2 : 4));
}


template <int WT>
hipError_t launch_flow_w(FlowArgs& a, hipStream_t st) {
  constexpr int EPV = WT == 1 ? 8 : 32;
  const int lg = round_lg(a.H / EPV);
  if (lg < 0) return hipErrorInvalidValue;
  a.rg = rgw_for(WT, lg) * kFW;
  a.gu_blocks = (a.I + a.rg - 1) / a.rg;
  a.NGU = (a.T * a.k + (a.shared ? 1 : 0)) * a.gu_blocks;
  a.rd = 2 * kFW;
  a.ND = (a.H + a.rd - 1) / a.rd;
  switch (lg) {
    case 1: return launch_flow_c<WT, 1, rgw_for(WT, 1)>(a, st);
    case 2: return launch_flow_c<WT, 2, rgw_for(WT, 2)>(a, st);
    case 3: return launch_flow_c<WT, 3, rgw_for(WT, 3)>(a, st);
    case 4: return launch_flow_c<WT, 4, rgw_for(WT, 4)>(a, st);
    case 6: return launch_flow_c<WT, 6, rgw_for(WT, 6)>(a, st);
    case 8: return launch_flow_c<WT, 8, rgw_for(WT, 8)>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_flow_mxfp4(FlowArgs& a, hipStream_t st) { return launch_flow_w<2>(a, st); }

}  // namespace flow
}  // namespace moe

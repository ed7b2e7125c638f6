// decode_launch.hpp - grid sizing and variant choice of the one-kernel decode
// (kernel in decode_impl.hpp), instantiated once per weight format.
#pragma once
#include "decode_impl.hpp"

#ifndef MOE_DECODE_WPC
#define MOE_DECODE_WPC 2   // workgroups per compute unit (capped by occupancy)
#endif

namespace moe {
namespace dec {

// compute units of the current device, cached per device
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int WT, int LXC, int NVC, int M>
hipError_t launch_t(DecArgs& a, hipStream_t st) {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<WT, LXC, NVC, M>, kT, 0) !=
        hipSuccess)
      n = 0;
    return n;
  }();
  const int cus = device_cus();
  if (occ <= 0 || cus <= 0) return hipErrorInvalidConfiguration;
  // every workgroup must be resident at once (they all meet at one wait)
  const int cap = cus * (occ < MOE_DECODE_WPC ? occ : MOE_DECODE_WPC);
  // no more workgroups than about two gate/up rows each
  const int64_t units = (int64_t)(a.T * a.k < a.E ? a.T * a.k : a.E) + (a.shared ? 1 : 0);
  const int64_t useful = (units * a.I + 1) / 2;
  int G = (int)(useful < cap ? useful : cap);
  if (G > cus * occ || G > 1024 || G < 1) return hipErrorInvalidConfiguration;
  a.G = G;
  hipLaunchKernelGGL((decode_kernel<WT, LXC, NVC, M>), dim3(G), dim3(kT), 0, st, a);
  return hipGetLastError();
}

// the matrix-core MXFP4 decode (decode_mfma.hpp): every workgroup resident,
// as many as have row groups to take in the down phase
template <int M>
hipError_t launch_mf(DecArgs& a, hipStream_t st) {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<M>, kT, 0) !=
        hipSuccess)
      n = 0;
    return n;
  }();
  const int cus = device_cus();
  if (occ <= 0 || cus <= 0) return hipErrorInvalidConfiguration;
  const int cap = cus * (occ < MOE_DECODE_WPC ? occ : MOE_DECODE_WPC);
  const int64_t units = (int64_t)(a.T * a.k < a.E ? a.T * a.k : a.E) + (a.shared ? 1 : 0);
  const int64_t groups = units * (a.H / 8);
  int G = (int)(groups < cap ? groups : cap);
  // the gate/up row groups of a fully resident batch (units * I / 8) split
  // with no remainder when a grid within 3/4 of the cap allows it (a
  // single token always routes to that many units)
  const int64_t gu = units * (a.I / 8);
  for (int g = G; 4 * g >= 3 * G && g > 0; --g)
    if (gu % g == 0) {
      G = g;
      break;
    }
  if (G > cus * occ || G > 1024 || G < 1) return hipErrorInvalidConfiguration;
  a.G = G;
  hipLaunchKernelGGL((decode_mfma_kernel<M>), dim3(G), dim3(kT), 0, st, a);
  return hipGetLastError();
}

template <int WT, int LXC, int NVC>
hipError_t launch_m(DecArgs& a, hipStream_t st) {
  return a.E <= 256 ? launch_t<WT, LXC, NVC, 4>(a, st) : launch_t<WT, LXC, NVC, 16>(a, st);
}

template <int WT, int LXC>
hipError_t launch_n(DecArgs& a, hipStream_t st) {
  switch (nv_cap(a.nv)) {
    case 1: return launch_m<WT, LXC, 1>(a, st);
    case 2: return launch_m<WT, LXC, 2>(a, st);
    case 4: return launch_m<WT, LXC, 4>(a, st);
    case 8: return launch_m<WT, LXC, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int WT>
hipError_t launch_w(DecArgs& a, hipStream_t st) {
  // MXFP4 batches of 2..8 tokens on the matrix core; one token on the
  // vector kernel, which measured faster there (DeepSeek-shaped layer 41 vs
  // 47 us; from 2 tokens on the matrix core is ahead, 67 vs 70 us at 2, 105
  // vs 124 us at 4)
  if (WT == 2 && a.T >= 2 && a.T <= mf_max_tokens(a.H, a.I))
    return a.E <= 256 ? launch_mf<4>(a, st) : launch_mf<16>(a, st);
  switch (lx_cap(a.lx)) {
    case 1: return launch_n<WT, 1>(a, st);
    case 2: return launch_n<WT, 2>(a, st);
    case 4: return launch_n<WT, 4>(a, st);
    case 8: return launch_n<WT, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
}  // namespace moe

// decode_impl.hpp - small-batch MoE layer in one kernel: router, top-k, expert
// FFNs (gate/up + SwiGLU, down) and the weighted combine.
//
// The layer is the sparse expert execution of the FreeToken pages: each
// token runs only its top-k experts and the output is their gate-weighted
// sum ("FreeToken 753b Model Explained", section of the same name).  Expert
// weights are reached through a slot table; experts without a slot are
// skipped, so the output is the partial sum over the resident subset
// (explainx.ai guide, "Decode: decide whether to move an expert or compute
// where it lives").
//
// Decode is bound by reading the selected experts' weights once from HBM.
// The kernel's workgroups take one of three roles, by block index:
//   router   [0, NR)        one wave per router row forms z[t][e]; the last
//                           router to finish ranks every token (DPP arg-max)
//                           and publishes the plan: distinct resident
//                           experts in first-appearance order (then the
//                           shared expert), each with its (pair, token, gate
//                           weight) list.  Without a router (ids given) one
//                           workgroup builds the plan.
//   gate/up  [NR, +NGU)     one (expert, block of RG rows of I) each: waits
//                           for the plan, streams its gate and up rows once,
//                           writes h = silu(g) * u for the expert's tokens
//   down     [.., +ND)      one block of RD rows of H each: waits for the
//                           plan, loads its down rows of every selected
//                           expert into registers while gate/up streams,
//                           waits for all h, then forms
//                           y[t][r] = sum_e w[t][e] * (W_down[e][r] . h[t][e])
//                           in a fixed order and overwrites y (no atomics).
// Waits are on counters with release/acquire fences and are bounded (an
// expired wait sets an error word instead of spinning forever).  Every wait
// is on workgroups with lower block indices, which the dispatcher starts
// first, so the roles cannot deadlock.
#pragma once
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace flow {

constexpr int kFT = 256;            // threads per workgroup
constexpr int kFW = kFT / 64;       // waves per workgroup
constexpr int kMaxE = 1024;
constexpr int kMaxPairs = 256;      // T * k per launch
constexpr int kMaxUnits = kMaxPairs + 1;
constexpr int kMaxT = 16;           // tokens per launch (larger batches are split)
constexpr int kMaxEntries = kMaxPairs + kMaxT;
constexpr int kHStage = 8192;       // floats of h staged in LDS per down pass
constexpr unsigned kSpinLimit = 1u << 20;

// header words of the workspace: every counter on its own 128-byte line, so
// polls of one do not queue behind updates of another
enum {
  kHRouted = 0, kHPlan = 32, kHGateUp = 64, kHExit = 96, kHError = 128, kHTiming = 160,
  kHStamps = 192
};

struct Plan {
  int n_units;                      // routed + shared
  int n_routed;
  int unit_slot[kMaxUnits];         // slot of each routed unit (shared: unused)
  int unit_start[kMaxUnits + 1];    // entries [start, start_next) per unit
  int ent_pair[kMaxEntries];        // pair id: t*k + j, or T*k + t for shared
  int ent_tok[kMaxEntries];
  float ent_gw[kMaxEntries];
};

struct FlowArgs {
  const uint16_t* x;
  const void* wr;          // router weights, null when ids/w are given
  int router_f32;
  int32_t* ids;            // [T][k]: out when routing, else in
  float* w;
  const int32_t* slot_of;
  const uint8_t* pool;
  const uint8_t* shared;
  unsigned* hdr;
  Plan* plan;
  float* z;                // [T][E]
  float* h;                // [T*k + T][I]
  float* y;                // [T][H]
  int64_t expert_bytes;
  int64_t off[6];
  int T, H, I, E, k, renorm;
  int NR, NGU, gu_blocks, rg, ND, rd;
};

// phase timing (header word kHTiming non-zero): 100 MHz wall clock at
// workgroup 0's start (slot 0) and exit (3), the planner's start (1) and
// publish (2), and the last workgroup's exit (4), as uint64 from word kHStamps
__device__ __forceinline__ void stamp(const FlowArgs& a, int i, bool any_block = false) {
  if ((any_block || blockIdx.x == 0) && threadIdx.x == 0 && a.hdr[kHTiming])
    reinterpret_cast<unsigned long long*>(a.hdr + kHStamps)[i] = wall_clock64();
}

// thread 0 only: wait until *p >= target, then acquire.  Polls back off
// (64 to 1024 cycles) so that a thousand waiting workgroups do not flood the
// line the counter sits on.
__device__ void wait_geq(const FlowArgs& a, unsigned* p, unsigned target) {
  unsigned spins = 0;
  int nap = 1;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (nap == 1) __builtin_amdgcn_s_sleep(1);
    else if (nap == 2) __builtin_amdgcn_s_sleep(2);
    else if (nap == 4) __builtin_amdgcn_s_sleep(4);
    else if (nap == 8) __builtin_amdgcn_s_sleep(8);
    else __builtin_amdgcn_s_sleep(16);
    if (nap < 16) nap <<= 1;
    if (++spins > kSpinLimit) {
      __hip_atomic_store(a.hdr + kHError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// thread 0 only: make this workgroup's writes visible, then count it
__device__ unsigned signal_add(unsigned* p) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// plan: top-k (or the given ids) -> units and their token lists
// ---------------------------------------------------------------------------
struct PlanLds {
  int ids[kMaxPairs];
  float w[kMaxPairs];
  int first[kMaxE];            // lowest pair per expert, then its unit
  int unit_expert[kMaxUnits];
  int cnt[kMaxUnits];
  int n_routed;
  int shared_base;
};

template <int M>
__device__ void build_plan(const FlowArgs& a, PlanLds& S, bool route) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, k = a.k, E = a.E, P = T * k;
  if (route) {
    for (int t = wave; t < T; t += kFW)
      topk_one_token<M>(a.z + (int64_t)t * E, E, k, a.renorm, &S.ids[t * k], &S.w[t * k]);
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += kFT) {
      a.ids[p] = S.ids[p];
      a.w[p] = S.w[p];
    }
  } else {
    for (int p = threadIdx.x; p < P; p += kFT) {
      S.ids[p] = a.ids[p];
      S.w[p] = a.w[p];
    }
  }
  for (int e = threadIdx.x; e < E; e += kFT) S.first[e] = 0x7fffffff;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kFT) {
    const int e = S.ids[p];
    bool ok = e >= 0 && e < E;
    if (ok && a.slot_of) ok = a.slot_of[e] >= 0;
    S.ids[p] = ok ? e : -1;
    if (ok) atomicMin(&S.first[e], p);
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int c = 0; c < P; c += 64) {
      const int p = c + lane;
      const int e = p < P ? S.ids[p] : -1;
      const bool isfirst = e >= 0 && S.first[e] == p;
      const uint64_t mask = __ballot(isfirst);
      const int rank = base + __popcll(mask & ((1ull << lane) - 1ull));
      if (isfirst) {
        S.unit_expert[rank] = e;
        a.plan->unit_slot[rank] = a.slot_of ? a.slot_of[e] : e;
        S.first[e] = rank;
      }
      base += __popcll(mask);
    }
    if (lane == 0) S.n_routed = base;
  }
  __syncthreads();
  const int n_routed = S.n_routed;
  // entries per routed unit, in pair order (one thread per unit)
  for (int u = threadIdx.x; u < n_routed; u += kFT) {
    const int e = S.unit_expert[u];
    int c = 0;
    for (int p = 0; p < P; ++p) c += S.ids[p] == e;
    S.cnt[u] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int pos = 0;
    for (int u = 0; u < n_routed; ++u) {
      a.plan->unit_start[u] = pos;
      const int c = S.cnt[u];
      S.cnt[u] = pos;
      pos += c;
    }
    const int n_units = n_routed + (a.shared ? 1 : 0);
    S.shared_base = pos;
    if (a.shared) {
      a.plan->unit_start[n_routed] = pos;
      pos += T;
    }
    a.plan->unit_start[n_units] = pos;
    a.plan->n_units = n_units;
    a.plan->n_routed = n_routed;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < n_routed; u += kFT) {
    const int e = S.unit_expert[u];
    int pos = S.cnt[u];
    for (int p = 0; p < P; ++p) {
      if (S.ids[p] == e) {
        a.plan->ent_pair[pos] = p;
        a.plan->ent_tok[pos] = p / k;
        a.plan->ent_gw[pos] = S.w[p];
        ++pos;
      }
    }
  }
  if (a.shared) {
    const int base = S.shared_base;
    for (int t = threadIdx.x; t < T; t += kFT) {
      a.plan->ent_pair[base + t] = P + t;
      a.plan->ent_tok[base + t] = t;
      a.plan->ent_gw[base + t] = 1.f;
    }
  }
}

// dot of one 16-byte weight vector with the matching h (fp32) elements
template <int WT>
__device__ __forceinline__ float wdot_h(const uint4 q, uint32_t sc, const float* hv) {
  if (WT == 1) {
    const float4 h0 = *reinterpret_cast<const float4*>(hv);
    const float4 h1 = *reinterpret_cast<const float4*>(hv + 4);
    float s = bf16_lo(q.x) * h0.x;
    s = fmaf(bf16_hi(q.x), h0.y, s);
    s = fmaf(bf16_lo(q.y), h0.z, s);
    s = fmaf(bf16_hi(q.y), h0.w, s);
    s = fmaf(bf16_lo(q.z), h1.x, s);
    s = fmaf(bf16_hi(q.z), h1.y, s);
    s = fmaf(bf16_lo(q.w), h1.z, s);
    return fmaf(bf16_hi(q.w), h1.w, s);
  } else {
    // one 32-bit word (8 codes) at a time keeps few h values live
    const float4* h4 = reinterpret_cast<const float4*>(hv);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 ha = h4[2 * i], hb = h4[2 * i + 1];
      const v2f c0 = fp4x2_to_f32x2<0>(w[i]);
      const v2f c1 = fp4x2_to_f32x2<1>(w[i]);
      const v2f c2 = fp4x2_to_f32x2<2>(w[i]);
      const v2f c3 = fp4x2_to_f32x2<3>(w[i]);
      acc = fmaf(c0.x, ha.x, acc);
      acc = fmaf(c0.y, ha.y, acc);
      acc = fmaf(c1.x, ha.z, acc);
      acc = fmaf(c1.y, ha.w, acc);
      acc = fmaf(c2.x, hb.x, acc);
      acc = fmaf(c2.y, hb.y, acc);
      acc = fmaf(c3.x, hb.z, acc);
      acc = fmaf(c3.y, hb.w, acc);
    }
    return acc * e8m0_to_f32(sc);
  }
}

union FlowLds {
  PlanLds plan;
  struct {
    int n_units;
    int slot;
    int start, end;
    int pair[kMaxT];
    int tok[kMaxT];
  } gu;
  struct {
    int n_units;
    int slot[kMaxUnits];
    int start[kMaxUnits + 1];
    int pair[kMaxEntries];
    int tok[kMaxEntries];
    float gw[kMaxEntries];
    float h[kHStage];          // h of the entries of one pass
  } dn;
};

// WT: 1 BF16, 2 MXFP4.  LG: 16-byte vectors per lane per gate/up row.  RGW:
// gate/up rows per wave.  RDW: down rows per wave.  PF: down vectors per lane
// kept in registers across the wait.  TC: tokens per down pass.  M: logits
// per lane in top-k.
template <int WT, int LG, int RGW, int RDW, int PF, int TC, int M>
__global__ __launch_bounds__(kFT, 4) void flow_kernel(FlowArgs a) {
  __shared__ FlowLds S;
  __shared__ int s_flag;
  constexpr int EPV = WT == 1 ? 8 : 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bid = blockIdx.x;
  const int T = a.T, H = a.H, I = a.I, E = a.E;
  const bool route = a.wr != nullptr;
  stamp(a, 0);

  if (bid < a.NR) {
    // ------------------------------ router ------------------------------
    if (route) {
      const int epv_r = a.router_f32 ? 4 : 8;
      const int nvr = H / epv_r;
      const int row_bytes = H * (a.router_f32 ? 4 : 2);
      const int e = bid * kFW + wave;
      if (e < E) {
        const uint8_t* row = static_cast<const uint8_t*>(a.wr) + (int64_t)e * row_bytes;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int t0 = 0; t0 < T; t0 += 4) {
          for (int i0 = 0; i0 * 64 < nvr; i0 += 4) {
            uint4 wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int v = lane + 64 * (i0 + i);
              wv[i] = v < nvr ? ldg16(row + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int v = lane + 64 * (i0 + i);
              if (v >= nvr) continue;
#pragma unroll
              for (int tt = 0; tt < 4; ++tt) {
                if (t0 + tt >= T) break;
                const uint16_t* xt = a.x + (int64_t)(t0 + tt) * H;
                float s = acc[tt];
                if (a.router_f32) {
                  const uint2 xx = *reinterpret_cast<const uint2*>(xt + v * 4);
                  s = fmaf(__uint_as_float(wv[i].x), bf16_lo(xx.x), s);
                  s = fmaf(__uint_as_float(wv[i].y), bf16_hi(xx.x), s);
                  s = fmaf(__uint_as_float(wv[i].z), bf16_lo(xx.y), s);
                  s = fmaf(__uint_as_float(wv[i].w), bf16_hi(xx.y), s);
                } else {
                  const uint4 xx = ldg16(xt + v * 8);
                  s = dot2_bf16(wv[i].x, xx.x, s);
                  s = dot2_bf16(wv[i].y, xx.y, s);
                  s = dot2_bf16(wv[i].z, xx.z, s);
                  s = dot2_bf16(wv[i].w, xx.w, s);
                }
                acc[tt] = s;
              }
            }
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (t0 + tt >= T) break;
            const float s = wave_sum_dpp(acc[tt]);
            if (lane == 0) a.z[(int64_t)(t0 + tt) * E + e] = s;
            acc[tt] = 0.f;
          }
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) s_flag = signal_add(a.hdr + kHRouted) == (unsigned)(a.NR - 1);
      __syncthreads();
      if (s_flag) {
        if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
        stamp(a, 1, true);
        build_plan<M>(a, S.plan, true);
        __syncthreads();
        if (threadIdx.x == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __hip_atomic_store(a.hdr + kHPlan, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        stamp(a, 2, true);
      }
    } else {
      build_plan<M>(a, S.plan, false);
      __syncthreads();
      if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(a.hdr + kHPlan, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else if (bid < a.NR + a.NGU) {
    // ------------------------------ gate / up ----------------------------
    const int g = bid - a.NR;
    if (threadIdx.x == 0) {
      wait_geq(a, a.hdr + kHPlan, 1u);
      S.gu.n_units = __hip_atomic_load(&a.plan->n_units, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int n_items = S.gu.n_units * a.gu_blocks;
    if (g < n_items) {
      const int u = g / a.gu_blocks;
      const int i0 = (g - u * a.gu_blocks) * a.rg;
      if (threadIdx.x == 0) {
        S.gu.slot = u < a.plan->n_routed ? a.plan->unit_slot[u] : -1;
        S.gu.start = a.plan->unit_start[u];
        S.gu.end = a.plan->unit_start[u + 1];
      }
      __syncthreads();
      const int ntok = min(S.gu.end - S.gu.start, kMaxT);
      for (int q = threadIdx.x; q < ntok; q += kFT) {
        S.gu.pair[q] = a.plan->ent_pair[S.gu.start + q];
        S.gu.tok[q] = a.plan->ent_tok[S.gu.start + q];
      }
      const uint8_t* base =
          S.gu.slot < 0 ? a.shared : a.pool + (int64_t)S.gu.slot * a.expert_bytes;
      const int nvh = H / EPV;
      uint4 gq[RGW][LG], uq[RGW][LG];
      uint32_t gs[RGW][LG], us[RGW][LG];
#pragma unroll
      for (int rr = 0; rr < RGW; ++rr) {
        const int i = i0 + wave * RGW + rr;
#pragma unroll
        for (int l = 0; l < LG; ++l) {
          const int v = lane + 64 * l;
          gq[rr][l] = uq[rr][l] = make_uint4(0, 0, 0, 0);
          gs[rr][l] = us[rr][l] = 0;
          if (i < I && v < nvh) {
            if (WT == 1) {
              gq[rr][l] = ldg16(base + a.off[0] + ((int64_t)i * H + (int64_t)v * 8) * 2);
              uq[rr][l] = ldg16(base + a.off[1] + ((int64_t)i * H + (int64_t)v * 8) * 2);
            } else {
              gq[rr][l] = ldg16(base + a.off[0] + (int64_t)i * (H / 2) + (int64_t)v * 16);
              uq[rr][l] = ldg16(base + a.off[2] + (int64_t)i * (H / 2) + (int64_t)v * 16);
              gs[rr][l] = (base + a.off[1])[(int64_t)i * (H / 32) + v];
              us[rr][l] = (base + a.off[3])[(int64_t)i * (H / 32) + v];
            }
          }
        }
      }
      __syncthreads();
      for (int q = 0; q < ntok; ++q) {
        const uint16_t* xt = a.x + (int64_t)S.gu.tok[q] * H;
        float gp[RGW], up[RGW];
#pragma unroll
        for (int rr = 0; rr < RGW; ++rr) gp[rr] = up[rr] = 0.f;
#pragma unroll
        for (int l = 0; l < LG; ++l) {
          const int v = lane + 64 * l;
          if (v >= nvh) continue;
          if (WT == 1) {
            const uint4 xx = ldg16(xt + (int64_t)v * 8);
#pragma unroll
            for (int rr = 0; rr < RGW; ++rr) {
              float g2 = gp[rr], u2 = up[rr];
              g2 = dot2_bf16(gq[rr][l].x, xx.x, g2);
              g2 = dot2_bf16(gq[rr][l].y, xx.y, g2);
              g2 = dot2_bf16(gq[rr][l].z, xx.z, g2);
              gp[rr] = dot2_bf16(gq[rr][l].w, xx.w, g2);
              u2 = dot2_bf16(uq[rr][l].x, xx.x, u2);
              u2 = dot2_bf16(uq[rr][l].y, xx.y, u2);
              u2 = dot2_bf16(uq[rr][l].z, xx.z, u2);
              up[rr] = dot2_bf16(uq[rr][l].w, xx.w, u2);
            }
          } else {
            uint32_t xp[16];
            const uint4* xs = reinterpret_cast<const uint4*>(xt + (int64_t)v * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint4 t4 = xs[j];
              xp[4 * j] = t4.x; xp[4 * j + 1] = t4.y; xp[4 * j + 2] = t4.z; xp[4 * j + 3] = t4.w;
            }
#pragma unroll
            for (int rr = 0; rr < RGW; ++rr) {
              gp[rr] = fmaf(dot_fp4_bf16_block(gq[rr][l], xp), e8m0_to_f32(gs[rr][l]), gp[rr]);
              up[rr] = fmaf(dot_fp4_bf16_block(uq[rr][l], xp), e8m0_to_f32(us[rr][l]), up[rr]);
            }
          }
        }
#pragma unroll
        for (int rr = 0; rr < RGW; ++rr) {
          const float gsum = wave_sum_dpp(gp[rr]);
          const float usum = wave_sum_dpp(up[rr]);
          const int i = i0 + wave * RGW + rr;
          if (lane == 0 && i < I)
            a.h[(int64_t)S.gu.pair[q] * I + i] = gsum / (1.0f + expf(-gsum)) * usum;
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) signal_add(a.hdr + kHGateUp);
    }
  } else {
    // ------------------------------ down ---------------------------------
    const int d = bid - a.NR - a.NGU;
    if (threadIdx.x == 0) {
      wait_geq(a, a.hdr + kHPlan, 1u);
      S.dn.n_units = __hip_atomic_load(&a.plan->n_units, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int n_units = S.dn.n_units;
    const int n_routed = a.plan->n_routed;
    for (int u = threadIdx.x; u <= n_units; u += kFT) {
      S.dn.start[u] = a.plan->unit_start[u];
      if (u < n_units) S.dn.slot[u] = u < n_routed ? a.plan->unit_slot[u] : -1;
    }
    __syncthreads();
    const int n_ent = min(S.dn.start[n_units], kMaxEntries);
    for (int q = threadIdx.x; q < n_ent; q += kFT) {
      S.dn.pair[q] = a.plan->ent_pair[q];
      S.dn.tok[q] = a.plan->ent_tok[q];
      S.dn.gw[q] = a.plan->ent_gw[q];
    }
    const int r0 = d * a.rd + wave * RDW;
    const int nvi = I / EPV;
    const int per_unit = RDW * nvi;
    const int n_slots = n_units * per_unit;
    __syncthreads();
    auto slot_load = [&](int s, uint4& q, uint32_t& sc) {
      const int u = s / per_unit;
      const int rem = s - u * per_unit;
      const int rr = rem / nvi, v = rem - rr * nvi;
      const int row = r0 + rr;
      q = make_uint4(0, 0, 0, 0);
      sc = 0;
      if (row < H) {
        const int slot = S.dn.slot[u];
        const uint8_t* b = slot < 0 ? a.shared : a.pool + (int64_t)slot * a.expert_bytes;
        if (WT == 1) {
          q = ldg16(b + a.off[2] + ((int64_t)row * I + (int64_t)v * 8) * 2);
        } else {
          q = ldg16(b + a.off[4] + (int64_t)row * (I / 2) + (int64_t)v * 16);
          sc = (b + a.off[5])[(int64_t)row * (I / 32) + v];
        }
      }
    };
    uint4 pre[PF];
    uint32_t psc[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int s = lane + 64 * j;
      if (s < n_slots) slot_load(s, pre[j], psc[j]);
      else { pre[j] = make_uint4(0, 0, 0, 0); psc[j] = 0; }
    }
    if (threadIdx.x == 0) wait_geq(a, a.hdr + kHGateUp, (unsigned)(n_units * a.gu_blocks));
    __syncthreads();
    // Passes over entry ranges [e0, e1) whose h fits the LDS stage; a slot
    // contributes in every pass that holds entries of its expert.
    const int cap = kHStage / I;              // entries per pass (>= 1: I <= kHStage)
    int u_lo = 0;
    for (int e0 = 0; e0 < n_ent; e0 += cap) {
      const int e1 = min(n_ent, e0 + cap);
      while (S.dn.start[u_lo + 1] <= e0) ++u_lo;
      int u_hi = u_lo;
      while (u_hi + 1 < n_units && S.dn.start[u_hi + 1] < e1) ++u_hi;
      __syncthreads();
      {
        const int n4 = (e1 - e0) * (I / 4);
        for (int q = threadIdx.x; q < n4; q += kFT) {
          const int en = e0 + q / (I / 4), c4 = q % (I / 4);
          reinterpret_cast<float4*>(S.dn.h)[q] =
              reinterpret_cast<const float4*>(a.h + (int64_t)S.dn.pair[en] * I)[c4];
        }
      }
      __syncthreads();
      const int s_lo = u_lo * per_unit, s_hi = (u_hi + 1) * per_unit;
      float acc[RDW][kMaxT];
#pragma unroll
      for (int r2 = 0; r2 < RDW; ++r2)
#pragma unroll
        for (int tt = 0; tt < kMaxT; ++tt) acc[r2][tt] = 0.f;
      auto consume = [&](int s, const uint4& q, uint32_t sc) {
        const int u = s / per_unit;
        const int rem = s - u * per_unit;
        const int rr = rem / nvi, v = rem - rr * nvi;
        if (r0 + rr >= H) return;
        const int ea = max(S.dn.start[u], e0), eb = min(S.dn.start[u + 1], e1);
        for (int en = ea; en < eb; ++en) {
          const int t = S.dn.tok[en];
          const float c = S.dn.gw[en] * wdot_h<WT>(q, sc, &S.dn.h[(en - e0) * I + v * EPV]);
#pragma unroll
          for (int r2 = 0; r2 < RDW; ++r2)
#pragma unroll
            for (int t2 = 0; t2 < TC; ++t2)
              if (r2 == rr && t2 == t) acc[r2][t2] += c;
        }
      };
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int s = lane + 64 * j;
        if (s >= s_lo && s < s_hi && s < n_slots) consume(s, pre[j], psc[j]);
      }
      constexpr int SB = 4;     // streamed slots in flight per lane
      int s_first = lane + 64 * PF;
      if (s_first < s_lo) s_first += ((s_lo - s_first + 63) / 64) * 64;
      for (int s = s_first; s - lane < s_hi; s += 64 * SB) {
        uint4 q[SB];
        uint32_t sc[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (s + 64 * i < s_hi) slot_load(s + 64 * i, q[i], sc[i]);
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (s + 64 * i < s_hi) consume(s + 64 * i, q[i], sc[i]);
      }
#pragma unroll
      for (int r2 = 0; r2 < RDW; ++r2) {
#pragma unroll
        for (int tt = 0; tt < TC; ++tt) {
          const float v = wave_sum_dpp(acc[r2][tt]);
          const int row = r0 + r2;
          if (lane == 0 && row < H && tt < T) {
            float* yp = a.y + (int64_t)tt * H + row;
            *yp = (e0 == 0 ? 0.f : *yp) + v;
          }
        }
      }
    }
    if (n_ent == 0) {
      // nothing resident: y is zero
#pragma unroll
      for (int r2 = 0; r2 < RDW; ++r2)
        for (int t = lane; t < T; t += 64)
          if (r0 + r2 < H) a.y[(int64_t)t * H + r0 + r2] = 0.f;
    }
  }

  // ------------------------------ exit ------------------------------------
  stamp(a, 3);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(a.hdr + kHExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(a.hdr + kHRouted, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.hdr + kHPlan, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.hdr + kHGateUp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.hdr + kHExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.hdr[kHTiming])
        reinterpret_cast<unsigned long long*>(a.hdr + kHStamps)[4] = wall_clock64();
    }
  }
}

// ---------------------------------------------------------------------------
// standalone router (moe_route, T <= 64): one wave per row, last workgroup ranks
// ---------------------------------------------------------------------------
struct RouteArgs {
  const uint16_t* x;
  const void* wr;
  int T, H, E, k, renorm;
  float* z;
  int32_t* ids;
  float* w;
  unsigned* ticket;
};

template <bool RF32, int L, int M>
__global__ __launch_bounds__(kFT) void route_kernel(RouteArgs a) {
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * kFW + wave;
  const int H = a.H, E = a.E, T = a.T;
  constexpr int EPV = RF32 ? 4 : 8;
  const int nvr = H / EPV;
  if (e < E) {
    const uint8_t* row = static_cast<const uint8_t*>(a.wr) + (int64_t)e * H * (RF32 ? 4 : 2);
    uint4 wv[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int v = lane + 64 * i;
      wv[i] = v < nvr ? ldg16(row + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
    }
    for (int t = 0; t < T; ++t) {
      const uint16_t* xt = a.x + (int64_t)t * H;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int v = lane + 64 * i;
        if (v >= nvr) continue;
        if (RF32) {
          const uint2 xx = *reinterpret_cast<const uint2*>(xt + v * 4);
          acc = fmaf(__uint_as_float(wv[i].x), bf16_lo(xx.x), acc);
          acc = fmaf(__uint_as_float(wv[i].y), bf16_hi(xx.x), acc);
          acc = fmaf(__uint_as_float(wv[i].z), bf16_lo(xx.y), acc);
          acc = fmaf(__uint_as_float(wv[i].w), bf16_hi(xx.y), acc);
        } else {
          const uint4 xx = ldg16(xt + v * 8);
          acc = dot2_bf16(wv[i].x, xx.x, acc);
          acc = dot2_bf16(wv[i].y, xx.y, acc);
          acc = dot2_bf16(wv[i].z, xx.z, acc);
          acc = dot2_bf16(wv[i].w, xx.w, acc);
        }
      }
      acc = wave_sum_dpp(acc);
      if (lane == 0) a.z[(int64_t)t * E + e] = acc;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) s_last = signal_add(a.ticket) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  for (int t = wave; t < T; t += kFW)
    topk_one_token<M>(a.z + (int64_t)t * E, E, a.k, a.renorm, a.ids + (int64_t)t * a.k,
                      a.w + (int64_t)t * a.k);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool RF32, int L, int M>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((route_kernel<RF32, L, M>), dim3((a.E + kFW - 1) / kFW), dim3(kFT), 0, st,
                     a);
  return hipGetLastError();
}

template <bool RF32, int L>
hipError_t launch_route_l(const RouteArgs& a, hipStream_t st) {
  if (a.E <= 64) return launch_route_t<RF32, L, 1>(a, st);
  if (a.E <= 128) return launch_route_t<RF32, L, 2>(a, st);
  if (a.E <= 256) return launch_route_t<RF32, L, 4>(a, st);
  return launch_route_t<RF32, L, 16>(a, st);
}

template <bool RF32>
hipError_t launch_route_r(const RouteArgs& a, hipStream_t st) {
  const int l = (a.H / (RF32 ? 4 : 8) + 63) / 64;
  if (l <= 1) return launch_route_l<RF32, 1>(a, st);
  if (l <= 2) return launch_route_l<RF32, 2>(a, st);
  if (l <= 4) return launch_route_l<RF32, 4>(a, st);
  if (l <= 8) return launch_route_l<RF32, 8>(a, st);
  if (l <= 12) return launch_route_l<RF32, 12>(a, st);
  return launch_route_l<RF32, 16>(a, st);
}

// 16-byte vectors per lane per row, rounded up to a compiled variant
inline int round_lg(int nvec) {
  const int l = (nvec + 63) / 64;
  if (l <= 4) return l < 1 ? 1 : l;
  if (l <= 6) return 6;
  if (l <= 8) return 8;
  return -1;
}

}  // namespace flow
}  // namespace moe

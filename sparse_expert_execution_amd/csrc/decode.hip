// decode.hip - small-batch expert FFNs: grouped GEMV over the distinct
// resident experts, SwiGLU, and the down projection with the weighted
// combine.  Weight rows stream from HBM once per call with 16-byte loads
// per lane; MXFP4 codes are decoded in registers.
//
// The layer: each token runs through the k experts the router picked, and
// its output is the gate-weighted sum of their outputs ("FreeToken 753b
// Model Explained", section of the same name).  Expert weights are reached
// through a slot table; experts without a slot are skipped, so the output is
// the partial sum over the resident subset (explainx.ai guide, "Decode:
// decide whether to move an expert or compute where it lives").
#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPairs = 1024;
constexpr int kMaxExperts = 1024;

struct DecodeArgs {
  const uint16_t* x;        // [T][H] bf16
  const int32_t* ids;       // [T][k]
  const float* w;           // [T][k]
  const int32_t* slot_of;   // [E] or null (identity)
  const uint8_t* pool;      // slot base
  const uint8_t* shared;    // shared expert block or null
  float* h;                 // [T*k + T][I] fp32 (workspace)
  float* y;                 // [T][H]
  int64_t expert_bytes;
  int64_t off[6];           // section offsets inside an expert block
  int T, H, I, E, k;
};

// Canonical unit list, built identically by every workgroup: the distinct
// resident routed experts in order of first appearance over pairs
// p = t*k + j, followed by the shared expert when present.
struct Units {
  int n_routed;
  int s_ids[kMaxPairs];         // expert of pair p, -1 if skipped
  int s_unit_expert[kMaxPairs]; // expert of unit u
  int s_unit_slot[kMaxPairs];   // slot of unit u
  int s_first[kMaxExperts];     // lowest pair index per expert
  int s_scan[4];
};

__device__ void build_units(const DecodeArgs& a, Units& U) {
  const int P = a.T * a.k;
  for (int e = threadIdx.x; e < a.E; e += kThreads) U.s_first[e] = 0x7fffffff;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kThreads) {
    int e = a.ids[p];
    int ok = (e >= 0 && e < a.E);
    if (ok && a.slot_of) ok = a.slot_of[e] >= 0;
    U.s_ids[p] = ok ? e : -1;
    if (ok) atomicMin(&U.s_first[e], p);
  }
  __syncthreads();
  // each thread owns 4 consecutive pairs
  int cnt = 0, flags = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int p = threadIdx.x * 4 + i;
    if (p < P) {
      int e = U.s_ids[p];
      if (e >= 0 && U.s_first[e] == p) { flags |= 1 << i; ++cnt; }
    }
  }
  int total;
  int off = block256_exclusive_scan(cnt, &total, U.s_scan);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (flags & (1 << i)) {
      int e = U.s_ids[threadIdx.x * 4 + i];
      U.s_unit_expert[off] = e;
      U.s_unit_slot[off] = a.slot_of ? a.slot_of[e] : e;
      ++off;
    }
  }
  if (threadIdx.x == 0) U.n_routed = total;
  __syncthreads();
}

__device__ __forceinline__ const uint8_t* unit_base(const DecodeArgs& a, const Units& U, int u) {
  if (u >= U.n_routed) return a.shared;
  return a.pool + (int64_t)U.s_unit_slot[u] * a.expert_bytes;
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  grid.x = unit (T*k + shared upper bound), grid.y = row
// block of ROWS = 4 waves * RW rows of I.  Each wave loads RW gate rows and
// RW up rows once, then for every token of its unit forms g and u, and
// writes h = silu(g) * u for that (token, expert) pair.
// WT: 1 = BF16 weights (8 elements / 16 B), 2 = MXFP4 (32 elements / 16 B).
// L: 16-byte vectors per lane per row (ceil(H / epv / 64)).
// ---------------------------------------------------------------------------
template <int WT, int L, int RW>
__global__ __launch_bounds__(kThreads) void gateup_kernel(DecodeArgs a) {
  __shared__ Units U;
  __shared__ int s_tok[kMaxPairs];
  __shared__ int s_ntok;
  build_units(a, U);
  const int u = blockIdx.x;
  const int n_units = U.n_routed + (a.shared ? 1 : 0);
  if (u >= n_units) return;
  const bool is_shared = u >= U.n_routed;
  const int P = a.T * a.k;
  if (threadIdx.x == 0) s_ntok = 0;
  __syncthreads();
  if (is_shared) {
    for (int t = threadIdx.x; t < a.T; t += kThreads) s_tok[t] = P + t;
    if (threadIdx.x == 0) s_ntok = a.T;
  } else {
    const int e = U.s_unit_expert[u];
    for (int p = threadIdx.x; p < P; p += kThreads)
      if (U.s_ids[p] == e) s_tok[atomicAdd(&s_ntok, 1)] = p;
  }
  __syncthreads();
  const int ntok = s_ntok;

  constexpr int EPV = WT == 1 ? 8 : 32;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nvec = a.H / EPV;
  const int row0 = (blockIdx.y * 4 + wv) * RW;
  const uint8_t* base = unit_base(a, U, u);

  // weights: RW gate rows then RW up rows
  uint4 wq[2 * RW][L];
  uint32_t sc[2 * RW][L];
#pragma unroll
  for (int r = 0; r < 2 * RW; ++r) {
    const int row = row0 + (r % RW);
    const bool row_ok = row < a.I;
    const int mat = r / RW;  // 0 gate, 1 up
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int v = lane + 64 * i;
      wq[r][i] = make_uint4(0, 0, 0, 0);
      sc[r][i] = 0;
      if (row_ok && v < nvec) {
        if (WT == 1) {
          const uint8_t* m = base + a.off[mat];
          wq[r][i] = ldg16(m + ((int64_t)row * a.H + (int64_t)v * EPV) * 2);
        } else {
          const uint8_t* c = base + a.off[2 * mat];
          const uint8_t* s = base + a.off[2 * mat + 1];
          wq[r][i] = ldg16(c + (int64_t)row * (a.H / 2) + (int64_t)v * 16);
          sc[r][i] = s[(int64_t)row * (a.H / 32) + v];
        }
      }
    }
  }

  for (int it = 0; it < ntok; ++it) {
    const int pair = s_tok[it];
    const int t = pair < P ? pair / a.k : pair - P;
    const uint16_t* xt = a.x + (int64_t)t * a.H;
    float acc[2 * RW];
#pragma unroll
    for (int r = 0; r < 2 * RW; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int v = lane + 64 * i;
      if (v < nvec) {
        if (WT == 1) {
          const uint4 xv = ldg16(xt + (int64_t)v * 8);
#pragma unroll
          for (int r = 0; r < 2 * RW; ++r) {
            float s = acc[r];
            s = dot2_bf16(wq[r][i].x, xv.x, s);
            s = dot2_bf16(wq[r][i].y, xv.y, s);
            s = dot2_bf16(wq[r][i].z, xv.z, s);
            s = dot2_bf16(wq[r][i].w, xv.w, s);
            acc[r] = s;
          }
        } else {
          uint32_t xp[16];
          const uint4* xs = reinterpret_cast<const uint4*>(xt + (int64_t)v * 32);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint4 q = xs[j];
            xp[4 * j + 0] = q.x; xp[4 * j + 1] = q.y; xp[4 * j + 2] = q.z; xp[4 * j + 3] = q.w;
          }
#pragma unroll
          for (int r = 0; r < 2 * RW; ++r)
            acc[r] = fmaf(dot_fp4_bf16_block(wq[r][i], xp), e8m0_to_f32(sc[r][i]), acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2 * RW; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const int row = row0 + r;
        if (row < a.I) {
          const float g = acc[r], up = acc[RW + r];
          const float sg = g / (1.0f + expf(-g));
          a.h[(int64_t)pair * a.I + row] = sg * up;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down projection + weighted combine.  grid.x = row block of H (4 waves, one
// row each), grid.y = token chunk of TC tokens.  Every workgroup walks the
// canonical unit list in order, UB units at a time (weights for UB units are
// in flight together), and accumulates w[t][j] * (W_down row . h[pair]) per
// token in registers; y is overwritten, so no zero fill and no atomics.
// ---------------------------------------------------------------------------
template <int WT, int L, int TC, int UB>
__global__ __launch_bounds__(kThreads) void down_kernel(DecodeArgs a) {
  __shared__ Units U;
  build_units(a, U);
  const int n_units = U.n_routed + (a.shared ? 1 : 0);
  constexpr int EPV = WT == 1 ? 8 : 32;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wv;
  const int t0 = blockIdx.y * TC;
  const int nvec = a.I / EPV;
  const int P = a.T * a.k;
  const bool row_ok = row < a.H;

  float acc[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) acc[c] = 0.f;

  for (int ub = 0; ub < n_units; ub += UB) {
    uint4 wq[UB][L];
    uint32_t sc[UB][L];
    int pair[UB][TC];
    float gw[UB][TC];
#pragma unroll
    for (int b = 0; b < UB; ++b) {
      const int u = ub + b;
      bool any = false;
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        pair[b][c] = -1;
        gw[b][c] = 0.f;
        const int t = t0 + c;
        if (u < n_units && t < a.T) {
          if (u >= U.n_routed) {
            pair[b][c] = P + t;
            gw[b][c] = 1.f;
          } else {
            const int e = U.s_unit_expert[u];
            for (int j = 0; j < a.k; ++j) {
              if (U.s_ids[t * a.k + j] == e) {
                pair[b][c] = t * a.k + j;
                gw[b][c] = a.w[t * a.k + j];
                break;
              }
            }
          }
        }
        any |= pair[b][c] >= 0;
      }
      const uint8_t* base = (u < n_units) ? unit_base(a, U, u) : nullptr;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int v = lane + 64 * i;
        wq[b][i] = make_uint4(0, 0, 0, 0);
        sc[b][i] = 0;
        if (any && row_ok && v < nvec) {
          if (WT == 1) {
            wq[b][i] = ldg16(base + a.off[2] + ((int64_t)row * a.I + (int64_t)v * EPV) * 2);
          } else {
            wq[b][i] = ldg16(base + a.off[4] + (int64_t)row * (a.I / 2) + (int64_t)v * 16);
            sc[b][i] = (base + a.off[5])[(int64_t)row * (a.I / 32) + v];
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < UB; ++b) {
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        if (pair[b][c] < 0) continue;
        const float* hp = a.h + (int64_t)pair[b][c] * a.I;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < L; ++i) {
          const int v = lane + 64 * i;
          if (v < nvec) {
            if (WT == 1) {
              const float4 h0 = *reinterpret_cast<const float4*>(hp + v * 8);
              const float4 h1 = *reinterpret_cast<const float4*>(hp + v * 8 + 4);
              const uint4 q = wq[b][i];
              part = fmaf(bf16_lo(q.x), h0.x, part);
              part = fmaf(bf16_hi(q.x), h0.y, part);
              part = fmaf(bf16_lo(q.y), h0.z, part);
              part = fmaf(bf16_hi(q.y), h0.w, part);
              part = fmaf(bf16_lo(q.z), h1.x, part);
              part = fmaf(bf16_hi(q.z), h1.y, part);
              part = fmaf(bf16_lo(q.w), h1.z, part);
              part = fmaf(bf16_hi(q.w), h1.w, part);
            } else {
              float hv[32];
              const float4* h4 = reinterpret_cast<const float4*>(hp + v * 32);
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                float4 f = h4[j];
                hv[4 * j] = f.x; hv[4 * j + 1] = f.y; hv[4 * j + 2] = f.z; hv[4 * j + 3] = f.w;
              }
              part = fmaf(dot_fp4_f32_block(wq[b][i], hv), e8m0_to_f32(sc[b][i]), part);
            }
          }
        }
        acc[c] = fmaf(gw[b][c], part, acc[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    const float s = wave_sum(acc[c]);
    const int t = t0 + c;
    if (lane == 0 && row_ok && t < a.T) a.y[(int64_t)t * a.H + row] = s;
  }
}

template <int WT, int L>
hipError_t launch_gateup(const DecodeArgs& a, hipStream_t st) {
  constexpr int RW = 2;
  const int n_units_max = a.T * a.k + (a.shared ? 1 : 0);
  dim3 grid(n_units_max, (a.I + 4 * RW - 1) / (4 * RW));
  hipLaunchKernelGGL((gateup_kernel<WT, L, RW>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int WT, int L>
hipError_t launch_down(const DecodeArgs& a, hipStream_t st) {
  constexpr int TC = 4, UB = 4;
  dim3 grid((a.H + 3) / 4, (a.T + TC - 1) / TC);
  hipLaunchKernelGGL((down_kernel<WT, L, TC, UB>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// vectors per lane per row, rounded up to a compiled variant
int pick_L(int nvec) {
  int l = (nvec + 63) / 64;
  if (l <= 1) return 1;
  if (l <= 2) return 2;
  if (l <= 3) return 3;
  if (l <= 4) return 4;
  if (l <= 6) return 6;
  if (l <= 8) return 8;
  if (l <= 12) return 12;
  if (l <= 16) return 16;
  return -1;
}

template <int WT>
hipError_t dispatch_gateup(const DecodeArgs& a, hipStream_t st) {
  switch (pick_L(a.H / (WT == 1 ? 8 : 32))) {
    case 1: return launch_gateup<WT, 1>(a, st);
    case 2: return launch_gateup<WT, 2>(a, st);
    case 3: return launch_gateup<WT, 3>(a, st);
    case 4: return launch_gateup<WT, 4>(a, st);
    case 6: return launch_gateup<WT, 6>(a, st);
    case 8: return launch_gateup<WT, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int WT>
hipError_t dispatch_down(const DecodeArgs& a, hipStream_t st) {
  switch (pick_L(a.I / (WT == 1 ? 8 : 32))) {
    case 1: return launch_down<WT, 1>(a, st);
    case 2: return launch_down<WT, 2>(a, st);
    case 3: return launch_down<WT, 3>(a, st);
    case 4: return launch_down<WT, 4>(a, st);
    case 6: return launch_down<WT, 6>(a, st);
    case 8: return launch_down<WT, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_shape_supported(int wtype, int H, int I) {
  const int epv = wtype == 1 ? 8 : 32;
  const int lg = pick_L(H / epv), ld = pick_L(I / epv);
  return lg > 0 && lg <= 8 && ld > 0 && ld <= 8;
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t st) {
  DecodeArgs a;
  a.x = static_cast<const uint16_t*>(d.x);
  a.ids = d.ids;
  a.w = d.w;
  a.slot_of = d.slot_of;
  a.pool = static_cast<const uint8_t*>(d.pool);
  a.shared = static_cast<const uint8_t*>(d.shared);
  a.h = d.h;
  a.y = d.y;
  a.expert_bytes = d.expert_bytes;
  for (int i = 0; i < 6; ++i) a.off[i] = d.off[i];
  a.T = d.T; a.H = d.H; a.I = d.I; a.E = d.E; a.k = d.k;
  hipError_t err;
  if (d.wtype == 1) {
    err = dispatch_gateup<1>(a, st);
    if (err == hipSuccess) err = dispatch_down<1>(a, st);
  } else {
    err = dispatch_gateup<2>(a, st);
    if (err == hipSuccess) err = dispatch_down<2>(a, st);
  }
  return err;
}

}  // namespace moe

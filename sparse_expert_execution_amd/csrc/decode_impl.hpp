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
// Decode is bound by reading the selected experts' weights once from HBM, so
// the kernel is a persistent grid (every workgroup resident at once) that
// keeps as many of those reads in flight as it can:
//   1. every workgroup stages x into LDS, takes its share of the router dot
//      products z[t][e] = W_r[e] . x[t] (stored tagged with the launch's
//      generation), clears its slice of y and starts on its share of the
//      shared expert's gate/up rows, which need no routing.
//   2. every workgroup polls the logits until they carry this launch's
//      generation, ranks the tokens itself (softmax + rank count for small
//      batches, a DPP arg-max per token otherwise; the same result in every
//      workgroup) and lists the distinct resident experts in first-appearance
//      order with their (pair, token, weight) entries.
//   3. gate/up: the rows of I of all selected experts are split evenly over
//      the grid; a wave streams one gate row and one up row at a time (two in
//      flight), dots them with each of the expert's tokens and writes
//      h = silu(g) * u to the workspace, tagged with the launch's generation.
//   4. each workgroup issues the loads of its first down rows; there is no
//      grid-wide wait: the h values a workgroup needs are polled one by one
//      until they carry this launch's generation.
//   5. down: the rows of H of every expert (its tokens in chunks of two) are
//      split evenly over the grid; each row is dotted with h of each of the
//      chunk's tokens and the gate-weighted result added into y[t][row] with
//      an fp32 atomic, once every workgroup has cleared its slice of y.
// Waits are bounded: an expired wait sets an error word and lets the kernel
// finish with wrong results instead of hanging.
#pragma once
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace dec {

constexpr int kT = 512;             // threads per workgroup (one workgroup per CU)
constexpr int kW = kT / 64;         // waves per workgroup
constexpr int kMaxE = 1024;
constexpr int kMaxT = 16;           // tokens per launch (larger batches are split)
constexpr int kMaxK = 8;
constexpr int kMaxPairs = kMaxT * kMaxK;
constexpr int kMaxUnits = kMaxPairs + 1;
constexpr int kMaxEntries = kMaxPairs + kMaxT;
constexpr int kXStage16 = 7680;     // 16-byte words of staged x (120 KB)
constexpr int kHStage4 = 1536;      // float4s of the per-wave h lists (24 KB)
constexpr int kYOut = 512;          // y results per wave list in the down phase
constexpr int kDnH4 = kXStage16 + kHStage4 - kW * kYOut / 2;  // float4s of staged h (down)
constexpr int kMaxCE = 2;           // entries per virtual unit of the down phase, at most
constexpr int kMfTab = 64;          // row groups per batch of the matrix-core path, at most
constexpr unsigned kSpinLimit = 1u << 21;

// a value the same in every lane of the wave, kept in a scalar register
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Header words of the decode workspace (8 KB), every counter on its own
// 128-byte line.  A grid-wide count is spread over kNCtr lines (workgroup b
// counts on line b % kNCtr) so that the atomics of a full grid do not queue
// on one address.
constexpr int kLine = 32;           // words per 128-byte line
constexpr int kNCtr = 16;
enum {
  kHGen = 0,                        // generation of the last finished launch
  kHError = 32,                     // 1: a wait expired
  kHTiming = 64,                    // non-zero: record phase stamps
  kHExitTop = 96,                   // exit groups complete
  kHYZero = 128,                    // kNCtr lines: workgroups that cleared their y slice
  kHExit = kHYZero + kNCtr * kLine,   // kNCtr lines: workgroups exited
  kHStamps = kHExit + kNCtr * kLine   // uint64 phase stamps
};

struct DecArgs {
  const uint16_t* x;       // [T][H] bf16
  const void* wr;          // router weights, null when ids/w are given
  int router_f32;
  int32_t* ids;            // [T][k]: out when routing, else in
  float* w;
  const int32_t* slot_of;  // null: expert e sits in slot e
  const uint8_t* pool;
  const uint8_t* shared;
  unsigned* hdr;
  uint64_t* z;             // kZCopies x [T][E] logits tagged with the generation
  int64_t zstride;         // uint64 words between the copies
  uint64_t* h;             // [T*k + T][I] h values tagged with the generation
  unsigned long long* st;  // [workgroup][16] phase stamps
  float* y;                // [T][H]
  int64_t expert_bytes;
  int64_t off[6];
  int64_t goff;            // NVFP4: offset of the gate, up, down fp32 scales
  int T, H, I, E, k, renorm;
  int G;                   // workgroups in the grid, all resident at once
  int route;               // 0: ids and w are inputs
  int lx;                  // 16-byte vectors per lane per gate/up row
  int lr;                  // lanes per down row (a power of two <= 64)
  int nv;                  // 16-byte vectors per lane per down row
  unsigned gen;            // this launch's generation (set in the kernel)
};

// phase timing (header word kHTiming non-zero): 100 MHz wall clock of
// workgroup 0 at start (0), expert list ready (1), past the grid-wide wait
// (2), exit (3), router dot products done (5), first token's logits in (6),
// gate/up done (7), gate/up counted (8), top-k done (9), h staged (11), a
// down pass done (12), and of the last
// workgroup's exit (4), as uint64 from kHStamps; the same stamps of the
// grid's last workgroup 16 slots further; every workgroup's stamps also go to
// its own 16 slots of a.st
__device__ __forceinline__ void stamp(bool on, const DecArgs& a, int i) {
  if (on && threadIdx.x == 0) {
    const unsigned long long c = wall_clock64();
    a.st[blockIdx.x * 16 + i] = c;
    if (blockIdx.x == 0 || blockIdx.x == gridDim.x - 1)
      reinterpret_cast<unsigned long long*>(a.hdr + kHStamps)[i + (blockIdx.x ? 16 : 0)] = c;
  }
}

// Data that one workgroup hands to others (z, h, the cleared y) is written
// with agent-coherent stores and read with agent-coherent loads, so a hand-off
// needs no cache write-back or invalidation: the writer waits for its stores
// to complete before it is counted, the reader polls the count before it
// loads.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }



// every wave waits for its coherent stores, then thread 0 counts the
// workgroup on its line of a spread count
__device__ void signal_done(unsigned* count) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(count + (blockIdx.x % kNCtr) * kLine, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// wave 0 only: wait until the lines of a spread count add up to target (the
// header's error word is set when the wait gives up).  It takes the header
// rather than the kernel's arguments: a call the compiler does not inline
// would otherwise copy the whole argument block into scratch memory, and
// every later argument read would go through it.
__device__ void wait_count(unsigned* hdr, unsigned* count, unsigned target) {
  const int lane = threadIdx.x & 63;
  unsigned spins = 0;
  int nap = 1;
  for (;;) {
    const unsigned v = lane < kNCtr ? __hip_atomic_load(count + lane * kLine, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0u;
    if (__builtin_amdgcn_readfirstlane((unsigned)wave_sum_dpp((float)v)) >= target) break;
    if (nap == 1) __builtin_amdgcn_s_sleep(1);
    else if (nap == 2) __builtin_amdgcn_s_sleep(2);
    else if (nap == 4) __builtin_amdgcn_s_sleep(4);
    else __builtin_amdgcn_s_sleep(8);
    if (nap < 8) nap <<= 1;
    if (++spins > kSpinLimit) {
      if (lane == 0)
        __hip_atomic_store(hdr + kHError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// Logits handed from the router workgroups to every workgroup: each z is
// stored with the launch's generation in its upper half, and a reader polls
// its entries until all carry this launch's generation (a launch's
// generation is one more than the header's, which the last workgroup out
// advances).  No count and no wait for store completion are needed.
__device__ __forceinline__ void z_store(uint64_t* p, float z, unsigned gen) {
  __hip_atomic_store(p, ((uint64_t)gen << 32) | __float_as_uint(z), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Every logit is written to kZCopies copies of z, and workgroup b polls copy
// b % kZCopies: all workgroups poll the logits at once, and a single copy's
// few cache lines would queue their requests at one memory channel.
__device__ __forceinline__ const uint64_t* zcopy(const DecArgs& a) {
  return a.z + (int64_t)(blockIdx.x % kZCopies) * a.zstride;
}

// one wave: logits of expert lane + 64 i of row zt into v (-inf past E)
template <int M>
__device__ __forceinline__ void z_load(const DecArgs& a, const uint64_t* zt, unsigned gen, float v[M]) {
  const int lane = threadIdx.x & 63;
  bool have[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    have[i] = lane + 64 * i >= a.E;
    v[i] = -INFINITY;
  }
  unsigned spins = 0;
  for (;;) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (!have[i]) {
        const uint64_t q =
            __hip_atomic_load(zt + lane + 64 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)(q >> 32) == gen) {
          v[i] = __uint_as_float((unsigned)q);
          have[i] = true;
        } else {
          all = false;
        }
      }
    }
    if (__all(all)) break;
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      if (lane == 0)
        __hip_atomic_store(a.hdr + kHError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// [lo, hi) of an even split of n items over G parts
__device__ __forceinline__ void split(int64_t n, int G, int j, int64_t& lo, int64_t& hi) {
  lo = n * j / G;
  hi = n * (j + 1) / G;
}

// Per-wave list of (index, value) results in LDS, written to memory in one
// burst.  Waits on vector memory count loads and stores together, in issue
// order, so a store or atomic issued between a load and the use of its data
// would make that use wait for the store as well; results are therefore
// collected here and written out when the list fills or the phase ends.
struct WaveOut {
  int2* buf;
  int cap, n;                    // n is the same in every lane
};

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
struct PlanLds {
  int ids[kMaxPairs];
  float w[kMaxPairs];
  float zsel[kMaxPairs];         // logit of each selected pair
  float mx[kMaxT], inv[kMaxT];   // softmax max and 1 / sum per token
  int first[kMaxE];              // lowest pair per expert, then its unit
  int unit_expert[kMaxUnits];
  int unit_slot[kMaxUnits];      // -1: the shared expert
  int unit_start[kMaxUnits + 1]; // entries [start, next start) per unit
  int cnt[kMaxUnits];
  int ent_pair[kMaxEntries];     // t*k + j, or T*k + t for the shared expert
  int ent_tok[kMaxEntries];
  float ent_gw[kMaxEntries];
  // down work: each unit's entries in chunks of at most CE (virtual units)
  int vu_unit[kMaxEntries], vu_e0[kMaxEntries], vu_n[kMaxEntries];
  int n_routed, n_units, n_vu;
  // matrix-core path: the row groups of one batch (slot of the expert block,
  // -1 the shared expert; first row; unit).  A slot, not a pointer: a
  // pointer read back from LDS loses its address space and every load
  // through it becomes a flat load, whose waits cannot be counted.
  int mf_slot[kMfTab], mf_row[kMfTab], mf_unit[kMfTab];
  int mf_hoff[kMfTab];     // down: byte offset of the group's unit's h stage
};

struct DecLds {
  PlanLds p;
  union {
    struct {                       // routing and gate/up
      // x of every token: 16-byte word (t * CPV + c) * NV + v holds elements
      // 8c..8c+7 of weight vector v (CPV = elements per vector / 8, NV
      // vectors per row), so the lanes of a wave read consecutive words
      uint4 xs[kXStage16];
      float4 hs[kHStage4];         // per-wave lists of gate/up h results
    } g;
    // the matrix-core path lays out its own stages in the same bytes
    uint8_t raw[(kXStage16 + kHStage4) * 16];
    struct {                       // down
      int2 yout[kW * kYOut];       // per-wave lists of y results
      // h of the entries of one down pass; an entry's I values as float4s at
      // (c * V + v) for elements 4c..4c+3 of 16-byte weight vector v (V
      // vectors per row), so the lanes of a row group read consecutive float4s
      float4 hst[kDnH4];
    } d;
  };
};

// Boundary b of a split of the rows of units [0, nu) (R rows each) over G
// parts by cost, where a row of unit u weighs A + B * (its entries): the cost
// ahead of unit u is (A u + B unit_start[u]) R, and boundary b is the row
// where the cost passes b / G of the total (a binary search over the units).
// Adjacent parts compute the same boundary, so the ranges tile the rows;
// with B = 0 it is the even split.
__device__ __forceinline__ int cost_bound(const PlanLds& P, int nu, int R, int A, int B, int b,
                                          int G) {
  auto cost = [&](int u) -> int64_t {
    return ((int64_t)A * u + (int64_t)B * uni(P.unit_start[u])) * R;
  };
  const int64_t target = cost(nu) * b / G;
  int lo = 0, hi = nu;                    // the last unit u with cost(u) <= target
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cost(mid) <= target) lo = mid;
    else hi = mid - 1;
  }
  if (lo >= nu) return nu * R;
  const int64_t wu =
      (int64_t)A + (int64_t)B * (uni(P.unit_start[lo + 1]) - uni(P.unit_start[lo]));
  return uni((int)(lo * R + (target - cost(lo)) / wu));
}

// ---------------------------------------------------------------------------
// routing: z rows (router workgroups) and the per-workgroup expert list
// ---------------------------------------------------------------------------
// Router dot products z[t][e] = W_r[e] . x[t] over the whole grid: item i is
// (expert i % E, tokens kRTG * (i / E) ...), taken by workgroup i % G, wave
// (i / G) % kW, so every workgroup has a share.  A row is read in rounds of
// kRL 16-byte vectors per lane; x comes from the LDS stage.
constexpr int kRTG = 4;    // tokens per router item
constexpr int kRL = 8;     // row vectors per lane per round

struct RouterRow {
  uint4 v[kRL];
};

__device__ __forceinline__ int router_items(const DecArgs& a) {
  return a.E * ((a.T + kRTG - 1) / kRTG);
}
__device__ __forceinline__ int router_rounds(const DecArgs& a) {
  const int nvr = a.H / (a.router_f32 ? 4 : 8);
  return (nvr + 64 * kRL - 1) / (64 * kRL);
}

__device__ __forceinline__ void router_load(const DecArgs& a, int item, int c, RouterRow& w) {
  const int lane = threadIdx.x & 63;
  const int e = item % a.E;
  const int nvr = a.H / (a.router_f32 ? 4 : 8);
  const uint8_t* row =
      static_cast<const uint8_t*>(a.wr) + (int64_t)e * a.H * (a.router_f32 ? 4 : 2);
#pragma unroll
  for (int r = 0; r < kRL; ++r) {
    const int v = lane + 64 * (c * kRL + r);
    w.v[r] = v < nvr ? ldg16(row + (int64_t)v * 16) : make_uint4(0, 0, 0, 0);
  }
}

// 8 bf16 values of token t, elements 8u .. 8u + 7, from the x stage
template <int WT>
__device__ __forceinline__ uint4 xs8(const DecArgs& a, const DecLds& S, int t, int u) {
  if (WT == 1) return S.g.xs[t * (a.H / 8) + u];
  return S.g.xs[(t * 4 + (u & 3)) * (a.H / 32) + (u >> 2)];
}

template <int WT>
__device__ __forceinline__ void router_dot(const DecArgs& a, const DecLds& S, int item, int c,
                                           const RouterRow& w, float acc[kRTG]) {
  const int lane = threadIdx.x & 63;
  const int t0 = (item / a.E) * kRTG;
  const int nvr = a.H / (a.router_f32 ? 4 : 8);
#pragma unroll
  for (int r = 0; r < kRL; ++r) {
    const int v = lane + 64 * (c * kRL + r);
    if (v >= nvr) continue;
#pragma unroll
    for (int tt = 0; tt < kRTG; ++tt) {
      if (t0 + tt >= a.T) break;
      float s = acc[tt];
      if (a.router_f32) {
        const uint4 xx = xs8<WT>(a, S, t0 + tt, v >> 1);
        const uint32_t x0 = (v & 1) ? xx.z : xx.x, x1 = (v & 1) ? xx.w : xx.y;
        s = fmaf(__uint_as_float(w.v[r].x), bf16_lo(x0), s);
        s = fmaf(__uint_as_float(w.v[r].y), bf16_hi(x0), s);
        s = fmaf(__uint_as_float(w.v[r].z), bf16_lo(x1), s);
        s = fmaf(__uint_as_float(w.v[r].w), bf16_hi(x1), s);
      } else {
        const uint4 xx = xs8<WT>(a, S, t0 + tt, v);
        s = dot2_bf16(w.v[r].x, xx.x, s);
        s = dot2_bf16(w.v[r].y, xx.y, s);
        s = dot2_bf16(w.v[r].z, xx.z, s);
        s = dot2_bf16(w.v[r].w, xx.w, s);
      }
      acc[tt] = s;
    }
  }
}

// this wave's router items from `item` on (its first round already loaded
// into w), each z written with an agent-coherent store
template <int WT>
__device__ __forceinline__ void router_items_run(const DecArgs& a, const DecLds& S, int item, RouterRow& w,
                                 unsigned gen) {
  const int lane = threadIdx.x & 63;
  const int n_items = router_items(a), nr = router_rounds(a);
  bool loaded = true;
  for (; item < n_items; item += a.G * kW) {
    float acc[kRTG] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nr; ++c) {
      if (!loaded) router_load(a, item, c, w);
      loaded = false;
      router_dot<WT>(a, S, item, c, w, acc);
    }
    const int e = item % a.E, t0 = (item / a.E) * kRTG;
#pragma unroll
    for (int tt = 0; tt < kRTG; ++tt) {
      if (t0 + tt >= a.T) break;
      const float z = wave_sum_dpp(acc[tt]);
      if (lane < kZCopies)
        z_store(a.z + lane * a.zstride + (int64_t)(t0 + tt) * a.E + e, z, gen);
    }
  }
}

// sum over aligned groups of lr lanes (a power of two <= 64), result in every
// lane of the group
__device__ __forceinline__ float group_sum(float v, int lr) {
  if (lr == 64) return wave_sum_dpp(v);
  if (lr >= 2) v += dpp_f<kDppXor1>(v);
  if (lr >= 4) v += dpp_f<kDppXor2>(v);
  if (lr >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (lr >= 16) v += dpp_f<kDppMirror>(v);
  if (lr == 32) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
  }
  return v;
}

// Expert list of this launch, built the same way in every workgroup: the
// distinct resident experts in order of first appearance over the (token,
// rank) pairs, each with its pairs in order, then the shared expert.
// Top-k of every token when T * E <= kRankItems, by the whole workgroup: the
// logits go to LDS (polled until they carry this launch's generation); an
// expert's rank is the number of experts ahead of it (larger logit, or equal
// logit and lower id), so the k experts of rank < k land directly in
// descending order.  Leaves ids, each selected logit (zsel) and each token's
// softmax max and 1 / sum (mx, inv; max-subtracted, fp32).
constexpr int kRankItems = 128;

__device__ __forceinline__ void rank_topk(const DecArgs& a, DecLds& S, unsigned gen, float* zs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, E = a.E, k = a.k, n = T * E;
  const int E4 = (E + 3) & ~3;             // rows padded to whole float4s with -inf
  for (int i = threadIdx.x; i < T * E4; i += kT) {
    const int t = i / E4, e = i - t * E4;
    float z = -INFINITY;
    if (e < E) {
      const uint64_t* p = zcopy(a) + (int64_t)t * E + e;
      unsigned spins = 0;
      uint64_t q = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      while ((unsigned)(q >> 32) != gen) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          __hip_atomic_store(a.hdr + kHError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        q = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      z = __uint_as_float((unsigned)q);
    }
    zs[i] = z;
  }
  __syncthreads();
  for (int t = wave; t < T; t += kW) {
    const float* zt = zs + t * E4;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, zt[e]);
    m = wave_max_dpp(m);
    float ps = 0.f;
    for (int e = lane; e < E; e += 64) ps += expf(zt[e] - m);
    ps = wave_sum_dpp(ps);
    if (lane == 0) {
      S.p.mx[t] = m;
      S.p.inv[t] = 1.0f / ps;
    }
  }
  // sp threads per expert, each counting over every sp-th float4 of the row
  int sp = 1;
  while (sp < 8 && n * sp * 2 <= kT) sp <<= 1;
  for (int i = threadIdx.x; i < n * sp; i += kT) {
    const int item = i / sp, part = i - item * sp;
    const int t = item / E, e = item - t * E;
    const float4* zt4 = reinterpret_cast<const float4*>(zs + t * E4);
    const float my = zs[t * E4 + e];
    int rank = 0;
#pragma unroll 4
    for (int c = part; c < E4 / 4; c += sp) {
      const float4 z4 = zt4[c];
      const int e2 = 4 * c;
      rank += (z4.x > my) | ((z4.x == my) & (e2 < e));
      rank += (z4.y > my) | ((z4.y == my) & (e2 + 1 < e));
      rank += (z4.z > my) | ((z4.z == my) & (e2 + 2 < e));
      rank += (z4.w > my) | ((z4.w == my) & (e2 + 3 < e));
    }
    rank = (int)group_sum((float)rank, sp);
    if (part == 0 && rank < k) {
      S.p.ids[t * k + rank] = e;
      S.p.zsel[t * k + rank] = my;
    }
  }
  __syncthreads();
}

// inclusive prefix sum over the lanes of a wave (all lanes active): the DPP
// scan, or log2(64) steps of __shfl_up.  The two are equal; which one a
// kernel takes is a measured choice (the DPP form took the DeepSeek-shaped
// MXFP4 T=1 call from 44.8 to 43.7 us, while the Qwen-shaped BF16 call went
// from 28.4 to 28.8 us, i.e. code placement, not the scan, decides there).
template <bool DPP>
__device__ __forceinline__ int wave_scan(int v) {
  if (DPP) return wave_scan_dpp(v);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// The expert list by one wave when T * k + (shared expert) <= 64 (one pair,
// and at most one unit, per lane), with
// ballots and wave-ordered LDS accesses instead of workgroup barriers: units
// in first-appearance order of their expert over the pairs, a unit's entries
// in any order (each entry's result is independent of the others), then the
// shared expert's T entries and the virtual units of the down phase.  from_zsel:
// the gate weights come from the selected logits and the softmax statistics
// (renormalised here when asked), else they are in L.w.
template <int CE, bool DPP>
__device__ __forceinline__ void build_units_wave(const DecArgs& a, DecLds& S, bool route, bool from_zsel) {
  PlanLds& L = S.p;
  const int lane = threadIdx.x & 63;
  const int T = a.T, k = a.k, E = a.E, P = T * k;
  const int p = lane;
  int e = -1;
  float wp = 0.f;
  if (p < P) {
    e = L.ids[p];
    if (from_zsel) {
      const int t = p / k;
      wp = expf(L.zsel[p] - L.mx[t]) * L.inv[t];
    } else {
      wp = L.w[p];
    }
  }
  if (from_zsel && a.renorm) {
    if (p < P) L.w[p] = wp;
    float sum = 0.f;
    if (p < P) {
      const int t0 = (p / k) * k;
      for (int j = 0; j < k; ++j) sum += L.w[t0 + j];
      wp /= sum;
    }
  }
  if (route && blockIdx.x == 0 && p < P) {
    a.ids[p] = e;
    a.w[p] = wp;
  }
  int slot = -1;
  if (p < P && e >= 0 && e < E) slot = a.slot_of ? a.slot_of[e] : e;
  const bool ok = slot >= 0;
  if (ok) L.first[e] = 0x7fffffff;
  if (ok) atomicMin(&L.first[e], p);
  const bool isfirst = ok && L.first[e] == p;
  const uint64_t fm = __ballot(isfirst);
  const int n_routed = __popcll(fm);
  if (isfirst) {
    const int u = __popcll(fm & ((1ull << lane) - 1ull));
    L.unit_expert[u] = e;
    L.unit_slot[u] = slot;
    L.first[e] = u;                        // from here on: the expert's unit
  }
  if (lane <= n_routed) L.cnt[lane] = 0;
  const int u = ok ? L.first[e] : 0;
  int li = 0;
  if (ok) li = atomicAdd(&L.cnt[u], 1);
  const bool sh = a.shared != nullptr;
  const int n_units = n_routed + (sh ? 1 : 0);
  const int c = lane < n_routed ? L.cnt[lane] : (sh && lane == n_routed ? T : 0);
  const int incl = wave_scan<DPP>(c);
  if (lane < n_units) L.unit_start[lane] = incl - c;
  if (lane == 0) L.unit_start[n_units] = __builtin_amdgcn_readlane(incl, 63);
  if (sh && lane == n_routed) L.unit_slot[lane] = -1;
  const int start = incl - c;
  const int ustart = __shfl(start, u);     // with every lane active
  if (ok) {
    const int pos = ustart + li;
    L.ent_pair[pos] = p;
    L.ent_tok[pos] = p / k;
    L.ent_gw[pos] = wp;
  }
  if (sh) {
    const int base = __shfl(start, n_routed);
    if (lane < T) {
      L.ent_pair[base + lane] = P + lane;
      L.ent_tok[base + lane] = lane;
      L.ent_gw[base + lane] = 1.f;
    }
  }
  // virtual units: each unit's entries in chunks of CE
  const int nv = lane < n_units ? (c + CE - 1) / CE : 0;
  const int vincl = wave_scan<DPP>(nv);
  for (int j = 0; j < nv; ++j) {
    const int q = vincl - nv + j;
    L.vu_unit[q] = lane;
    L.vu_e0[q] = start + j * CE;
    L.vu_n[q] = c - j * CE < CE ? c - j * CE : CE;
  }
  if (lane == 63) L.n_vu = vincl;
  if (lane == 0) {
    L.n_routed = n_routed;
    L.n_units = n_units;
  }
}

// One routed token: its k experts are distinct (the router's own top-k), so
// the resident ones, in rank order, are the units, each with one entry, and
// the list follows from a ballot alone.  Every write below is independent
// (no LDS read back), which saves the chain of dependent LDS round trips of
// the general list (about 1.2 us of the call).  Wave 0 only; the result is
// the general list's for this case.
__device__ __forceinline__ void build_units_t1(const DecArgs& a, DecLds& S, bool from_zsel) {
  PlanLds& L = S.p;
  const int lane = threadIdx.x & 63;
  const int k = a.k, E = a.E;
  const bool live = lane < k;
  const int e = live ? L.ids[lane] : -1;
  float wp = 0.f;
  if (live) wp = from_zsel ? expf(L.zsel[lane] - L.mx[0]) * L.inv[0] : L.w[lane];
  if (from_zsel && a.renorm) {
    float sum = wp;
    sum += dpp_f<kDppXor1>(sum);       // k <= 8 lanes: a row-local sum is enough
    sum += dpp_f<kDppXor2>(sum);
    sum += dpp_f<kDppHalfMirror>(sum);
    if (live) wp /= sum;
  }
  if (blockIdx.x == 0 && live) {
    a.ids[lane] = e;
    a.w[lane] = wp;
  }
  int slot = -1;
  if (live && e >= 0 && e < E) slot = a.slot_of ? a.slot_of[e] : e;
  const bool ok = slot >= 0;
  const uint64_t m = __ballot(ok);
  const int n_routed = __popcll(m);
  const int u = __popcll(m & ((1ull << lane) - 1ull));
  if (ok) {
    L.unit_expert[u] = e;
    L.unit_slot[u] = slot;
    L.unit_start[u] = u;
    L.ent_pair[u] = lane;
    L.ent_tok[u] = 0;
    L.ent_gw[u] = wp;
    L.vu_unit[u] = u;
    L.vu_e0[u] = u;
    L.vu_n[u] = 1;
  }
  const int n_units = n_routed + (a.shared ? 1 : 0);
  if (lane == 0) {
    if (a.shared) {
      L.unit_slot[n_routed] = -1;
      L.unit_start[n_routed] = n_routed;
      L.ent_pair[n_routed] = k;
      L.ent_tok[n_routed] = 0;
      L.ent_gw[n_routed] = 1.f;
      L.vu_unit[n_routed] = n_routed;
      L.vu_e0[n_routed] = n_routed;
      L.vu_n[n_routed] = 1;
    }
    L.unit_start[n_units] = n_units;
    L.n_routed = n_routed;
    L.n_units = n_units;
    L.n_vu = n_units;
  }
}

// Expert list of this launch, built the same way in every workgroup: the
// distinct resident experts in order of first appearance over the (token,
// rank) pairs, each with its pairs, then the shared expert.
template <int M, int CE, bool DPP>
__device__ __forceinline__ void build_units(const DecArgs& a, DecLds& S, bool route, bool timing, unsigned gen,
                                            float* zs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, k = a.k, E = a.E, P = T * k;
  PlanLds& L = S.p;
  const bool from_zsel = route && T * E <= kRankItems;
  if (from_zsel) {
    rank_topk(a, S, gen, zs);
  } else if (route) {
    for (int t = wave; t < T; t += kW) {
      float v[M];
      z_load<M>(a, zcopy(a) + (int64_t)t * E, gen, v);
      stamp(timing, a, 6);
      topk_select<M>(v, E, k, a.renorm, &L.ids[t * k], &L.w[t * k]);
    }
    __syncthreads();
  } else {
    for (int p = threadIdx.x; p < P; p += kT) {
      L.ids[p] = a.ids[p];
      L.w[p] = a.w[p];
    }
    __syncthreads();
  }
  stamp(timing, a, 9);
  if (route && T == 1) {
    if (wave == 0) build_units_t1(a, S, from_zsel);
    __syncthreads();
    return;
  }
  if (P + (a.shared ? 1 : 0) <= 64) {
    if (wave == 0) build_units_wave<CE, DPP>(a, S, route, from_zsel);
    __syncthreads();
    return;
  }
  if (from_zsel) {
    for (int p = threadIdx.x; p < P; p += kT)
      L.w[p] = expf(L.zsel[p] - L.mx[p / k]) * L.inv[p / k];
    __syncthreads();
    if (a.renorm) {
      for (int t = threadIdx.x; t < T; t += kT) {
        float s = 0.f;
        for (int j = 0; j < k; ++j) s += L.w[t * k + j];
        for (int j = 0; j < k; ++j) L.w[t * k + j] /= s;
      }
      __syncthreads();
    }
  }
  for (int e = threadIdx.x; e < E; e += kT) L.first[e] = 0x7fffffff;
  __syncthreads();
  if (route && blockIdx.x == 0) {
    for (int p = threadIdx.x; p < P; p += kT) {
      a.ids[p] = L.ids[p];
      a.w[p] = L.w[p];
    }
  }
  for (int p = threadIdx.x; p < P; p += kT) {
    const int e = L.ids[p];
    bool ok = e >= 0 && e < E;
    if (ok && a.slot_of) ok = a.slot_of[e] >= 0;
    if (ok) atomicMin(&L.first[e], p);
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int c = 0; c < P; c += 64) {
      const int p = c + lane;
      const int e = p < P ? L.ids[p] : -1;
      const bool isfirst = e >= 0 && e < E && L.first[e] == p;
      const uint64_t mask = __ballot(isfirst);
      const int rank = base + __popcll(mask & ((1ull << lane) - 1ull));
      if (isfirst) {
        L.unit_expert[rank] = e;
        L.unit_slot[rank] = a.slot_of ? a.slot_of[e] : e;
      }
      base += __popcll(mask);
    }
    if (lane == 0) L.n_routed = base;
  }
  __syncthreads();
  const int n_routed = L.n_routed;
  for (int u = threadIdx.x; u < n_routed; u += kT) {
    const int e = L.unit_expert[u];
    int c = 0;
    for (int p = 0; p < P; ++p) c += L.ids[p] == e;
    L.cnt[u] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int pos = 0;
    for (int u = 0; u < n_routed; ++u) {
      L.unit_start[u] = pos;
      pos += L.cnt[u];
    }
    int n_units = n_routed;
    if (a.shared) {
      L.unit_start[n_routed] = pos;
      L.unit_slot[n_routed] = -1;
      pos += T;
      ++n_units;
    }
    L.unit_start[n_units] = pos;
    L.n_units = n_units;
    int nvu = 0;
    for (int u = 0; u < n_units; ++u) {
      const int e1 = L.unit_start[u + 1];
      for (int e = L.unit_start[u]; e < e1; e += CE) {
        L.vu_unit[nvu] = u;
        L.vu_e0[nvu] = e;
        L.vu_n[nvu] = e1 - e < CE ? e1 - e : CE;
        ++nvu;
      }
    }
    L.n_vu = nvu;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < n_routed; u += kT) {
    const int e = L.unit_expert[u];
    int pos = L.unit_start[u];
    for (int p = 0; p < P; ++p) {
      if (L.ids[p] == e) {
        L.ent_pair[pos] = p;
        L.ent_tok[pos] = p / k;
        L.ent_gw[pos] = L.w[p];
        ++pos;
      }
    }
  }
  if (a.shared) {
    const int base = L.unit_start[n_routed];
    for (int t = threadIdx.x; t < T; t += kT) {
      L.ent_pair[base + t] = P + t;
      L.ent_tok[base + t] = t;
      L.ent_gw[base + t] = 1.f;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ const uint8_t* unit_base(const DecArgs& a, int slot) {
  return slot < 0 ? a.shared : a.pool + (int64_t)slot * a.expert_bytes;
}

// ---------------------------------------------------------------------------
// gate/up rows
// ---------------------------------------------------------------------------
// x of every token into LDS in the layout DecLds::xs describes
template <int WT>
__device__ __forceinline__ void stage_x(const DecArgs& a, DecLds& S) {
  constexpr int CPV = WT == 1 ? 1 : 4;
  const int NV = a.H / (8 * CPV);
  const int n = a.T * a.H / 8;
  for (int q = threadIdx.x; q < n; q += kT) {
    const int t = q / (a.H / 8), w8 = q - t * (a.H / 8);
    const int v = w8 / CPV, c = w8 - v * CPV;
    S.g.xs[(t * CPV + c) * NV + v] = ldg16(a.x + (int64_t)t * a.H + w8 * 8);
  }
}

template <int LXC>
struct GuBuf {
  uint4 g[LXC], u[LXC];
  uint32_t gs[LXC], us[LXC];   // MXFP4: e8m0 byte; NVFP4: two E4M3 bytes
  float gg, ug;                // NVFP4: the matrices' fp32 scales
};

// row i of the gate and up matrices of the expert at base, this lane's vectors
template <int WT, int LXC>
__device__ __forceinline__ void gu_load(const DecArgs& a, const uint8_t* base, int i, int lane,
                                        GuBuf<LXC>& b) {
  constexpr int EPV = WT == 1 ? 8 : 32;
  const int nvh = a.H / EPV;
#pragma unroll
  for (int l = 0; l < LXC; ++l) {
    const int v = lane + 64 * l;
    b.g[l] = b.u[l] = make_uint4(0, 0, 0, 0);
    b.gs[l] = b.us[l] = 0;
    if (l < a.lx && v < nvh) {
      if (WT == 1) {
        b.g[l] = ldg16(base + a.off[0] + ((int64_t)i * a.H + (int64_t)v * 8) * 2);
        b.u[l] = ldg16(base + a.off[1] + ((int64_t)i * a.H + (int64_t)v * 8) * 2);
      } else if (WT == 2) {
        b.g[l] = ldg16(base + a.off[0] + (int64_t)i * (a.H / 2) + (int64_t)v * 16);
        b.u[l] = ldg16(base + a.off[2] + (int64_t)i * (a.H / 2) + (int64_t)v * 16);
        b.gs[l] = (base + a.off[1])[(int64_t)i * (a.H / 32) + v];
        b.us[l] = (base + a.off[3])[(int64_t)i * (a.H / 32) + v];
      } else {
        b.g[l] = ldg16(base + a.off[0] + (int64_t)i * (a.H / 2) + (int64_t)v * 16);
        b.u[l] = ldg16(base + a.off[2] + (int64_t)i * (a.H / 2) + (int64_t)v * 16);
        b.gs[l] = *reinterpret_cast<const uint16_t*>(base + a.off[1] +
                                                     (int64_t)i * (a.H / 16) + 2 * v);
        b.us[l] = *reinterpret_cast<const uint16_t*>(base + a.off[3] +
                                                     (int64_t)i * (a.H / 16) + 2 * v);
      }
    }
  }
  if (WT == 3) {
    b.gg = *reinterpret_cast<const float*>(base + a.goff);
    b.ug = *reinterpret_cast<const float*>(base + a.goff + 4);
  }
}

// h = silu(g . x_t) * (u . x_t) for entry q of the row's expert (token t);
// the result is the same in every lane
template <int WT, int LXC>
__device__ __forceinline__ float gu_dot(const DecArgs& a, const DecLds& S, const GuBuf<LXC>& b,
                                        int t, int lane) {
  constexpr int EPV = WT == 1 ? 8 : 32;
  constexpr int CPV = EPV / 8;
  const int nvh = a.H / EPV;
  float gp = 0.f, up = 0.f;
#pragma unroll
  for (int l = 0; l < LXC; ++l) {
    const int v = lane + 64 * l;
    if (l >= a.lx || v >= nvh) continue;
    if (WT == 1) {
      const uint4 xx = S.g.xs[t * nvh + v];
      gp = dot2_bf16(b.g[l].x, xx.x, gp);
      gp = dot2_bf16(b.g[l].y, xx.y, gp);
      gp = dot2_bf16(b.g[l].z, xx.z, gp);
      gp = dot2_bf16(b.g[l].w, xx.w, gp);
      up = dot2_bf16(b.u[l].x, xx.x, up);
      up = dot2_bf16(b.u[l].y, xx.y, up);
      up = dot2_bf16(b.u[l].z, xx.z, up);
      up = dot2_bf16(b.u[l].w, xx.w, up);
    } else {
      uint32_t xp[16];
#pragma unroll
      for (int c = 0; c < CPV; ++c) {
        const uint4 t4 = S.g.xs[(t * CPV + c) * nvh + v];
        xp[4 * c] = t4.x; xp[4 * c + 1] = t4.y; xp[4 * c + 2] = t4.z; xp[4 * c + 3] = t4.w;
      }
      if (WT == 2) {
        gp = fmaf(dot_fp4_bf16_block(b.g[l], xp), e8m0_to_f32(b.gs[l]), gp);
        up = fmaf(dot_fp4_bf16_block(b.u[l], xp), e8m0_to_f32(b.us[l]), up);
      } else {
        float s0, s1;
        dot_fp4_bf16_halves(b.g[l], xp, s0, s1);
        gp = fmaf(s0, e4m3_to_f32(b.gs[l] & 0xffu), fmaf(s1, e4m3_to_f32(b.gs[l] >> 8), gp));
        dot_fp4_bf16_halves(b.u[l], xp, s0, s1);
        up = fmaf(s0, e4m3_to_f32(b.us[l] & 0xffu), fmaf(s1, e4m3_to_f32(b.us[l] >> 8), up));
      }
    }
  }
  float gsum = wave_sum_dpp(gp);
  float usum = wave_sum_dpp(up);
  if (WT == 3) {
    gsum *= b.gg;
    usum *= b.ug;
  }
  return gsum / (1.0f + expf(-gsum)) * usum;
}

// h results of a wave to memory, each tagged with the launch's generation
// (an index past h is dropped)
__device__ __forceinline__ void flush_h(const DecArgs& a, WaveOut& o) {
  const int lane = threadIdx.x & 63;
  const int n = (a.T * a.k + a.T) * a.I;
  for (int q = lane; q < o.n; q += 64) {
    const int2 p = o.buf[q];
    if ((unsigned)p.x < (unsigned)n)
      __hip_atomic_store(a.h + p.x, ((uint64_t)a.gen << 32) | (uint32_t)p.y, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  o.n = 0;
}

// Rows [q0, q1) of a flattened (unit, row of I) list; wave w takes rows
// q0 + w, q0 + w + kW, ... with RG rows of loads in flight; after() runs once
// the first rows' loads are issued (every wave calls it).  h results gather in
// a per-wave list in the h stage of LDS.  SHARED: the list is the shared
// expert's I rows and its entries are all T tokens (known before routing).
template <int WT, int LXC, int RG, bool SHARED, class After>
__device__ __forceinline__ void gateup_range(const DecArgs& a, DecLds& S, int64_t q0, int64_t q1,
                             After&& after) {
  const int lane = threadIdx.x & 63, wave = uni((int)(threadIdx.x >> 6));
  const int I = a.I;
  const int64_t first = q0 + wave;
  const int nq = first < q1 ? (int)((q1 - first + kW - 1) / kW) : 0;
  // (unit, row) cursors of the row computed next and of the row loaded next;
  // both step by kW rows, so only the first position takes a division
  int cu = -1, ci = 0;
  if (nq > 0) {
    if (SHARED) {
      ci = (int)first;
    } else {
      cu = (int)(first / I);
      ci = (int)(first - (int64_t)cu * I);
    }
  }
  auto step = [&](int& u, int& i) {
    i += kW;
    if (!SHARED)
      while (i >= I) {
        i -= I;
        ++u;
      }
  };
  int lu = cu, li = ci;
  auto load = [&](GuBuf<LXC>& b) {
    gu_load<WT, LXC>(a, SHARED ? a.shared : unit_base(a, S.p.unit_slot[lu]), li, lane, b);
  };
  WaveOut out;
  out.cap = kHStage4 / kW * 2;
  out.buf = reinterpret_cast<int2*>(S.g.hs) + wave * out.cap;
  out.n = 0;
  GuBuf<LXC> buf[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r)
    if (r < nq) {
      load(buf[r]);
      step(lu, li);
    }
  after();                                 // more loads, behind the first rows
  for (int m0 = 0; m0 < nq; m0 += RG) {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int m = m0 + r;
      if (m < nq) {
        const int e0 = SHARED ? 0 : S.p.unit_start[cu];
        const int ne = SHARED ? a.T : S.p.unit_start[cu + 1] - e0;
        float mine = 0.f;        // lane q keeps entry q's h
        for (int q = 0; q < ne; ++q) {
          const int t = SHARED ? q : S.p.ent_tok[e0 + q];
          const float hv = gu_dot<WT, LXC>(a, S, buf[r], t, lane);
          if (lane == q) mine = hv;
        }
        if (m + RG < nq) {
          load(buf[r]);
          step(lu, li);
        }
        if (out.n + ne > out.cap) flush_h(a, out);
        if (lane < ne) {
          const int pair = SHARED ? a.T * a.k + lane : S.p.ent_pair[e0 + lane];
          out.buf[out.n + lane] = make_int2(pair * I + ci, __float_as_int(mine));
        }
        out.n += ne;
        step(cu, ci);
      }
    }
  }
  flush_h(a, out);
}

// ---------------------------------------------------------------------------
// down rows
// ---------------------------------------------------------------------------
// The work is the rows of H of every virtual unit (a unit's entries in chunks
// of at most CE), flattened unit-major and split evenly over the grid.  A
// workgroup walks its share in passes: a pass stages h of the entries it needs
// into LDS once and gathers its y results in per-wave lists, written out at
// the pass end.  Within a pass the rows go segment by segment (a segment: the
// pass's rows of one virtual unit) in steps of kW * rpw rows, each wave taking
// rpw rows per step with lr lanes per row and nv vectors per lane (lane j of a
// row group holds vectors j, j + lr, ...), so a lane needs the same h values
// for every row of a segment and keeps them in registers.  The loads of the
// next DD steps stay in flight across segment boundaries.
template <int NVC>
struct DnBuf {
  uint4 q[NVC];
  uint32_t s[NVC];   // MXFP4: the aligned word holding the scale byte
};

struct DnLane {
  int rpw;       // rows per wave per step (64 / lr)
  int grp, j;    // this lane's row group and its lane in the group
  int sh;        // log2 of the rows per step (kW * rpw)
};


// Cursor over the segments of a pass that ends at row p1 (rows of the
// flattened virtual-unit list, which stays below 2^31); every field is the
// same in all lanes.  A segment's weights base and its entries' tokens and
// gate weights are read once, when the cursor enters it.
template <int CE>
struct DnCur {
  int lo, hi;          // rows of the segment
  int v;               // its virtual unit
  int s, ns;           // the step in it, its steps
  int e0, n;           // its entries
  int tokH[CE];        // token * H of each entry
  float gw[CE];        // gate weight of each entry (NVFP4: times the down scale)
  const uint8_t* base; // the unit's weights
};

template <int CE>
__device__ __forceinline__ void dn_enter(const DecArgs& a, const DecLds& S, const DnLane& L,
                                         int v, int lo, int p1, DnCur<CE>& c) {
  c.v = uni(v);
  c.lo = uni(lo);
  const int e = (c.v + 1) * a.H;
  c.hi = uni(e < p1 ? e : p1);
  c.s = 0;
  c.ns = uni((c.hi - c.lo + (1 << L.sh) - 1) >> L.sh);
  c.e0 = uni(S.p.vu_e0[v]);
  c.n = uni(S.p.vu_n[v]);
#pragma unroll
  for (int i = 0; i < CE; ++i) {
    const int en = c.e0 + (i < c.n ? i : 0);
    c.tokH[i] = uni(S.p.ent_tok[en]) * a.H;
    c.gw[i] = uni(S.p.ent_gw[en]);
  }
  c.base = unit_base(a, uni(S.p.unit_slot[uni(S.p.vu_unit[v])]));
  if (a.goff > 0) {                          // NVFP4: fold the down matrix's scale in
    const float gd = *reinterpret_cast<const float*>(c.base + a.goff + 8);
#pragma unroll
    for (int i = 0; i < CE; ++i) c.gw[i] *= gd;
  }
}

// the segment holding row d (any row of the pass)
template <int CE>
__device__ __forceinline__ void dn_seg(const DecArgs& a, const DecLds& S, const DnLane& L, int d,
                                       int p1, DnCur<CE>& c) {
  dn_enter(a, S, L, d / a.H, d, p1, c);
}

// past the pass's last step the cursor stays on its last segment
template <int CE>
__device__ __forceinline__ void dn_next(const DecArgs& a, const DecLds& S, const DnLane& L, int p1,
                                        DnCur<CE>& c) {
  c.s = uni(c.s + 1);
  if (c.s >= c.ns && c.hi < p1) dn_enter(a, S, L, c.v + 1, c.hi, p1, c);
}

template <int CE>
__device__ __forceinline__ int dn_row(const DnLane& L, const DnCur<CE>& c, int wave) {
  return c.lo + (c.s << L.sh) + wave * L.rpw + L.grp;
}

// End of the pass that starts at row p0 of a share ending at d1: as many
// segments as the h stage and the y lists hold (the last one may be cut at a
// step); *steps = the pass's steps.  The first step always fits (kMaxCE
// entries of I values fit the stage, kMaxCE * rpw results a list).
__device__ __forceinline__ int pass_end(const DecArgs& a, const DecLds& S, int p0, int d1, const DnLane& L,
                        int* steps) {
  const int E0 = uni(S.p.vu_e0[p0 / a.H]);
  const int hcap = kDnH4 * 4 / a.I;
  int slots = 0, total = 0;
  int d = p0;
  while (d < d1) {
    const int v = d / a.H;
    const int e = (v + 1) * a.H;
    const int hi = e < d1 ? e : d1;
    const int n = uni(S.p.vu_n[v]);
    if (uni(S.p.vu_e0[v]) + n - E0 > hcap) break;
    const int ns = (hi - d + (1 << L.sh) - 1) >> L.sh;
    const int per = n * L.rpw;
    if (slots + ns * per > kYOut) {
      const int k = (kYOut - slots) / per;
      d += k << L.sh;
      total += k;
      break;
    }
    slots += ns * per;
    total += ns;
    d = hi;
  }
  *steps = uni(total);
  return uni(d);
}

// Always NVC loads (rows past the segment read its first row, vectors past nv
// read vector j; neither is used), so that every step issues the same loads
// and the waits for a step's data can be counted exactly.  MXFP4 scales come
// as the aligned 32-bit word that holds the byte (within the expert block:
// the scale array starts and ends on a 32-byte boundary of a 256-byte aligned
// expert block).
template <int WT, int NVC, int CE>
__device__ __forceinline__ void dn_load(const DecArgs& a, const DnLane& L, const DnCur<CE>& c,
                                        int wave, DnBuf<NVC>& b) {
  const int row = dn_row(L, c, wave);
  const int r = (row < c.hi ? row : c.lo) - c.v * a.H;
#pragma unroll
  for (int n = 0; n < NVC; ++n) {
    const int v = L.j + (n < a.nv ? a.lr * n : 0);
    if (WT == 1) {
      b.q[n] = ldg16(c.base + a.off[2] + ((int64_t)r * a.I + (int64_t)v * 8) * 2);
    } else {
      b.q[n] = ldg16(c.base + a.off[4] + (int64_t)r * (a.I / 2) + (int64_t)v * 16);
      const int so = WT == 2 ? r * (a.I / 32) + v : r * (a.I / 16) + 2 * v;
      b.s[n] = *reinterpret_cast<const uint32_t*>(c.base + a.off[5] + (so & ~3));
    }
  }
}

// the scale byte (MXFP4) or the two scale bytes (NVFP4) of vector v of row r
// within its loaded word
template <int WT>
__device__ __forceinline__ uint32_t dn_scale(const DecArgs& a, int r, int v, uint32_t word) {
  if (WT == 2) return (word >> (((r * (a.I / 32) + v) & 3) * 8)) & 0xffu;
  return (word >> (((r * (a.I / 16) + 2 * v) & 3) * 8)) & 0xffffu;
}

// y results of a wave to memory (fp32 atomics; index -1: none; an index past
// y is dropped rather than written)
__device__ __forceinline__ void flush_y(const DecArgs& a, WaveOut& o) {
  const int lane = threadIdx.x & 63;
  const int n = a.T * a.H;
  for (int q = lane; q < o.n; q += 64) {
    const int2 p = o.buf[q];
    if (p.x >= 0 && p.x < n) unsafeAtomicAdd(a.y + p.x, __int_as_float(p.y));
  }
  o.n = 0;
}

// dot of one 16-byte weight vector with its EPV h values (EPV / 4 float4s)
template <int WT>
__device__ __forceinline__ float wdot_h(const uint4 q, uint32_t sc, const float4* h4) {
  if (WT == 1) {
    // h as BF16 hi parts (h4[0]) and lo parts (h4[1]): exact products, fp32 sums
    const float4 hf = h4[0], lf = h4[1];
    float s = dot2_bf16(q.x, __float_as_uint(hf.x), 0.f);
    s = dot2_bf16(q.y, __float_as_uint(hf.y), s);
    s = dot2_bf16(q.z, __float_as_uint(hf.z), s);
    s = dot2_bf16(q.w, __float_as_uint(hf.w), s);
    s = dot2_bf16(q.x, __float_as_uint(lf.x), s);
    s = dot2_bf16(q.y, __float_as_uint(lf.y), s);
    s = dot2_bf16(q.z, __float_as_uint(lf.z), s);
    return dot2_bf16(q.w, __float_as_uint(lf.w), s);
  } else {
    // MXFP4: one sum times the e8m0 scale; NVFP4: the two 16-element halves
    // (words 0-1, 2-3) each times its E4M3 scale
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hx = WT == 2 ? 0 : i >> 1;
      const float4 ha = h4[2 * i], hc = h4[2 * i + 1];
      const v2f c0 = fp4x2_to_f32x2<0>(w[i]);
      const v2f c1 = fp4x2_to_f32x2<1>(w[i]);
      const v2f c2 = fp4x2_to_f32x2<2>(w[i]);
      const v2f c3 = fp4x2_to_f32x2<3>(w[i]);
      float a = acc[hx];
      a = fmaf(c0.x, ha.x, a);
      a = fmaf(c0.y, ha.y, a);
      a = fmaf(c1.x, ha.z, a);
      a = fmaf(c1.y, ha.w, a);
      a = fmaf(c2.x, hc.x, a);
      a = fmaf(c2.y, hc.y, a);
      a = fmaf(c3.x, hc.z, a);
      a = fmaf(c3.y, hc.w, a);
      acc[hx] = a;
    }
    if (WT == 2) return acc[0] * e8m0_to_f32(sc);
    return fmaf(acc[0], e4m3_to_f32(sc & 0xffu), acc[1] * e4m3_to_f32(sc >> 8));
  }
}

// h values of a segment's entries kept in registers per lane: EPV floats per
// down vector and entry, as long as that stays within 32 floats per entry
// (else they are read from the stage per row)
template <int WT, int NVC, int CE>
struct HRegs {
  static constexpr int EPV = WT == 1 ? 8 : 32;
  static constexpr bool kOn = NVC * EPV <= 32;
  float4 v[kOn ? CE : 1][kOn ? NVC : 1][EPV / 4];
};

// this lane's h values of staged entries [er, er + n)
template <int WT, int NVC, int CE>
__device__ __forceinline__ void h_regs(const DecArgs& a, const DecLds& S, int j, int er, int n,
                                       HRegs<WT, NVC, CE>& hv) {
  constexpr int EPV = WT == 1 ? 8 : 32;
  if constexpr (HRegs<WT, NVC, CE>::kOn) {
    const int V = a.I / EPV, I4 = a.I / 4;
#pragma unroll
    for (int i = 0; i < CE; ++i) {
      if (i >= n) break;
#pragma unroll
      for (int nn = 0; nn < NVC; ++nn) {
        if (nn >= a.nv) break;
#pragma unroll
        for (int c = 0; c < EPV / 4; ++c)
          hv.v[i][nn][c] = S.d.hst[(er + i) * I4 + c * V + j + a.lr * nn];
      }
    }
  }
}

// the lane's row of the cursor's step . h of each entry of the segment
// (staged entries from er), each result times the entry's gate weight listed
// for y[token][row]; rows past the segment list index -1
template <int WT, int NVC, int CE>
__device__ __forceinline__ void dn_compute(const DecArgs& a, const DecLds& S, const DnLane& L,
                                           const DnCur<CE>& c, int wave, int er,
                                           const DnBuf<NVC>& b, const HRegs<WT, NVC, CE>& hv,
                                           WaveOut& out) {
  constexpr int EPV = WT == 1 ? 8 : 32;
  const int row = dn_row(L, c, wave);
  const bool valid = row < c.hi;
  const int r = (valid ? row : c.lo) - c.v * a.H;
  const int V = a.I / EPV;
  uint32_t sc[NVC];
#pragma unroll
  for (int nn = 0; nn < NVC; ++nn)
    sc[nn] = WT == 1 ? 0u : dn_scale<WT>(a, r, L.j + (nn < a.nv ? a.lr * nn : 0), b.s[nn]);
#pragma unroll
  for (int i = 0; i < CE; ++i) {
    if (i >= c.n) break;
    float s = 0.f;
    if constexpr (HRegs<WT, NVC, CE>::kOn) {
#pragma unroll
      for (int nn = 0; nn < NVC; ++nn) {
        if (nn >= a.nv) break;
        s += wdot_h<WT>(b.q[nn], sc[nn], hv.v[i][nn]);
      }
    } else {
      const float4* hs = S.d.hst + (er + i) * (a.I / 4);
#pragma unroll
      for (int nn = 0; nn < NVC; ++nn) {
        if (nn >= a.nv) break;
        float4 h4[EPV / 4];
#pragma unroll
        for (int q = 0; q < EPV / 4; ++q) h4[q] = hs[q * V + L.j + a.lr * nn];
        s += wdot_h<WT>(b.q[nn], sc[nn], h4);
      }
    }
    s = group_sum(s, a.lr);
    if (L.j == 0)
      out.buf[out.n + L.grp] = make_int2(valid ? c.tokH[i] + r : -1, __float_as_int(c.gw[i] * s));
    out.n += L.rpw;
  }
}

// stage h of entries [c0, c1) into LDS (transposed layout): each value is
// polled until it carries this launch's generation; a thread loads the four
// values of up to four float4s before it checks any of them
template <int WT>
__device__ __forceinline__ void stage_h(const DecArgs& a, DecLds& S, int c0, int c1) {
  constexpr int EPV = WT == 1 ? 8 : 32;
  constexpr int B = 4;
  const int I4 = a.I / 4, V = a.I / EPV;
  const int n4 = (c1 - c0) * I4;
  for (int q0 = threadIdx.x; q0 < n4; q0 += B * kT) {
    uint64_t w[B][4];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = q0 + b * kT;
      if (q < n4) {
        const int e = q / I4, c4 = q - e * I4;
        const uint64_t* src = a.h + (int64_t)S.p.ent_pair[c0 + e] * a.I + c4 * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[b][j] = __hip_atomic_load(src + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = q0 + b * kT;
      if (q < n4) {
        const int e = q / I4, c4 = q - e * I4;
        const uint64_t* src = a.h + (int64_t)S.p.ent_pair[c0 + e] * a.I + c4 * 4;
        unsigned spins = 0;
        for (;;) {
          bool all = true;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if ((unsigned)(w[b][j] >> 32) != a.gen) {
              all = false;
              w[b][j] = __hip_atomic_load(src + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          if (all) break;
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kSpinLimit) {
            __hip_atomic_store(a.hdr + kHError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        const int v = c4 / (EPV / 4), cc = c4 - v * (EPV / 4);
        const float h0 = __uint_as_float((uint32_t)w[b][0]), h1 = __uint_as_float((uint32_t)w[b][1]);
        const float h2 = __uint_as_float((uint32_t)w[b][2]), h3 = __uint_as_float((uint32_t)w[b][3]);
        if (WT == 1) {
          // BF16 weights: the vector's 8 h values as BF16 hi parts (first
          // float4) and lo parts (second), so a row takes two dot2 per pair
          uint32_t hi0, lo0, hi1, lo1;
          bf16_split2(h0, h1, hi0, lo0);
          bf16_split2(h2, h3, hi1, lo1);
          uint2* dst = reinterpret_cast<uint2*>(S.d.hst + e * I4 + v);
          dst[cc] = make_uint2(hi0, hi1);
          reinterpret_cast<uint2*>(S.d.hst + e * I4 + V + v)[cc] = make_uint2(lo0, lo1);
        } else {
          S.d.hst[e * I4 + cc * V + v] = make_float4(h0, h1, h2, h3);
        }
      }
    }
  }
}

// Exit of a launch: workgroups are counted per group (b % kNCtr), then the
// groups; the last workgroup out clears the counts and advances the
// generation, so the next launch on this workspace starts from zero.
__device__ __forceinline__ void finish_launch(const DecArgs& a, unsigned gen) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int bid = blockIdx.x, G = a.G;
    const int grp = bid % kNCtr;
    const unsigned gsize = (unsigned)((G - grp + kNCtr - 1) / kNCtr);
    const unsigned ngrp = (unsigned)(G < kNCtr ? G : kNCtr);
    const unsigned old = __hip_atomic_fetch_add(a.hdr + kHExit + grp * kLine, 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gsize - 1 &&
        __hip_atomic_fetch_add(a.hdr + kHExitTop, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == ngrp - 1) {
      for (int j = 0; j < kNCtr; ++j) {
        __hip_atomic_store(a.hdr + kHYZero + j * kLine, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.hdr + kHExit + j * kLine, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(a.hdr + kHExitTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.hdr + kHGen, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.hdr[kHTiming])
        reinterpret_cast<unsigned long long*>(a.hdr + kHStamps)[4] = wall_clock64();
    }
  }
}

// ---------------------------------------------------------------------------
// the kernel.  WT: 1 BF16, 2 MXFP4.  LXC, NVC: register capacity (vectors per
// lane) of a gate/up row and of a down row.  M: logits per lane in the wave
// top-k (E <= 64 M).  RG gate/up rows and DD steps of
// down rows are loaded ahead.
// ---------------------------------------------------------------------------
template <int WT, int LXC, int NVC, int M>
__global__ __launch_bounds__(kT) void decode_kernel(DecArgs a) {
  constexpr int RGV = WT == 1 ? 32 : 16;   // gate/up vectors in flight per lane
  constexpr int RG = RGV / (2 * LXC) > 0 ? RGV / (2 * LXC) : 1;
  constexpr int DDV = WT == 1 ? 16 : (LXC >= 4 ? 4 : 8);  // down vectors in flight per lane
  constexpr int DD = NVC >= DDV ? 1 : DDV / NVC;
  constexpr int CE = kMaxCE;               // entries per down virtual unit
  __shared__ DecLds S;
  const int lane = threadIdx.x & 63, wave = uni((int)(threadIdx.x >> 6));
  const int bid = blockIdx.x, G = a.G;
  const bool route = a.route != 0;
  const bool timing = a.hdr[kHTiming] != 0;     // uniform: a scalar load
  const unsigned gen =
      __hip_atomic_load(a.hdr + kHGen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  a.gen = gen;
  stamp(timing, a, 0);

  // 1. router dot products (every workgroup), with x staged into LDS while
  // the first row loads are in flight; clear y; the shared expert's gate/up
  // rows
  RouterRow rw;
  const int item0 = bid + G * wave;
  if (route && item0 < router_items(a)) router_load(a, item0, 0, rw);
  stage_x<WT>(a, S);
  __syncthreads();
  if (route) {
    router_items_run<WT>(a, S, item0, rw, uni((int)gen));
    stamp(timing, a, 5);
  }
  {
    int64_t lo, hi;
    split((int64_t)a.T * a.H, G, bid, lo, hi);
    for (int64_t i = lo + threadIdx.x; i < hi; i += kT) coherent_store(a.y + i, 0.f);
  }
  if (a.shared) {
    int64_t lo, hi;
    split(a.I, G, bid, lo, hi);
    gateup_range<WT, LXC, RG, true>(a, S, lo, hi, [] {});
  }
  // the slice of y is clear (counted once its stores are done; checked
  // before the first y result is added)
  signal_done(a.hdr + kHYZero);
  stamp(timing, a, 8);

  // 2. the expert list
  build_units<M, CE, WT != 1>(a, S, route, timing, gen, reinterpret_cast<float*>(S.g.hs));
  stamp(timing, a, 1);
  const int n_routed = S.p.n_routed;

  // 3. routed gate/up rows
  DnLane L;
  L.rpw = 64 / a.lr;
  L.grp = lane / a.lr;
  L.j = lane - L.grp * a.lr;
  L.sh = 31 - __builtin_clz(kW * L.rpw);
  int d0, d1;
  {
    int64_t lo, hi;
    split((int64_t)S.p.n_vu * a.H, G, bid, lo, hi);
    d0 = uni((int)lo);
    d1 = uni((int)hi);
  }
  int p_steps = 0;
  int p1 = d0 < d1 ? pass_end(a, S, d0, d1, L, &p_steps) : d0;
  DnCur<CE> lc;                            // load cursor of the down rows
  if (d0 < d1) dn_seg(a, S, L, d0, p1, lc);
  DnBuf<NVC> ring[DD];
  {
    int64_t lo, hi;
    split((int64_t)n_routed * a.I, G, bid, lo, hi);
    gateup_range<WT, LXC, RG, false>(a, S, lo, hi, [] {});
  }

  // 4. issue the loads of the first down steps; h is polled per value when
  // staged (no grid-wide wait)
  stamp(timing, a, 7);
  if (d0 < d1) {
#pragma unroll
    for (int d = 0; d < DD; ++d) {
      dn_load<WT, NVC, CE>(a, L, lc, wave, ring[d]);
      dn_next(a, S, L, p1, lc);
    }
  }
  // the y-cleared count, read now and checked before the first y add
  const unsigned yz = lane < kNCtr ? __hip_atomic_load(a.hdr + kHYZero + lane * kLine,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0u;
  bool y_clear = false;
  stamp(timing, a, 2);

  // 5. down rows, pass by pass
  WaveOut out;                             // y results
  out.cap = kYOut;
  out.buf = S.d.yout + wave * kYOut;
  out.n = 0;
  bool first = true;                       // the ring holds the pass's first steps
  for (int p0 = d0; p0 < d1; p0 = p1) {
    if (!first) {
      p1 = pass_end(a, S, p0, d1, L, &p_steps);
      dn_seg(a, S, L, p0, p1, lc);
    }
    const int vl = (p1 - 1) / a.H;
    const int E0 = uni(S.p.vu_e0[p0 / a.H]), E1 = uni(S.p.vu_e0[vl]) + uni(S.p.vu_n[vl]);
    __syncthreads();
    stage_h<WT>(a, S, E0, E1);
    if (!first) {
#pragma unroll
      for (int d = 0; d < DD; ++d) {
        dn_load<WT, NVC, CE>(a, L, lc, wave, ring[d]);
        dn_next(a, S, L, p1, lc);
      }
    }
    first = false;
    __syncthreads();
    stamp(timing, a, 11);
    DnCur<CE> cc;                          // compute cursor
    dn_seg(a, S, L, p0, p1, cc);
    HRegs<WT, NVC, CE> hv;
    for (int s0 = 0; s0 < p_steps; s0 += DD) {
#pragma unroll
      for (int d = 0; d < DD; ++d) {
        if (s0 + d < p_steps) {
          if (cc.s == 0) h_regs<WT, NVC, CE>(a, S, L.j, cc.e0 - E0, cc.n, hv);
          dn_compute<WT, NVC, CE>(a, S, L, cc, wave, cc.e0 - E0, ring[d], hv, out);
          dn_next(a, S, L, p1, cc);
        }
        dn_load<WT, NVC, CE>(a, L, lc, wave, ring[d]);
        dn_next(a, S, L, p1, lc);
      }
    }
    if (!y_clear) {
      if (__builtin_amdgcn_readfirstlane((unsigned)wave_sum_dpp((float)yz)) < (unsigned)G)
        wait_count(a.hdr, a.hdr + kHYZero, (unsigned)G);
      y_clear = true;
    }
    flush_y(a, out);
    stamp(timing, a, 12);
  }

  // exit: counted per group of workgroups (b % kNCtr), then per group; the
  // last workgroup out clears the counts and advances the generation
  stamp(timing, a, 3);
  finish_launch(a, gen);
}

// capacities compiled per weight format
inline int lx_cap(int lx) { return lx <= 1 ? 1 : lx <= 2 ? 2 : lx <= 4 ? 4 : lx <= 8 ? 8 : -1; }
inline int nv_cap(int nv) { return nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : -1; }

// largest I a down pass takes (kMaxCE entries of I values fit its h stage)
constexpr int kMaxI = 6144;
static_assert(kMaxCE * kMaxI <= 4 * kDnH4, "a down pass must hold kMaxCE entries");

// tokens one launch can take: x of all of them must fit the LDS stage
inline int max_tokens(int H) {
  const int t = kXStage16 * 8 / H;
  return t < kMaxT ? t : kMaxT;
}

// Down row mapping of I / EPV vectors per row: lr = the largest power of two
// <= 64 dividing it, nv = vectors per lane.  False when nv exceeds 8.
inline bool down_map(int nvec, int* lr, int* nv) {
  if (nvec <= 0) return false;
  int l = 64;
  while (nvec % l) l >>= 1;
  *lr = l;
  *nv = nvec / l;
  return *nv <= 8;
}

// ---------------------------------------------------------------------------
// standalone router (moe_route, T <= 64): one wave per row, last workgroup ranks
// ---------------------------------------------------------------------------
constexpr int kRT = 256;            // threads per router workgroup
constexpr int kRW = kRT / 64;

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
__global__ __launch_bounds__(kRT) void route_kernel(RouteArgs a) {
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * kRW + wave;
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
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int t = wave; t < T; t += kRW)
    topk_one_token<M>(a.z + (int64_t)t * E, E, a.k, a.renorm, a.ids + (int64_t)t * a.k,
                      a.w + (int64_t)t * a.k);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool RF32, int L, int M>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((route_kernel<RF32, L, M>), dim3((a.E + kRW - 1) / kRW), dim3(kRT), 0, st, a);
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

}  // namespace dec
}  // namespace moe

#include "decode_mfma.hpp"

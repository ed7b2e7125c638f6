// route.hip - router logits, softmax and wavefront top-k.
//
// Each token in each MoE layer is sent to a few of many experts ("FreeToken
// 753b Model Explained", section of the same name: six of 256 per layer for
// the DeepSeek-V4-Flash shape).  The pages do not give the gate; this is
// softmax over all experts, then the k largest probabilities in descending
// order, ties to the lower expert id.  Ranking is done on the fp32 logits
// (same order as the probabilities, no exp ties).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// ---- small T: one wave per expert row, tokens looped ------------------------
// grid.x = ceil(E / 4); each wave keeps its router row in registers and forms
// z[t][e] for every token.  RF32: router weights in fp32 (else bf16).
template <bool RF32, int L>
__global__ __launch_bounds__(256) void logits_rows_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ wr, int T, int H,
    int E, float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  constexpr int EPV = RF32 ? 4 : 8;  // elements per 16-byte vector
  const int nvec = H / EPV;
  uint4 wv[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int v = lane + 64 * i;
    wv[i] = make_uint4(0, 0, 0, 0);
    if (v < nvec) {
      const uint8_t* row = static_cast<const uint8_t*>(wr) + (int64_t)e * H * (RF32 ? 4 : 2);
      wv[i] = ldg16(row + (int64_t)v * 16);
    }
  }
  for (int t = 0; t < T; ++t) {
    const uint16_t* xt = x + (int64_t)t * H;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int v = lane + 64 * i;
      if (v >= nvec) continue;
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
    acc = wave_sum(acc);
    if (lane == 0) z[(int64_t)t * E + e] = acc;
  }
}

// ---- large T: 64 tokens x 64 experts per workgroup, LDS-tiled fp32 FMA ----
// Products of bf16 (or bf16 x fp32) values accumulated in fp32.
template <bool RF32>
__global__ __launch_bounds__(256) void logits_tiled_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ wr, int T, int H,
    int E, float* __restrict__ z) {
  constexpr int TM = 64, TN = 64, TK = 32;
  __shared__ float sx[TK][TM + 1];
  __shared__ float sw[TK][TN + 1];
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TN;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 16 x 16 threads
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += TK) {
    // 64 x 32 tile of x and of W_r: 2048 elements each, 8 per thread
    for (int i = threadIdx.x; i < TM * TK; i += 256) {
      const int r = i / TK, c = i % TK;
      const int t = t0 + r, e = e0 + r;
      sx[c][r] = (t < T) ? __uint_as_float((uint32_t)x[(int64_t)t * H + k0 + c] << 16) : 0.f;
      float wval = 0.f;
      if (e < E) {
        if (RF32) wval = static_cast<const float*>(wr)[(int64_t)e * H + k0 + c];
        else wval = __uint_as_float((uint32_t) static_cast<const uint16_t*>(wr)[(int64_t)e * H + k0 + c] << 16);
      }
      sw[c][r] = wval;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < TK; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sx[c][ty * 4 + i]; b[i] = sw[c][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + ty * 4 + i, e = e0 + tx * 4 + j;
      if (t < T && e < E) z[(int64_t)t * E + e] = acc[i][j];
    }
}

// ---- softmax + top-k: one wave per token ------------------------------------
// Each lane holds up to 16 logits (E <= 1024).  k rounds of a wave arg-max
// (largest logit, lower id on ties) pick the experts in descending order.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int T,
                                                   int E, int k, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zt = z + (int64_t)t * E;
  constexpr int M = 16;
  float v[M];
  float live[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? zt[e] : -INFINITY;
    live[i] = v[i];
  }
  // max logit and softmax denominator
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < M; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int e = lane + 64 * i;
    if (e < E) s += expf(v[i] - m);
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  float wsum = 0.f;
  float my_w = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    // local best: largest value, lowest id
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (live[i] > bv || (live[i] == bv && e < bi))) { bv = live[i]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    // remove the winner
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (lane + 64 * i == bi) live[i] = -INFINITY;
    const float p = expf(bv - m) * inv;
    wsum += p;
    if (lane == j) { my_w = p; my_id = bi; }
  }
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    w[(int64_t)t * k + lane] = renorm ? my_w / wsum : my_w;
  }
}

template <bool RF32>
hipError_t launch_rows(const void* x, const void* wr, int T, int H, int E, float* z,
                       hipStream_t st) {
  const int nvec = H / (RF32 ? 4 : 8);
  const int L = (nvec + 63) / 64;
  dim3 grid((E + 3) / 4);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
#define MOE_ROWS_CASE(n) \
  case n: hipLaunchKernelGGL((logits_rows_kernel<RF32, n>), grid, dim3(256), 0, st, xb, wr, T, H, E, z); break;
  switch (L) {
    MOE_ROWS_CASE(1) MOE_ROWS_CASE(2) MOE_ROWS_CASE(3) MOE_ROWS_CASE(4)
    MOE_ROWS_CASE(5) MOE_ROWS_CASE(6) MOE_ROWS_CASE(7) MOE_ROWS_CASE(8)
    MOE_ROWS_CASE(9) MOE_ROWS_CASE(10) MOE_ROWS_CASE(11) MOE_ROWS_CASE(12)
    MOE_ROWS_CASE(13) MOE_ROWS_CASE(14) MOE_ROWS_CASE(15) MOE_ROWS_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROWS_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* x, const void* w_router, int router_f32, int T,
                        int H, int E, int k, int renorm, float* logits,
                        int32_t* ids, float* w, hipStream_t st) {
  hipError_t err;
  if (T <= 64) {
    err = router_f32 ? launch_rows<true>(x, w_router, T, H, E, logits, st)
                     : launch_rows<false>(x, w_router, T, H, E, logits, st);
  } else {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (router_f32)
      hipLaunchKernelGGL((logits_tiled_kernel<true>), grid, dim3(256), 0, st, xb, w_router, T, H, E, logits);
    else
      hipLaunchKernelGGL((logits_tiled_kernel<false>), grid, dim3(256), 0, st, xb, w_router, T, H, E, logits);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, k,
                     renorm, ids, w);
  return hipGetLastError();
}

}  // namespace moe

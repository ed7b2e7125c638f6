// device.hpp - small device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---- bf16 ----------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ v2bf as_v2bf(uint32_t w) { return __builtin_bit_cast(v2bf, w); }

// dot of two packed bf16 pairs accumulated into fp32 (products are exact)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_v2bf(a), as_v2bf(b), acc, false);
}

// Two fp32 values as BF16 parts: hi = RNE(v), lo = RNE(v - hi) (the
// difference is exact in fp32), packed low element first.  hi + lo is v to
// within about 2^-17 of |v|.
__device__ __forceinline__ void bf16_split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const v2bf h = {(__bf16)a, (__bf16)b};
  hi = __builtin_bit_cast(uint32_t, h);
  const v2bf l = {(__bf16)(a - bf16_lo(hi)), (__bf16)(b - bf16_hi(hi))};
  lo = __builtin_bit_cast(uint32_t, l);
}

// ---- e2m1 (MXFP4 element) decode ------------------------------------------
// Two e2m1 codes held in byte SEL of `word` -> two bf16 values (exact: every
// e2m1 value is a bf16), packed low element first.  Uses the gfx950 scaled
// FP4 convert with scale 1.0, so the values are the bare e2m1 values.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t word) {
  v2bf r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

template <int SEL>
__device__ __forceinline__ v2f fp4x2_to_f32x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// e8m0 scale byte -> 2^(s-127) as an fp32 (s = 0 is the denormal 2^-127,
// s = 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  s &= 0xffu;
  if (s == 0) return __uint_as_float(0x00400000u);
  if (s == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(s << 23);
}

// OCP E4M3FN byte -> fp32 (bias 7; exponent 0: m * 2^-9; NaN codes are never
// produced by the encoder and are not special-cased)
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -v : v;
}

// non-negative fp32 -> E4M3 code with round-to-nearest-even, saturating at
// 448 (0x7E)
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  if (!(t < 448.f)) return 0x7Eu;
  const uint32_t bits = __float_as_uint(t);
  const int ex = (int)((bits >> 23) & 0xffu) - 127;
  if (ex < -6) return (uint32_t)rintf(t * 512.f);      // subnormal steps of 2^-9
  uint32_t m3 = (bits >> 20) & 7u;
  const uint32_t rem = bits & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  const uint32_t code = ((uint32_t)(ex + 7) << 3) + m3;  // a mantissa carry bumps the exponent
  return code > 0x7Eu ? 0x7Eu : code;
}

// sums over the two 16-element halves of one 16-byte e2m1 block times 32 bf16
// x values (16 packed pairs), fp32 accumulation, no scale applied
__device__ __forceinline__ void dot_fp4_bf16_halves(const uint4 q, const uint32_t* xp, float& s0,
                                                    float& s1) {
  float a0 = 0.f, a1 = 0.f;
  a0 = dot2_bf16(fp4x2_to_bf16x2<0>(q.x), xp[0], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<1>(q.x), xp[1], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<2>(q.x), xp[2], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<3>(q.x), xp[3], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<0>(q.y), xp[4], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<1>(q.y), xp[5], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<2>(q.y), xp[6], a0);
  a0 = dot2_bf16(fp4x2_to_bf16x2<3>(q.y), xp[7], a0);
  a1 = dot2_bf16(fp4x2_to_bf16x2<0>(q.z), xp[8], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<1>(q.z), xp[9], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<2>(q.z), xp[10], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<3>(q.z), xp[11], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<0>(q.w), xp[12], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<1>(q.w), xp[13], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<2>(q.w), xp[14], a1);
  a1 = dot2_bf16(fp4x2_to_bf16x2<3>(q.w), xp[15], a1);
  s0 = a0;
  s1 = a1;
}

// sum over the 32 e2m1 values of one 16-byte block times 32 bf16 x values
// (x given as 16 packed bf16 pairs), fp32 accumulation, no scale applied.
__device__ __forceinline__ float dot_fp4_bf16_block(const uint4 q, const uint32_t* xp) {
  float acc = 0.f;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(w[i]), xp[4 * i + 0], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(w[i]), xp[4 * i + 1], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(w[i]), xp[4 * i + 2], acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(w[i]), xp[4 * i + 3], acc);
  }
  return acc;
}

// sum over the 32 e2m1 values of one block times 32 fp32 h values.
__device__ __forceinline__ float dot_fp4_f32_block(const uint4 q, const float* h) {
  float acc = 0.f;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v2f a = fp4x2_to_f32x2<0>(w[i]);
    v2f b = fp4x2_to_f32x2<1>(w[i]);
    v2f c = fp4x2_to_f32x2<2>(w[i]);
    v2f d = fp4x2_to_f32x2<3>(w[i]);
    acc = fmaf(a.x, h[8 * i + 0], acc);
    acc = fmaf(a.y, h[8 * i + 1], acc);
    acc = fmaf(b.x, h[8 * i + 2], acc);
    acc = fmaf(b.y, h[8 * i + 3], acc);
    acc = fmaf(c.x, h[8 * i + 4], acc);
    acc = fmaf(c.y, h[8 * i + 5], acc);
    acc = fmaf(d.x, h[8 * i + 6], acc);
    acc = fmaf(d.y, h[8 * i + 7], acc);
  }
  return acc;
}

// ---- e2m1 encode (round to nearest, ties to the even code, saturate) ------
// r is the element already divided by its block scale.  The magnitude code
// is the number of grid thresholds r passes; a threshold that sits exactly
// half way between two grid points counts only when the upper neighbour has
// the even code (mantissa bit 0).
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  float a = fabsf(r);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(r) >> 28) & 8u);
}

// block exponent X = floor(log2 amax) - 2, clamped to [-127, 127]; amax > 0.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  uint32_t b = __float_as_uint(amax);
  int e = (int)((b >> 23) & 0xffu);
  int fl;
  if (e == 0) {
    // denormal: value = m * 2^-149, floor(log2) = 31 - clz(m) - 149
    fl = (31 - __clz((int)(b & 0x7fffffu))) - 149;
  } else {
    fl = e - 127;
  }
  int X = fl - 2;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// v / 2^X by ldexpf, which scales by the power of two directly (no 2^-X
// multiplier is formed; for X = 127 it would be a denormal).  The quotient is
// exact wherever it can decide a code: |v / 2^X| >= 0.25 is a normal number.
__device__ __forceinline__ float mx_scale_down(float v, int X) {
  return ldexpf(v, -X);
}

// ---- wave reductions --------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// exclusive prefix sum over a 256-thread block (4 waves); returns the
// exclusive prefix of `v` and writes the block total to *total.
__device__ __forceinline__ int block256_exclusive_scan(int v, int* total, int* lds4) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == 63) lds4[wv] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int s = lds4[i];
    if (i < wv) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace moe

namespace moe {

// ---- DPP wave reductions (results identical in every lane) ----------------
// Butterflies inside each 16-lane row (quad_perm xor 1, xor 2, half-row
// mirror, row mirror), then the four row results combined through readlane.
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// inclusive prefix sum over the 64 lanes (all lanes active): shifts by 1, 2,
// 4, 8 inside each 16-lane row, then each row's total carried into the rows
// after it (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3)
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// order-preserving 32-bit key of a finite float (larger value, larger key;
// never 0) and back
__device__ __forceinline__ uint32_t fkey(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float fkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-k of one token's E logits by one wave, from the values each lane holds
// (v[i] = logit of expert lane + 64 i, -inf past E): softmax over all E
// (max-subtracted, fp32), then k rounds of a wave-wide arg-max, so the k ids
// come out in descending order of logit with ties going to the lower id.  A
// round takes the wave maximum of each lane's best 32-bit key, then among the
// lanes that hold it the lowest expert id.  Lanes 0..k-1 write ids_out /
// w_out (renormalised over the k when renorm).
template <int M>
__device__ inline void topk_select(float v[M], int E, int k, int renorm, int32_t* ids_out,
                                   float* w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t key[M];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const bool live = lane + 64 * i < E;
    key[i] = live ? fkey(v[i]) : 0u;
    m = fmaxf(m, v[i]);
  }
  m = wave_max_dpp(m);
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < M; ++i)
    if (key[i]) ps += expf(v[i] - m);
  const float inv = 1.0f / wave_sum_dpp(ps);
  float wsum = 0.f, my_w = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t lb = 0;
    int li = 0;
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (key[i] > lb) { lb = key[i]; li = i; }
    const uint32_t gm = wave_max_u32_dpp(lb);
    uint64_t win = __ballot(lb == gm);
    int id = 0x7fffffff;
    while (win) {                          // almost always a single lane
      const int l = __builtin_ctzll(win);
      const int cand = l + 64 * __builtin_amdgcn_readlane(li, l);
      id = cand < id ? cand : id;
      win &= win - 1;
    }
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (lane + 64 * i == id) key[i] = 0u;
    const float p = expf(fkey_value(gm) - m) * inv;
    wsum += p;
    if (lane == j) { my_w = p; my_id = id; }
  }
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = renorm ? my_w / wsum : my_w;
  }
}

// top-k of one token whose logits zt[0..E) are in memory (E <= 64 M)
template <int M>
__device__ inline void topk_one_token(const float* zt, int E, int k, int renorm, int32_t* ids_out,
                                      float* w_out) {
  const int lane = threadIdx.x & 63;
  float v[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? zt[e] : -INFINITY;
  }
  topk_select<M>(v, E, k, renorm, ids_out, w_out);
}

}  // namespace moe

// formats.hip - MXFP4 quantise / dequantise kernels, the exact partial-sum
// merge, and small fill kernels used by the expert cache.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// One thread per 32-element block: amax, shared exponent, 32 e2m1 codes.
// src is fp32 or bf16 [rows][K] with row stride ld (elements); output codes
// [rows][K/2], scales [rows][K/32].
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ src, int src_bf16,
                                                       int rows, int K, int64_t ld,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int nb = K / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)rows * nb) return;
  const int64_t r = gid / nb;
  const int b = (int)(gid % nb);
  float v[32];
  if (src_bf16) {
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + r * ld +
                                                    (int64_t)b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = s[i];
      v[8 * i + 0] = bf16_lo(q.x); v[8 * i + 1] = bf16_hi(q.x);
      v[8 * i + 2] = bf16_lo(q.y); v[8 * i + 3] = bf16_hi(q.y);
      v[8 * i + 4] = bf16_lo(q.z); v[8 * i + 5] = bf16_hi(q.z);
      v[8 * i + 6] = bf16_lo(q.w); v[8 * i + 7] = bf16_hi(q.w);
    }
  } else {
    const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(src) + r * ld +
                                                      (int64_t)b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = s[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t packed[4] = {0, 0, 0, 0};
  uint32_t sbyte = 0;
  if (amax > 0.f) {
    const int X = mx_block_exponent(amax);
    sbyte = (uint32_t)(X + 127);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = e2m1_code(mx_scale_down(v[i], X));
      packed[i / 8] |= c << (4 * (i % 8));
    }
  }
  *reinterpret_cast<uint4*>(codes + r * (K / 2) + (int64_t)b * 16) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[r * nb + b] = (uint8_t)sbyte;
}

// ---- NVFP4: e2m1 elements, an E4M3 scale per 16, an fp32 scale per matrix.
// The steps follow the encoder's fp32 definition: g = amax / 2688 (1 for a
// zero matrix); per block t = amax_b / (6 g) rounded to E4M3 (nearest even,
// saturating); d = E4M3(t) * g; codes = e2m1(v / d), all 0 when d = 0.
__device__ __forceinline__ float load_elem(const void* src, int src_bf16, int64_t i) {
  return src_bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(src)[i] << 16)
                  : static_cast<const float*>(src)[i];
}

__global__ void nvfp4_clear_kernel(float* slot) { *slot = 0.f; }

// matrix amax into *slot (fp32 bits compare like unsigned ints when >= 0)
__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const void* __restrict__ src,
                                                         int src_bf16, int64_t n, float* slot) {
  __shared__ float red[256];
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = fmaxf(m, fabsf(load_elem(src, src_bf16, i)));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(slot), __float_as_uint(red[0]));
}

__device__ __forceinline__ float nvfp4_global(float amax) { return amax > 0.f ? amax / 2688.f : 1.f; }

// one thread per 16-element block
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const void* __restrict__ src,
                                                          int src_bf16, int rows, int K,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          const float* __restrict__ amax_slot) {
  const int nb = K / 16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)rows * nb) return;
  const int64_t r = gid / nb;
  const int b = (int)(gid % nb);
  const float g = nvfp4_global(*amax_slot);
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = load_elem(src, src_bf16, r * K + (int64_t)b * 16 + i);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const uint32_t sbyte = e4m3_rne(amax / (6.f * g));
  const float d = e4m3_to_f32(sbyte) * g;
  uint32_t packed[2] = {0, 0};
  if (d > 0.f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) packed[i / 8] |= e2m1_code(v[i] / d) << (4 * (i % 8));
  }
  *reinterpret_cast<uint2*>(codes + r * (K / 2) + (int64_t)b * 8) = make_uint2(packed[0], packed[1]);
  scales[r * nb + b] = (uint8_t)sbyte;
}

__global__ void nvfp4_final_kernel(float* slot) { *slot = nvfp4_global(*slot); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  return ((u + 0x7fffu + ((u >> 16) & 1u)) >> 16) & 0xffffu;
}

// One thread per 8 elements: src fp32 or bf16 [rows][K] -> bf16 [rows][K].
__global__ __launch_bounds__(256) void pack_bf16_kernel(const void* __restrict__ src,
                                                        int src_bf16, int rows, int K,
                                                        uint16_t* __restrict__ dst) {
  const int n8 = K / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)rows * n8) return;
  const int64_t r = gid / n8;
  const int c8 = (int)(gid % n8);
  uint4 out;
  if (src_bf16) {
    out = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + r * K +
                                          (int64_t)c8 * 8);
  } else {
    const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(src) + r * K +
                                                      (int64_t)c8 * 8);
    const float4 a = s[0], b = s[1];
    out.x = f32_to_bf16_bits(a.x) | (f32_to_bf16_bits(a.y) << 16);
    out.y = f32_to_bf16_bits(a.z) | (f32_to_bf16_bits(a.w) << 16);
    out.z = f32_to_bf16_bits(b.x) | (f32_to_bf16_bits(b.y) << 16);
    out.w = f32_to_bf16_bits(b.z) | (f32_to_bf16_bits(b.w) << 16);
  }
  *reinterpret_cast<uint4*>(dst + r * K + (int64_t)c8 * 8) = out;
}

// One thread per block: the in-register decoder of the expert kernels times
// the e8m0 scale.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      int64_t n_blocks, float* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const uint4 q = ldg16(codes + b * 16);
  const float sc = e8m0_to_f32(scales[b]);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float4* o = reinterpret_cast<float4*>(out + b * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2f a = fp4x2_to_f32x2<0>(w[i]);
    const v2f c = fp4x2_to_f32x2<1>(w[i]);
    const v2f d = fp4x2_to_f32x2<2>(w[i]);
    const v2f e = fp4x2_to_f32x2<3>(w[i]);
    o[2 * i] = make_float4(a.x * sc, a.y * sc, c.x * sc, c.y * sc);
    o[2 * i + 1] = make_float4(d.x * sc, d.y * sc, e.x * sc, e.y * sc);
  }
}

__global__ __launch_bounds__(256) void merge_kernel(const float* a, const float* b, float* y,
                                                    size_t n, int vec) {
  const size_t n4 = vec ? n / 4 : 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 u = reinterpret_cast<const float4*>(a)[i];
    const float4 v = reinterpret_cast<const float4*>(b)[i];
    reinterpret_cast<float4*>(y)[i] = make_float4(u.x + v.x, u.y + v.y, u.z + v.z, u.w + v.w);
  }
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    y[i] = a[i] + b[i];
}

// streaming read of n16 16-byte words; each thread keeps U loads in flight
template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = i + u * stride < n16 ? src[i + u * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;   // keeps the loads live
}

// One thread per block and x vector: the per-block step of the decode
// kernels' gate/up rows.  MXFP4: the 32 e2m1 values converted to BF16 (scale
// 1.0), dotted with 32 BF16 x values in fp32, times the e8m0 scale.  NVFP4:
// the two 16-element half sums, each times its E4M3 scale.
__global__ __launch_bounds__(256) void dot_fp4_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ x,
                                                      int64_t n_blocks, int n_x, int nvfp4,
                                                      float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_blocks * n_x) return;
  const int64_t b = i / n_x;
  const int xv = (int)(i % n_x);
  const uint4 q = ldg16(codes + b * 16);
  uint32_t xp[16];
  const uint4* xs = reinterpret_cast<const uint4*>(x + (int64_t)xv * 32);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 v = xs[c];
    xp[4 * c] = v.x; xp[4 * c + 1] = v.y; xp[4 * c + 2] = v.z; xp[4 * c + 3] = v.w;
  }
  float r;
  if (!nvfp4) {
    r = fmaf(dot_fp4_bf16_block(q, xp), e8m0_to_f32(scales[b]), 0.f);
  } else {
    float s0, s1;
    dot_fp4_bf16_halves(q, xp, s0, s1);
    r = fmaf(s0, e4m3_to_f32(scales[2 * b]), fmaf(s1, e4m3_to_f32(scales[2 * b + 1]), 0.f));
  }
  out[i] = r;
}

// The decode wait-expired word (header word 32) to *out (if given), then
// cleared (if asked).
__global__ void decode_status_kernel(unsigned* hdr, int32_t* out, int clear) {
  const unsigned v = __hip_atomic_load(hdr + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (out) *out = (int32_t)v;
  if (clear) __hip_atomic_store(hdr + 32, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void fill_i32_kernel(int32_t* dst, int32_t value, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = value;
}

}  // namespace

hipError_t launch_quantize_nvfp4(const void* src, int src_bf16, int rows, int K, uint8_t* codes,
                                 uint8_t* scales, float* g, hipStream_t st) {
  if (rows <= 0 || K <= 0 || K % 16) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * K;
  hipLaunchKernelGGL(nvfp4_clear_kernel, dim3(1), dim3(1), 0, st, g);
  const int64_t blocks = (n + 256 * 16 - 1) / (256 * 16);
  hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256),
                     0, st, src, src_bf16, n, g);
  const int64_t nb = (int64_t)rows * (K / 16);
  hipLaunchKernelGGL(nvfp4_quant_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, src,
                     src_bf16, rows, K, codes, scales, g);
  hipLaunchKernelGGL(nvfp4_final_kernel, dim3(1), dim3(1), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const void* src, int src_bf16, int rows, int K, int64_t ld,
                                 uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t n = (int64_t)rows * (K / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                     src_bf16, rows, K, ld, codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const void* src, int src_bf16, int rows, int K, uint16_t* dst,
                            hipStream_t st) {
  const int64_t n = (int64_t)rows * (K / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                     src_bf16, rows, K, dst);
  return hipGetLastError();
}

hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t n_blocks,
                                float* out, hipStream_t st) {
  if (n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, st,
                     codes, scales, n_blocks, out);
  return hipGetLastError();
}

hipError_t launch_dot_fp4(const uint8_t* codes, const uint8_t* scales, const uint16_t* x,
                          int64_t n_blocks, int n_x, int nvfp4, float* out, hipStream_t st) {
  const int64_t n = n_blocks * n_x;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dot_fp4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, codes,
                     scales, x, n_blocks, n_x, nvfp4, out);
  return hipGetLastError();
}

hipError_t launch_decode_status(unsigned* hdr, int32_t* out, int clear, hipStream_t st) {
  hipLaunchKernelGGL(decode_status_kernel, dim3(1), dim3(1), 0, st, hdr, out, clear);
  return hipGetLastError();
}

hipError_t launch_merge(const float* a, const float* b, float* y, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  const int vec = ((((uintptr_t)a) | ((uintptr_t)b) | ((uintptr_t)y)) & 15) == 0;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, b, y, n, vec);
  return hipGetLastError();
}

// debug: one inclusive wave scan per 64 values
__global__ __launch_bounds__(64) void wave_scan_kernel(const int32_t* __restrict__ in,
                                                       int32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  out[i] = wave_scan_dpp(in[i]);
}

hipError_t launch_wave_scan(const int32_t* in, int32_t* out, int n_waves, hipStream_t st) {
  hipLaunchKernelGGL(wave_scan_kernel, dim3(n_waves), dim3(64), 0, st, in, out);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, size_t bytes, int blocks, uint32_t* out,
                             hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel<8>, dim3(blocks), dim3(256), 0, st,
                     static_cast<const uint4*>(src), n16, out);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* dst, int32_t value, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, value, n);
  return hipGetLastError();
}

}  // namespace moe

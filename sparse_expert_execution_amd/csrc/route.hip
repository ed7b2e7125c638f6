// route.hip - router logits (BF16 matrix cores for large batches), softmax and
// wavefront top-k.
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

// ---- large T, BF16 router: 64 tokens x 64 experts per workgroup on BF16 matrix
// cores (v_mfma_f32_16x16x32_bf16: exact products, fp32 accumulation).  Wave w
// takes tokens 16w..16w+15 of the tile against all 64 experts (4 tiles of 16).
// K goes in chunks of 64; a chunk of x and of W_r (8 KB each) is copied into
// LDS with global_load_lds (16 bytes a lane, no registers), kLgStages - 1
// chunks ahead, and read by all four waves.  In LDS a 16-row slice and
// 32-deep sub-block is one 1 KB fragment in MFMA operand order: lane l holds
// row l % 16, K elements 8 (l / 16) .. +7, so each lane's operand is one
// conflict-free 16-byte read.  A lane gets back rows 4 (l / 16) + i, column
// l % 16 of the 16 x 16 result.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

constexpr int kLgStages = 4;
struct LgStage {
  uint4 x[8 * 64];                  // fragments (slice * 2 + sub-block) of x
  uint4 w[8 * 64];                  // and of W_r
};

// the A fragment and 4 B fragments of one sub-block, with the wait inside
// the block: LDS reads the compiler could see would also wait for the copies
// still in flight into the other chunks' buffers
typedef unsigned int lg_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lg_frags(uint32_t aa, const uint32_t (&ba)[4], lg_u32x4& a,
                                         lg_u32x4 (&b)[4]) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %6\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %8\n\t"
      "ds_read_b128 %4, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
      : "v"(aa), "v"(ba[0]), "v"(ba[1]), "v"(ba[2]), "v"(ba[3])
      : "memory");
}

__device__ __forceinline__ uint4 lg_u4(const lg_u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

__global__ __launch_bounds__(256) void logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          int T, int H, int E,
                                                          float* __restrict__ z) {
  __shared__ LgStage s0, s1, s2, s3;
  auto stage = [&](int i) -> LgStage& { return i == 0 ? s0 : (i == 1 ? s1 : (i == 2 ? s2 : s3)); };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int r = lane & 15, kq = lane >> 4;
  // copy sources: wave w copies fragments 2w, 2w + 1 (slice w, both
  // sub-blocks) of x and of W_r; rows past T or E read row 0 (dropped)
  const uint16_t* xs;
  const uint16_t* wsrc;
  {
    const int t = t0 + wave * 16 + r, e = e0 + wave * 16 + r;
    xs = x + (int64_t)(t < T ? t : 0) * H + kq * 8;
    wsrc = wr + (int64_t)(e < E ? e : 0) * H + kq * 8;
  }
  auto issue = [&](int kc, LgStage& S) {
    const int k0 = kc * 64;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      __builtin_amdgcn_global_load_lds(xs + k0 + 32 * sb, &S.x[(wave * 2 + sb) * 64], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(wsrc + k0 + 32 * sb, &S.w[(wave * 2 + sb) * 64], 16, 0,
                                       0);
    }
  };
  constexpr int kCopies = 4;        // per wave per chunk

  v4f acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const LgStage& S) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      uint32_t ba[4];
#pragma unroll
      for (int n = 0; n < 4; ++n)
        ba[n] = (uint32_t)(uintptr_t)&S.w[(n * 2 + sb) * 64 + lane];
      lg_u32x4 a, b[4];
      lg_frags((uint32_t)(uintptr_t)&S.x[(wave * 2 + sb) * 64 + lane], ba, a, b);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lg_u4(a)),
                                                         as_bf16x8(lg_u4(b[n])), acc[n], 0, 0, 0);
    }
  };

  const int nk = H / 64;
#pragma unroll
  for (int i = 0; i < kLgStages - 1; ++i) issue(i < nk ? i : nk - 1, stage(i));
  for (int kc0 = 0; kc0 < nk; kc0 += kLgStages) {
#pragma unroll
    for (int i = 0; i < kLgStages; ++i) {
      const int kc = kc0 + i;
      if (kc < nk) {
        // this wave's copies of chunk kc are done once at most the later
        // kLgStages - 2 chunks' copies are outstanding; the barrier shows
        // every wave's copies and frees the buffer chunk kc - 1 used
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kLgStages - 2) * kCopies) : "memory");
        __builtin_amdgcn_s_barrier();
        const int kn = kc + kLgStages - 1;
        issue(kn < nk ? kn : nk - 1, stage((i + kLgStages - 1) % kLgStages));
        compute(stage(i));
      }
    }
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + n * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + wave * 16 + 4 * kq + i;
      if (t < T && e < E) z[(int64_t)t * E + e] = acc[n][i];
    }
  }
}

// ---- softmax + top-k: one wave per token --------------------------------------
template <int M>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int T, int E,
                                                   int k, int renorm, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_one_token<M>(z + (int64_t)t * E, E, k, renorm, ids + (int64_t)t * k, w + (int64_t)t * k);
}

}  // namespace

hipError_t launch_route_large(const void* x, const void* w_router, int router_f32, int T,
                              int H, int E, int k, int renorm, float* logits, int32_t* ids,
                              float* w, hipStream_t st) {
  dim3 grid((T + 63) / 64, (E + 63) / 64);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (!router_f32 && H % 64 == 0)
    hipLaunchKernelGGL(logits_mfma_kernel, grid, dim3(256), 0, st, xb,
                       static_cast<const uint16_t*>(w_router), T, H, E, logits);
  else if (router_f32)
    hipLaunchKernelGGL((logits_tiled_kernel<true>), grid, dim3(256), 0, st, xb, w_router, T, H, E,
                       logits);
  else
    hipLaunchKernelGGL((logits_tiled_kernel<false>), grid, dim3(256), 0, st, xb, w_router, T, H,
                       E, logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g((T + 3) / 4), b(256);
  if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, g, b, 0, st, logits, T, E, k, renorm, ids, w);
  else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, g, b, 0, st, logits, T, E, k, renorm, ids, w);
  else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, g, b, 0, st, logits, T, E, k, renorm, ids, w);
  else hipLaunchKernelGGL(topk_kernel<16>, g, b, 0, st, logits, T, E, k, renorm, ids, w);
  return hipGetLastError();
}

}  // namespace moe

// prefill_nvfp4.hip - the prefill expert GEMMs for NVFP4 weights, on the
// gfx950 BF16 matrix cores.
//
// NVFP4 is the format of the pages' GLM-5.2 and laptop builds ("FreeToken
// 753b Model Explained", "Performance Benchmarks and Model Fit"): e2m1 codes
// with an E4M3 scale per 16 elements along K and an fp32 scale per matrix.
// CDNA4's scaled FP4 matrix instructions take one power-of-two scale per 32
// elements, which an E4M3 scale per 16 is not, so these GEMMs expand each
// weight to e2m1 x E4M3 in BF16 -- exact, the product has at most 5
// significant bits -- and run v_mfma_f32_16x16x32_bf16 with x as given (BF16)
// and the matrix scale applied to the fp32 results.
//
// Precision contract: x BF16 as given; g = gs * (W_g x), u = us * (W_u x) in
// fp32; h = silu(g) * u rounded to BF16 (nearest even); o = ds * (W_d h) in
// fp32, written to the pair's partial row and combined as for MXFP4.
//
// Tiles come from the expert sort of prefill.hip: 128 sorted (token, expert)
// pairs of one expert.  A workgroup (4 waves) computes 128 rows x 64 columns:
// wave v takes rows 32 v .. 32 v + 31 (two 16-row slices) and all 64 columns
// (four 16-column slices).  Per K chunk of 128 the weight rows' codes and
// scales are loaded into registers one chunk ahead, expanded to BF16 by the
// whole workgroup into LDS (rows padded to 272 bytes, so a fragment read
// meets 16 distinct bank groups), and the activation fragments are loaded
// straight from memory (16 bytes a lane per 16 x 32 step).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kNvThreads = 256;
constexpr int kNvBM = 128;           // rows of a tile (the sort's tile)
static_assert(kNvBM == kPrefillMT, "a workgroup takes one tile of the expert sort");
constexpr int kNvBN = 64;            // weight rows (output columns) of a tile
constexpr int kNvKC = 128;           // K per chunk
constexpr int kNvLdsRow = kNvKC * 2 + 16;   // bytes of one expanded weight row in LDS

// token of pair p (a pair id outside [0, T (k + 1)) reads token 0)
__device__ __forceinline__ int nv_pair_token(const NvPrefillArgs& a, int p) {
  const int nr = a.T * a.k;
  if ((unsigned)p >= (unsigned)(nr + a.T)) return 0;
  return p < nr ? p / a.k : p - nr;
}

__device__ __forceinline__ const uint8_t* nv_bin_base(const NvPrefillArgs& a, int bin) {
  if (bin >= a.E) return a.shared;
  const int slot = a.slot_of ? a.slot_of[bin] : bin;
  return a.pool + (int64_t)slot * a.expert_bytes;
}

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t nv_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 8 e2m1 codes (one dword, low nibble first) times an E4M3 scale as 8 BF16
// values (16 bytes).  Each product is exact in fp32 and has at most 5
// significant bits, so its upper half is its BF16 value.
__device__ __forceinline__ uint4 nv_expand8(uint32_t word, float scale) {
  const v2f a = fp4x2_to_f32x2<0>(word);
  const v2f b = fp4x2_to_f32x2<1>(word);
  const v2f c = fp4x2_to_f32x2<2>(word);
  const v2f d = fp4x2_to_f32x2<3>(word);
  auto hi2 = [&](float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi * scale), __float_as_uint(lo * scale),
                                 0x07060302u);
  };
  return make_uint4(hi2(a.x, a.y), hi2(b.x, b.y), hi2(c.x, c.y), hi2(d.x, d.y));
}

template <int MODE>
__global__ __launch_bounds__(kNvThreads, 2) void nv_gemm_kernel(NvPrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kNvBN * kNvLdsRow];
  const int nout = MODE == 1 ? a.I : a.H;
  const int bn = MODE == 1 ? kNvBN / 2 : kNvBN;   // output columns of a workgroup
  const int nt = nout / bn;
  // row tiles in 8 contiguous runs, one per XCD, and a row tile's column
  // tiles one after another on its XCD, as in the MXFP4 GEMMs: activations
  // and shared weight tiles are served from that XCD's L2
  const int x = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int run = (a.tiles[0] + 7) >> 3;
  const int ti = kk / nt;
  const int tile = x * run + ti;
  if (ti >= run || tile >= a.tiles[0]) return;
  const int bin = a.tiles[1 + 2 * tile];
  const int row0 = a.tiles[2 + 2 * tile];
  const int seg_end = a.seg_start[bin + 1];
  const int col0 = (kk - ti * nt) * bn;
  const uint8_t* base = nv_bin_base(a, bin);
  const int K = MODE == 1 ? a.H : a.I;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fg = lane >> 4;

  // activation rows of this lane (two 16-row slices); rows past the segment
  // read the tile's first row and their results are dropped
  const uint16_t* arow[2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int r = row0 + 32 * wv + 16 * ms + fr;
    const int rr = r < seg_end ? r : row0;
    if (MODE == 1) arow[ms] = a.x + (int64_t)nv_pair_token(a, a.sorted_pair[rr]) * a.H;
    else arow[ms] = a.hb + (int64_t)rr * a.I;
  }
  // expansion share of this thread: weight row tid / 4 of the tile, quarter
  // tid % 4 of the chunk (32 values: 16 code bytes, 2 scale bytes)
  const int er = tid >> 2, eq = tid & 3;
  const uint8_t* ecodes;
  const uint8_t* escales;
  {
    int mat, n;
    if (MODE == 1) { mat = er >> 5; n = col0 + (er & 31); }
    else { mat = 2; n = col0 + er; }
    ecodes = base + a.off[2 * mat] + (int64_t)n * (K / 2) + eq * 16;
    escales = base + a.off[2 * mat + 1] + (int64_t)n * (K / 16) + eq * 2;
  }
  float msc[2];                        // matrix scales of the column slices' matrices
  {
    const float* gs = reinterpret_cast<const float*>(base + a.goff);
    if (MODE == 1) { msc[0] = gs[0]; msc[1] = gs[1]; }
    else { msc[0] = gs[2]; msc[1] = gs[2]; }
  }

  v4f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kNvKC;
  uint4 wq = *reinterpret_cast<const uint4*>(ecodes);
  uint32_t ws = *reinterpret_cast<const uint16_t*>(escales);
  // activation fragments of a chunk: step s, lane group g -> K0 + 32 s + 8 g
  uint4 av[2][4], an[2][4];
  auto load_a = [&](int K0, uint4 (&v)[2][4]) {
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        v[ms][s] = *reinterpret_cast<const uint4*>(arow[ms] + K0 + 32 * s + 8 * fg);
  };
  load_a(0, av);
  auto expand = [&](int buf, uint4 q, uint32_t s) {
    const float s0 = e4m3_to_f32(s & 0xffu), s1 = e4m3_to_f32(s >> 8);
    uint4* dst = reinterpret_cast<uint4*>(&lds[buf][er * kNvLdsRow + eq * 64]);
    dst[0] = nv_expand8(q.x, s0);
    dst[1] = nv_expand8(q.y, s0);
    dst[2] = nv_expand8(q.z, s1);
    dst[3] = nv_expand8(q.w, s1);
  };
  expand(0, wq, ws);
  __syncthreads();
  for (int c = 0; c < nk; ++c) {
    const int buf = c & 1;
    const int K0 = c * kNvKC;
    // the next chunk's weights and activations into registers
    if (c + 1 < nk) {
      wq = *reinterpret_cast<const uint4*>(ecodes + (K0 + kNvKC) / 2);
      ws = *reinterpret_cast<const uint16_t*>(escales + (K0 + kNvKC) / 16);
      load_a(K0 + kNvKC, an);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8bf bv[4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const uint4 q = *reinterpret_cast<const uint4*>(
            &lds[buf][(ns * 16 + fr) * kNvLdsRow + (32 * s + 8 * fg) * 2]);
        bv[ns] = __builtin_bit_cast(v8bf, q);
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) {
        const v8bf ax = __builtin_bit_cast(v8bf, av[ms][s]);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bv[ns], acc[ms][ns], 0, 0, 0);
      }
    }
    if (c + 1 < nk) {
      expand(buf ^ 1, wq, ws);
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s) av[ms][s] = an[ms][s];
    }
    __syncthreads();
  }

  if (MODE == 1) {
    // h = silu(gs * g) * (us * u) of h columns col0 + 16 j + fr, j = 0, 1
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 32 * wv + 16 * ms + 4 * fg + i;
        if (r >= seg_end) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float g = acc[ms][j][i] * msc[0];
          const float u = acc[ms][j + 2][i] * msc[1];
          const float h = g / (1.0f + expf(-g)) * u;
          a.hb[(int64_t)r * a.I + col0 + 16 * j + fr] = (uint16_t)nv_bf16_rne(h);
        }
      }
  } else {
    // o = ds * (W_d h) into the pair's row of the partial outputs
    const int nr = a.T * a.k;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 32 * wv + 16 * ms + 4 * fg + i;
        if (r >= seg_end) continue;
        const int p = a.sorted_pair[r];
        if ((unsigned)p >= (unsigned)(nr + a.T)) continue;
        const int prow = p < nr ? (p / a.k) * (a.k + 1) + (p % a.k) : (p - nr) * (a.k + 1) + a.k;
        float* dst = a.partial + (int64_t)prow * a.H + col0 + fr;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) dst[16 * ns] = acc[ms][ns][i] * msc[0];
      }
  }
}

}  // namespace

hipError_t launch_prefill_nvfp4_gemms(const NvPrefillArgs& a, int max_tiles, hipStream_t st) {
  const int groups = (max_tiles + 7) / 8;
  const int nt1 = a.I / (kNvBN / 2), nt2 = a.H / kNvBN;
  hipLaunchKernelGGL(nv_gemm_kernel<1>, dim3(groups * 8 * nt1), dim3(kNvThreads), 0, st, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(nv_gemm_kernel<2>, dim3(groups * 8 * nt2), dim3(kNvThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe

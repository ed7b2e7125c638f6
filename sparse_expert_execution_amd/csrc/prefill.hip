// prefill.hip - long-batch expert FFNs on the gfx950 scaled FP4 matrix cores.
//
// With thousands of tokens a layer touches nearly every expert (explainx.ai
// guide, "Prefill: load almost every expert without idling the GPU"), so the
// work is a grouped GEMM: (token, expert) pairs are counting-sorted by
// expert, each expert multiplies its token rows once per weight tile, and the
// per-pair outputs are combined with the gate weights afterwards.
//
// Precision contract: x is quantised to MXFP4 along H and h along I with the
// library's MXFP4 encoder; both products are FP4 x FP4 with e8m0 block scales
// on v_mfma_scale_f32_16x16x128_f8f6f4 with fp32 accumulation.  NVFP4 weights
// share steps 2-4 and 7 and run their GEMMs in prefill_nvfp4.hip.
//
// Pipeline (one stream, no host synchronisation):
//   1 quantise x rows                 x [T][H] bf16 -> codes/scales
//   2 per-chunk expert histogram      256 pairs per chunk
//   3 scan                            segment starts, per-chunk offsets, tiles
//   4 stable scatter                  sorted_pair[pos] = pair id
//   5 GEMM1 gate|up + SwiGLU + MXFP4  -> hq (sorted order)      (LDS-tiled)
//   6 GEMM2 down                      -> partial[t][j][H] fp32    (LDS-tiled)
//   7 combine                         y[t] = sum_j w[t][j] partial[t][j] (+ shared)
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kChunk = kPrefillChunk;
constexpr int kMT = kPrefillMT;

// ---- MFMA fragments ----------------------------------------------------------
// A 16-row x 128-K MXFP4 tile as one lane's operand: lane l supplies row
// l % 16 and the 32-element K block l / 16 (16 bytes of codes, one scale).
struct Frag {
  uint4 q;
  uint32_t s;
};

__device__ __forceinline__ Frag load_frag(const uint8_t* codes_row, const uint8_t* scales_row,
                                          int k0, bool ok) {
  Frag f;
  const int kb = threadIdx.x & 63;
  const int blk = (k0 >> 5) + (kb >> 4);
  if (ok) {
    f.q = ldg16(codes_row + (int64_t)blk * 16);
    f.s = scales_row[blk];
  } else {
    f.q = make_uint4(0, 0, 0, 0);
    f.s = 127;
  }
  return f;
}

__device__ __forceinline__ v4f mfma_fp4(const Frag& a, const Frag& b, v4f c) {
  v8i av = {(int)a.q.x, (int)a.q.y, (int)a.q.z, (int)a.q.w, 0, 0, 0, 0};
  v8i bv = {(int)b.q.x, (int)b.q.y, (int)b.q.z, (int)b.q.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)a.s, 0,
                                                          (int)b.s);
}

// output element (row, col) held by lane l, register i of a 16x16 tile
__device__ __forceinline__ int d_row(int lane, int i) { return 4 * (lane >> 4) + i; }
__device__ __forceinline__ int d_col(int lane) { return lane & 15; }

// ---- 1: quantise bf16 rows to MXFP4 -------------------------------------------
__global__ __launch_bounds__(256) void quant_bf16_kernel(const uint16_t* __restrict__ x, int T,
                                                         int H, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int nb = H / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * nb) return;
  const int64_t r = gid / nb;
  const int b = (int)(gid % nb);
  const uint4* s = reinterpret_cast<const uint4*>(x + r * H + (int64_t)b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = s[i];
    v[8 * i + 0] = bf16_lo(q.x); v[8 * i + 1] = bf16_hi(q.x);
    v[8 * i + 2] = bf16_lo(q.y); v[8 * i + 3] = bf16_hi(q.y);
    v[8 * i + 4] = bf16_lo(q.z); v[8 * i + 5] = bf16_hi(q.z);
    v[8 * i + 6] = bf16_lo(q.w); v[8 * i + 7] = bf16_hi(q.w);
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
    for (int i = 0; i < 32; ++i) packed[i / 8] |= e2m1_code(mx_scale_down(v[i], X)) << (4 * (i % 8));
  }
  *reinterpret_cast<uint4*>(codes + r * (H / 2) + (int64_t)b * 16) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[r * nb + b] = (uint8_t)sbyte;
}

// bin of a pair: routed expert (if resident), E for the shared expert, -1 skip
struct SortArgs {
  const int32_t* ids;
  const int32_t* slot_of;
  int T, k, E, has_shared, n_pairs, n_chunks, max_tiles;
  int32_t* chunk_counts;
  int32_t* seg_start;
  int32_t* tiles;
  int32_t* sorted_pair;
};

__device__ __forceinline__ int pair_bin(const SortArgs& a, int p) {
  const int nr = a.T * a.k;
  if (p >= nr) return a.E;  // shared
  const int e = a.ids[p];
  if (e < 0 || e >= a.E) return -1;
  if (a.slot_of && a.slot_of[e] < 0) return -1;
  return e;
}

// ---- 2: per-chunk histogram ----------------------------------------------------
__global__ __launch_bounds__(256) void sort_count_kernel(SortArgs a) {
  extern __shared__ int hist[];
  const int nb = a.E + 1;
  for (int b = threadIdx.x; b < nb; b += 256) hist[b] = 0;
  __syncthreads();
  const int p = blockIdx.x * kChunk + threadIdx.x;
  if (p < a.n_pairs) {
    const int b = pair_bin(a, p);
    if (b >= 0) atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += 256)
    a.chunk_counts[(int64_t)blockIdx.x * nb + b] = hist[b];
}

// ---- 3: scan (one workgroup) ----------------------------------------------------
// seg_start[b] = first sorted position of bin b (seg_start[E+1] = total);
// chunk_counts[c][b] becomes the first position of chunk c's pairs of bin b;
// tiles = {n_tiles, (bin, row0) ...} with row0 the absolute sorted position.
__global__ __launch_bounds__(1024) void sort_scan_kernel(SortArgs a) {
  extern __shared__ int sh[];
  const int nb = a.E + 1;
  int* tot = sh;            // [nb]
  int* ntile = sh + nb;     // [nb]
  // one thread per bin walks the chunks; the loops are unrolled so that many
  // of its loads are in flight at once
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    int s = 0;
#pragma unroll 16
    for (int c = 0; c < a.n_chunks; ++c) s += a.chunk_counts[(int64_t)c * nb + b];
    tot[b] = s;
    ntile[b] = (s + kMT - 1) / kMT;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int pos = 0, tp = 0;
    for (int b = 0; b < nb; ++b) {
      const int s = tot[b], n = ntile[b];
      tot[b] = pos;      // segment start
      ntile[b] = tp;     // first tile index
      pos += s;
      tp += n;
    }
    a.seg_start[nb] = pos;
    a.tiles[0] = tp < a.max_tiles ? tp : a.max_tiles;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    const int start = tot[b];
    const int end = (b + 1 < nb) ? tot[b + 1] : a.seg_start[nb];
    a.seg_start[b] = start;
    int pos = start;
    for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
      int n[16];                   // all loads of a batch before its stores
#pragma unroll
      for (int i = 0; i < 16; ++i)
        n[i] = c0 + i < a.n_chunks ? a.chunk_counts[(int64_t)(c0 + i) * nb + b] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < a.n_chunks) a.chunk_counts[(int64_t)(c0 + i) * nb + b] = pos;
        pos += n[i];
      }
    }
    int ti = ntile[b];
    for (int r0 = start; r0 < end; r0 += kMT, ++ti) {
      if (ti < a.max_tiles) {
        a.tiles[1 + 2 * ti] = b;
        a.tiles[2 + 2 * ti] = r0;
      }
    }
  }
}

// ---- 4: stable scatter ------------------------------------------------------------
__global__ __launch_bounds__(256) void sort_scatter_kernel(SortArgs a) {
  __shared__ int sbin[kChunk];
  const int nb = a.E + 1;
  const int p = blockIdx.x * kChunk + threadIdx.x;
  const int b = p < a.n_pairs ? pair_bin(a, p) : -1;
  sbin[threadIdx.x] = b;
  __syncthreads();
  if (b < 0) return;
  int rank = 0;
  for (int q = 0; q < (int)threadIdx.x; ++q) rank += (sbin[q] == b);
  // count and scatter read the same ids and slot table in stream order, so
  // every position is in range and written once; the guard (and the range
  // checks where the GEMMs read sorted_pair) keep a caller's concurrent
  // change of those inputs from turning into stores or loads out of bounds
  const int pos = a.chunk_counts[(int64_t)blockIdx.x * nb + b] + rank;
  if ((unsigned)pos < (unsigned)a.n_pairs) a.sorted_pair[pos] = p;
}

struct GemmArgs {
  const int32_t* slot_of;
  const uint8_t* pool;
  const uint8_t* shared;
  int64_t expert_bytes;
  int64_t off[6];
  int T, H, I, E, k;
  const int32_t* seg_start;
  const int32_t* tiles;
  const int32_t* sorted_pair;
  const uint8_t* xq_codes;
  const uint8_t* xq_scales;
  uint8_t* hq_codes;
  uint8_t* hq_scales;
  float* partial;
};

__device__ __forceinline__ const uint8_t* bin_base(const GemmArgs& a, int bin) {
  if (bin >= a.E) return a.shared;
  const int slot = a.slot_of ? a.slot_of[bin] : bin;
  return a.pool + (int64_t)slot * a.expert_bytes;
}

// token of pair p (a pair id outside [0, T (k + 1)) reads token 0)
__device__ __forceinline__ int pair_token(const GemmArgs& a, int p) {
  const int nr = a.T * a.k;
  if ((unsigned)p >= (unsigned)(nr + a.T)) return 0;
  return p < nr ? p / a.k : p - nr;
}

// ---- 5/6: grouped GEMMs on LDS tiles ----------------------------------------------
// One workgroup computes a 128-row (sorted pairs of one expert) x 256-column
// tile of A . B^T on v_mfma_scale_f32_16x16x128_f8f6f4 (K 128 per MFMA step).
// Operands reach LDS by global_load_lds copies (16 bytes a lane, no
// registers) several steps ahead of the matrix work; each buffer is its own
// LDS variable so the compiler can count the copies.  8 waves (two per SIMD,
// so one's matrix work covers the other's LDS waits) as 2 (64 rows) x 4
// (64 B rows); a wave holds 4 x 4 16x16 accumulators.
//   GEMM1: A = MXFP4(x) rows gathered by token, B = [gate rows c0..c0+127 ;
//          up rows c0..c0+127]; epilogue h = silu(g) * u -> MXFP4 along I.
//   GEMM2: A = MXFP4(h) rows (sorted order), B = down rows n0..n0+255;
//          epilogue writes the pair's partial output row.
// Two copy schemes:
//   wide (K a multiple of 512): a buffer holds two steps (K 256) and a copy
//     moves 8 rows x 128 bytes, whole cache lines.  Piece p (16 bytes) of
//     row i of a copy's 8 rows lands in slot 8 i + (p ^ (4 j + i / 2)), j
//     the copy's half of its 16-row slice, so each 16-lane group of a
//     fragment read meets 16 distinct bank groups.  The scale bytes of four
//     steps (16 per row) come in one copy per row, into a double-buffered
//     scale group.  3 buffers, 2 ahead.
//   narrow (otherwise): a buffer holds one step; a copy moves 16 rows x 64
//     bytes in fragment order (lane l: row l % 16, K block l / 16), and the
//     step's scale dword of each row rides along.  5 buffers, 4 ahead.
// A copy that serves 64 rows with 4 or 16 bytes each touches 64 cache lines;
// whole-line copies and grouped scales are what make the wide scheme faster.
constexpr int kBM = 128, kBN = 256;
constexpr int kGemmThreads = 512;   // 8 waves, two per SIMD
constexpr int kStages = 5;          // narrow
constexpr int kWStages = 3;         // wide

struct Stage {                      // narrow: one step
  uint4 a[(kBM / 16) * 64];         // 8 slices x 64 lanes x 16 bytes
  uint4 b[(kBN / 16) * 64];         // 16 slices
  uint32_t as[kBM];                 // 4 scale bytes (the step's K blocks) per row
  uint32_t bs[kBN];
};
struct WStage {                     // wide: two steps, a slice is 2 copies of 1 KB
  uint4 a[(kBM / 16) * 128];
  uint4 b[(kBN / 16) * 128];
};
struct ScaleGroup {                 // scale bytes of four steps (16 K blocks) per row
  uint4 as[kBM];
  uint4 bs[kBN];
};

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

// Four fragments (16 code bytes each) and their scale dwords from LDS byte
// addresses.  The reads are written out here, with their wait inside the same
// block, because LDS reads the compiler can see would make it wait for every
// copy still in flight into any step's buffer, not just the one being read.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_frag4(const uint32_t (&qa)[4], const uint32_t (&sa)[4],
                                          u32x4 (&q)[4], uint32_t (&sc)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b32 %4, %12\n\t"
      "ds_read_b32 %5, %13\n\t"
      "ds_read_b32 %6, %14\n\t"
      "ds_read_b32 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(sc[0]), "=&v"(sc[1]),
        "=&v"(sc[2]), "=&v"(sc[3])
      : "v"(qa[0]), "v"(qa[1]), "v"(qa[2]), "v"(qa[3]), "v"(sa[0]), "v"(sa[1]), "v"(sa[2]),
        "v"(sa[3])
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

struct Tile {
  int row0, seg_end, col0;
  const uint8_t* base;              // the expert's block
};

// Workgroup ids go round-robin over the 8 XCDs, each with its own L2.  The
// row tiles are cut into 8 contiguous runs, one per XCD, and an XCD's
// workgroups walk its run tile by tile, the nt column tiles of a row tile
// one after another: a row tile's A operand is fetched from HBM once and
// served from that L2 to its other column tiles, and the row tiles of one
// expert (consecutive in the sort) run on the same XCD at about the same
// time, so a weight tile they share is fetched once as well.  The grid has
// 8 * ceil(max_tiles / 8) * nt workgroups; those past the run exit.
__device__ __forceinline__ bool xcd_tile(const int32_t* tiles, int nt, int& tile, int& col) {
  const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int n = tiles[0];
  const int run = (n + 7) >> 3;
  const int i = k / nt;
  tile = x * run + i;
  col = k - i * nt;
  return i < run && tile < n;
}

template <int MODE>
__device__ __forceinline__ bool gemm_tile(const GemmArgs& a, Tile& t) {
  const int nout = MODE == 1 ? a.I : a.H;      // output columns of the whole GEMM
  const int bn = MODE == 1 ? kBN / 2 : kBN;    // output columns of one workgroup
  const int nt = (nout + bn - 1) / bn;
  int tile, col;
  if (!xcd_tile(a.tiles, nt, tile, col)) return false;
  const int bin = a.tiles[1 + 2 * tile];
  t.row0 = a.tiles[2 + 2 * tile];
  t.seg_end = a.seg_start[bin + 1];
  t.col0 = col * bn;
  t.base = bin_base(a, bin);
  return true;
}

// codes and scales of A row r (a sorted position; rows past the segment read
// the tile's first row, whose results are dropped)
template <int MODE>
__device__ __forceinline__ void a_row(const GemmArgs& a, const Tile& t, int r,
                                      const uint8_t*& c, const uint8_t*& sc) {
  const int rr = r < t.seg_end ? r : t.row0;
  if (MODE == 1) {
    const int tok = pair_token(a, a.sorted_pair[rr]);
    c = a.xq_codes + (int64_t)tok * (a.H / 2);
    sc = a.xq_scales + (int64_t)tok * (a.H / 32);
  } else {
    c = a.hq_codes + (int64_t)rr * (a.I / 2);
    sc = a.hq_scales + (int64_t)rr * (a.I / 32);
  }
}

// codes and scales of row rt of the B tile (GEMM1: gate rows, then up rows)
template <int MODE>
__device__ __forceinline__ void b_row(const GemmArgs& a, const Tile& t, int rt,
                                      const uint8_t*& c, const uint8_t*& sc) {
  const int K = MODE == 1 ? a.H : a.I;
  const int nout = MODE == 1 ? a.I : a.H;
  int mat, n;
  if (MODE == 1) { mat = rt >> 7; n = t.col0 + (rt & 127); }
  else { mat = 2; n = t.col0 + rt; }
  const int nn = n < nout ? n : 0;
  c = t.base + a.off[2 * mat] + (int64_t)nn * (K / 2);
  sc = t.base + a.off[2 * mat + 1] + (int64_t)nn * (K / 32);
}

// the wave's 4 x 4 MFMAs of one step from fragment and scale addresses
template <int MODE>
__device__ __forceinline__ void mma_step(const uint32_t (&aq)[4], const uint32_t (&as)[4],
                                         const uint32_t (&bq)[4], const uint32_t (&bs)[4],
                                         int fk, v4f (&acc)[4][4]) {
  Frag fa[4];
  {
    u32x4 q[4];
    uint32_t sc[4];
    lds_frag4(aq, as, q, sc);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      fa[ms].q = make_uint4(q[ms].x, q[ms].y, q[ms].z, q[ms].w);
      fa[ms].s = (sc[ms] >> (8 * fk)) & 0xffu;
    }
  }
  u32x4 q[4];
  uint32_t sc[4];
  lds_frag4(bq, bs, q, sc);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    Frag fb;
    fb.q = make_uint4(q[ns].x, q[ns].y, q[ns].z, q[ns].w);
    fb.s = (sc[ns] >> (8 * fk)) & 0xffu;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) acc[ms][ns] = mfma_fp4(fa[ms], fb, acc[ms][ns]);
  }
}

// B slice read by n-slice ns of wave column wn.  GEMM1: slices 0..7 gate,
// 8..15 up; wave wn takes 32 h columns of each (n-slices 0, 1 gate and 2, 3
// up).  GEMM2: 4 consecutive slices.
template <int MODE>
__device__ __forceinline__ int b_slice(int wn, int ns) {
  return MODE == 1 ? (ns >> 1) * 8 + wn * 2 + (ns & 1) : wn * 4 + ns;
}

template <int MODE>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const Tile& t,
                                              v4f (&acc)[4][4], int wm, int wn, int lane) {
  const int H = a.H, I = a.I;
  if (MODE == 1) {
    // h = silu(g) * u; each row's 32-column block (gate and up n-slice
    // pairs) to MXFP4
    const int c0 = t.col0 + wn * 32;             // first h column of this wave
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      {
        constexpr int blk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = t.row0 + wm * 64 + ms * 16 + d_row(lane, i);
          const float g0 = acc[ms][0][i], g1 = acc[ms][1][i];
          const float u0 = acc[ms][2][i], u1 = acc[ms][3][i];
          const float h0 = g0 / (1.0f + expf(-g0)) * u0;
          const float h1 = g1 / (1.0f + expf(-g1)) * u1;
          float amax = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
          uint32_t q0 = 0, q1 = 0, sbyte = 0;
          if (amax > 0.f) {
            const int X = mx_block_exponent(amax);
            sbyte = (uint32_t)(X + 127);
            q0 = e2m1_code(mx_scale_down(h0, X));
            q1 = e2m1_code(mx_scale_down(h1, X));
          }
          const uint32_t n0 = __shfl_xor(q0, 1, kWave);
          const uint32_t n1 = __shfl_xor(q1, 1, kWave);
          const int c = d_col(lane);
          const int cb = c0 + blk * 32;         // first column of the block
          if (r < t.seg_end) {
            uint8_t* dst = a.hq_codes + (int64_t)r * (I / 2) + cb / 2;
            if ((c & 1) == 0) {
              dst[c >> 1] = (uint8_t)(q0 | (n0 << 4));
              dst[8 + (c >> 1)] = (uint8_t)(q1 | (n1 << 4));
            }
            if (c == 0) a.hq_scales[(int64_t)r * (I / 32) + cb / 32] = (uint8_t)sbyte;
          }
        }
      }
    }
  } else {
    const int nr = a.T * a.k;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = t.row0 + wm * 64 + ms * 16 + d_row(lane, i);
        if (r >= t.seg_end) continue;
        const int p = a.sorted_pair[r];
        if ((unsigned)p >= (unsigned)(nr + a.T)) continue;
        int prow;
        if (p < nr) prow = (p / a.k) * (a.k + 1) + (p % a.k);
        else prow = (p - nr) * (a.k + 1) + a.k;
        float* dst = a.partial + (int64_t)prow * H + t.col0 + wn * 64 + d_col(lane);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          if (t.col0 + wn * 64 + ns * 16 < H) dst[ns * 16] = acc[ms][ns][i];
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(GemmArgs a) {
  __shared__ Stage st0, st1, st2, st3, st4;
  auto stage = [&](int s) -> Stage& {
    return s == 0 ? st0 : (s == 1 ? st1 : (s == 2 ? st2 : (s == 3 ? st3 : st4)));
  };
  Tile t;
  if (!gemm_tile<MODE>(a, t)) return;
  const int K = MODE == 1 ? a.H : a.I;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;         // 2 (64 rows) x 4 (64 B rows)
  const int fr = lane & 15, fk = lane >> 4;

  // copy sources of this lane: A slice wv; B slices 2 wv, 2 wv + 1; scale
  // dwords of A rows 64 (wv & 1) + lane and of B rows 64 (wv & 3) + lane
  const uint8_t* ac;
  const uint8_t* bc[2];
  const uint8_t* as_src;
  const uint8_t* bs_src;
  {
    const uint8_t* dummy;
    a_row<MODE>(a, t, t.row0 + wv * 16 + fr, ac, dummy);
#pragma unroll
    for (int j = 0; j < 2; ++j) b_row<MODE>(a, t, (2 * wv + j) * 16 + fr, bc[j], dummy);
    const uint8_t* c;
    a_row<MODE>(a, t, t.row0 + (wv & 1) * 64 + lane, c, as_src);
    b_row<MODE>(a, t, (wv & 3) * 64 + lane, c, bs_src);
  }
  // every wave issues the same number of copies per step (5), so one count
  // covers all: the scale dwords are copied by several waves (the same bytes
  // to the same place)
  auto issue = [&](int kt, Stage& S) {
    const int k0 = kt * 128;
    dma16(ac + k0 / 2 + fk * 16, &S.a[wv * 64]);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(bc[j] + k0 / 2 + fk * 16, &S.b[(2 * wv + j) * 64]);
    dma4(as_src + k0 / 32, &S.as[(wv & 1) * 64]);
    dma4(bs_src + k0 / 32, &S.bs[(wv & 3) * 64]);
  };
  constexpr int kCopies = 5;                   // copies per wave per step

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage& S) {
    uint32_t aq[4], as[4], bq[4], bs[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const int sl = wm * 4 + ms;
      aq[ms] = lds_addr(&S.a[sl * 64 + lane]);
      as[ms] = lds_addr(&S.as[sl * 16 + fr]);
    }
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int sl = b_slice<MODE>(wn, ns);
      bq[ns] = lds_addr(&S.b[sl * 64 + lane]);
      bs[ns] = lds_addr(&S.bs[sl * 16 + fr]);
    }
    mma_step<MODE>(aq, as, bq, bs, fk, acc);
  };

  const int nk = K / 128;
  // prologue: steps 0 .. kStages-2 (a step past the end re-reads the last)
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue(s < nk ? s : nk - 1, stage(s));
  for (int kt0 = 0; kt0 < nk; kt0 += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      const int kt = kt0 + s;
      if (kt < nk) {
        // this wave's copies of step kt are done once at most the later
        // kStages-2 steps' copies are outstanding; the barrier makes every
        // wave's copies visible and frees the buffer step kt-1 used
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kStages - 2) * kCopies) : "memory");
        __builtin_amdgcn_s_barrier();
        const int kn = kt + kStages - 1;
        issue(kn < nk ? kn : nk - 1, stage((s + kStages - 1) % kStages));
        compute(stage(s));
      }
    }
  }
  gemm_epilogue<MODE>(a, t, acc, wm, wn, lane);
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_wide_kernel(GemmArgs a) {
  __shared__ WStage ws0, ws1, ws2;
  __shared__ ScaleGroup sg0, sg1;
  auto stage = [&](int s) -> WStage& { return s == 0 ? ws0 : (s == 1 ? ws1 : ws2); };
  Tile t;
  if (!gemm_tile<MODE>(a, t)) return;
  const int K = MODE == 1 ? a.H : a.I;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  const int fr = lane & 15, fk = lane >> 4;

  // copy lanes: row ci = lane / 8 of the copy's 8 rows; its piece is
  // (lane % 8) ^ (4 j + ci / 2), so lane l lands in slot l = 8 ci + (lane % 8)
  const int ci = lane >> 3;
  const uint8_t* ac[2];              // A slice wv, halves j = 0, 1
  const uint8_t* bc[4];              // B slices 2 wv + (q >> 1), halves q & 1
  const uint8_t* ssrc = nullptr;     // scales: waves 0-1 A rows, 2-5 B rows
  {
    const uint8_t* dummy;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = (lane & 7) ^ (4 * j + (ci >> 1));
      a_row<MODE>(a, t, t.row0 + wv * 16 + 8 * j + ci, ac[j], dummy);
      ac[j] += p * 16;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = q & 1;
      const int p = (lane & 7) ^ (4 * j + (ci >> 1));
      b_row<MODE>(a, t, (2 * wv + (q >> 1)) * 16 + 8 * j + ci, bc[q], dummy);
      bc[q] += p * 16;
    }
    const uint8_t* c;
    if (wv < 2) a_row<MODE>(a, t, t.row0 + wv * 64 + lane, c, ssrc);
    else if (wv < 6) b_row<MODE>(a, t, (wv - 2) * 64 + lane, c, ssrc);
  }
  // Double step m = K steps 2m, 2m+1 = code bytes [128 m, 128 m + 128) of a
  // row.  Every wave issues 6 code copies per double step; on even m, waves
  // 0-5 first copy scale group m / 2 (K steps 2m .. 2m+3, row bytes
  // [16 (m/2), +16)), real steps only: copies complete in issue order, so the
  // codes' count covers it.
  auto issue = [&](int m, WStage& S, bool real) {
    if (real && (m & 1) == 0 && wv < 6) {
      ScaleGroup& G = ((m >> 1) & 1) ? sg1 : sg0;
      if (wv < 2) dma16(ssrc + (m >> 1) * 16, &G.as[wv * 64]);
      else dma16(ssrc + (m >> 1) * 16, &G.bs[(wv - 2) * 64]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(ac[j] + m * 128, &S.a[(wv * 2 + j) * 64]);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(bc[q] + m * 128, &S.b[((2 * wv + (q >> 1)) * 2 + (q & 1)) * 64]);
  };
  constexpr int kWCopies = 6;

  // fragment slot of this lane in its slice (uint4 units) for sub-step u:
  // row fr = 8 j + i, piece 4 u + fk
  uint32_t fo[2];
  {
    const int j = fr >> 3, i = fr & 7;
#pragma unroll
    for (int u = 0; u < 2; ++u) fo[u] = j * 64 + 8 * i + ((4 * u + fk) ^ (4 * j + (i >> 1)));
  }

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WStage& S, int m) {
    const ScaleGroup& G = ((m >> 1) & 1) ? sg1 : sg0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t so = ((2 * m + u) & 3) * 4;   // the step's dword in a row's 16 bytes
      uint32_t aq[4], as[4], bq[4], bs[4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int sl = wm * 4 + ms;
        aq[ms] = lds_addr(&S.a[sl * 128 + fo[u]]);
        as[ms] = lds_addr(&G.as[sl * 16 + fr]) + so;
      }
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const int sl = b_slice<MODE>(wn, ns);
        bq[ns] = lds_addr(&S.b[sl * 128 + fo[u]]);
        bs[ns] = lds_addr(&G.bs[sl * 16 + fr]) + so;
      }
      mma_step<MODE>(aq, as, bq, bs, fk, acc);
    }
  };

  const int nd = K / 256;                      // K % 512 == 0: nd even, >= 2
  issue(0, ws0, true);
  issue(1, ws1, true);
  for (int m0 = 0; m0 < nd; m0 += kWStages) {
#pragma unroll
    for (int s = 0; s < kWStages; ++s) {
      const int m = m0 + s;
      if (m < nd) {
        // this wave's copies of double step m are done once at most the next
        // one's are outstanding; the barrier makes every wave's copies
        // visible and frees the buffers double step m-1 used
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kWStages - 2) * kWCopies) : "memory");
        __builtin_amdgcn_s_barrier();
        const int mn = m + kWStages - 1;
        issue(mn < nd ? mn : nd - 1, stage((s + kWStages - 1) % kWStages), mn < nd);
        compute(stage(s), m);
      }
    }
  }
  gemm_epilogue<MODE>(a, t, acc, wm, wn, lane);
}

// ---- 7: combine ------------------------------------------------------------------
// y[t][c] = sum_j w[t][j] * partial[t][j][c] over resident pairs, in j order,
// plus the shared expert's row with weight 1.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_of,
                                                      int T, int H, int E, int k,
                                                      int has_shared, float* __restrict__ y) {
  const int nv = H / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * nv) return;
  const int t = (int)(gid / nv), c4 = (int)(gid % nv);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4* pr = reinterpret_cast<const float4*>(partial) + (int64_t)t * (k + 1) * nv + c4;
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    if (e < 0 || e >= E) continue;
    if (slot_of && slot_of[e] < 0) continue;
    const float g = w[t * k + j];
    const float4 v = pr[(int64_t)j * nv];
    acc.x = fmaf(g, v.x, acc.x); acc.y = fmaf(g, v.y, acc.y);
    acc.z = fmaf(g, v.z, acc.z); acc.w = fmaf(g, v.w, acc.w);
  }
  if (has_shared) {
    const float4 v = pr[(int64_t)k * nv];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  reinterpret_cast<float4*>(y)[(int64_t)t * nv + c4] = acc;
}

// ---- debug: one 16x16 tile of A (16 x 128) . B (16 x 128)^T through the same
// fragment loaders and MFMA wrapper as the GEMMs; out is [16][16] row-major.
__global__ __launch_bounds__(64) void mfma_tile_kernel(const uint8_t* ac, const uint8_t* as,
                                                       const uint8_t* bc, const uint8_t* bs,
                                                       float* out) {
  const int lane = threadIdx.x;
  const int r = lane & 15;
  const Frag fa = load_frag(ac + r * 64, as + r * 4, 0, true);
  const Frag fb = load_frag(bc + r * 64, bs + r * 4, 0, true);
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  acc = mfma_fp4(fa, fb, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[d_row(lane, i) * 16 + d_col(lane)] = acc[i];
}

}  // namespace

int prefill_max_tiles(int T, int k, int E) {
  const int64_t pairs = (int64_t)T * (k + 1);
  return (int)((pairs + kMT - 1) / kMT + E + 1);
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t st) {
  hipError_t err;
  const int nb = p.E + 1;
  const int has_shared = p.shared != nullptr;
  const int n_pairs = p.T * p.k + (has_shared ? p.T : 0);

  // 1 quantise x (MXFP4 weights; NVFP4 GEMMs take x as given)
  if (!p.nvfp4) {
    const int64_t n = (int64_t)p.T * (p.H / 32);
    hipLaunchKernelGGL(quant_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(p.x), p.T, p.H, p.xq_codes, p.xq_scales);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  SortArgs s;
  s.ids = p.ids; s.slot_of = p.slot_of; s.T = p.T; s.k = p.k; s.E = p.E;
  s.has_shared = has_shared; s.n_pairs = n_pairs; s.n_chunks = p.n_chunks;
  s.max_tiles = p.max_tiles; s.chunk_counts = p.chunk_counts; s.seg_start = p.seg_start;
  s.tiles = p.tiles; s.sorted_pair = p.sorted_pair;
  hipLaunchKernelGGL(sort_count_kernel, dim3(p.n_chunks), dim3(256), nb * sizeof(int), st, s);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(1024), 2 * nb * sizeof(int), st, s);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(p.n_chunks), dim3(256), 0, st, s);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  if (p.nvfp4) {
    NvPrefillArgs g;
    g.slot_of = p.slot_of; g.pool = static_cast<const uint8_t*>(p.pool);
    g.shared = static_cast<const uint8_t*>(p.shared); g.expert_bytes = p.expert_bytes;
    for (int i = 0; i < 6; ++i) g.off[i] = p.off[i];
    g.goff = p.goff;
    g.T = p.T; g.H = p.H; g.I = p.I; g.E = p.E; g.k = p.k;
    g.seg_start = p.seg_start; g.tiles = p.tiles; g.sorted_pair = p.sorted_pair;
    g.x = static_cast<const uint16_t*>(p.x);
    g.hb = reinterpret_cast<uint16_t*>(p.hq_codes);
    g.partial = p.partial;
    if ((err = launch_prefill_nvfp4_gemms(g, p.max_tiles, st)) != hipSuccess) return err;
  } else {
  GemmArgs g;
  g.slot_of = p.slot_of; g.pool = static_cast<const uint8_t*>(p.pool);
  g.shared = static_cast<const uint8_t*>(p.shared); g.expert_bytes = p.expert_bytes;
  for (int i = 0; i < 6; ++i) g.off[i] = p.off[i];
  g.T = p.T; g.H = p.H; g.I = p.I; g.E = p.E; g.k = p.k;
  g.seg_start = p.seg_start; g.tiles = p.tiles; g.sorted_pair = p.sorted_pair;
  g.xq_codes = p.xq_codes; g.xq_scales = p.xq_scales; g.hq_codes = p.hq_codes;
  g.hq_scales = p.hq_scales; g.partial = p.partial;
  {
    const int groups = (p.max_tiles + 7) / 8;
    const int nt1 = p.I / (kBN / 2), nt2 = (p.H + kBN - 1) / kBN;
    // K a multiple of 512: two-step buffers, whole-line copies, grouped scales
    if (p.H % 512 == 0)
      hipLaunchKernelGGL(gemm_wide_kernel<1>, dim3(groups * 8 * nt1), dim3(kGemmThreads), 0, st,
                         g);
    else
      hipLaunchKernelGGL(gemm_kernel<1>, dim3(groups * 8 * nt1), dim3(kGemmThreads), 0, st, g);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (p.I % 512 == 0)
      hipLaunchKernelGGL(gemm_wide_kernel<2>, dim3(groups * 8 * nt2), dim3(kGemmThreads), 0, st,
                         g);
    else
      hipLaunchKernelGGL(gemm_kernel<2>, dim3(groups * 8 * nt2), dim3(kGemmThreads), 0, st, g);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  {
    const int64_t n = (int64_t)p.T * (p.H / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       p.partial, p.ids, p.w, p.slot_of, p.T, p.H, p.E, p.k, has_shared, p.y);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_mfma_fp4_tile(const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales, float* out,
                                hipStream_t st) {
  hipLaunchKernelGGL(mfma_tile_kernel, dim3(1), dim3(64), 0, st, a_codes, a_scales, b_codes,
                     b_scales, out);
  return hipGetLastError();
}

}  // namespace moe

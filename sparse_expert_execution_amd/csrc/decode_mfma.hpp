// decode_mfma.hpp - the one-kernel decode for MXFP4 experts on CDNA4's
// scaled FP4 matrix instruction (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// Same layer, same phases and hand-offs as decode_kernel (decode_impl.hpp):
// router, top-k and the expert list are shared code; what differs is how an
// expert row meets its activations.  The vector form spends about two
// instructions per weight element on unpacking e2m1 codes and on dot
// products, plus the bookkeeping of one row per wave, and at decode sizes
// that, not HBM, sets its pace.  Here one instruction takes 16 weight rows
// x 128 elements of K with their e8m0 scales as stored (operand A, FP4), and
// the activations of up to 16 tokens (operand B, FP8 e4m3 with an e8m0 scale
// per 32): the unpacking and the scaling are done by the matrix core.
//
// The activations must be FP8 there, so each is split into e4m3 parts
// under one power-of-two scale per block of 32: hi = RNE(v / 2^e), the
// remainder (exact in fp32) times 16 as the next part, and so on.  Two parts
// hold a BF16 x exactly (8 significant bits, 4 per part) unless an element
// is below the block's largest by 2^-15 or more; h (fp32) gets three parts,
// about 12 significant bits.  The products are exact and the matrix core
// accumulates in fp32.
//
// Operand layouts (probes of the instruction on gfx950, FP4 A with FP8 B):
// lane l supplies A row l % 16 and the 32 consecutive elements 32 (l / 16)
// ... of the instruction's 128 K (16 bytes of codes and that block's scale).
// B column l % 16 takes, in its 32 bytes, K elements 16 (l / 16) + [0, 16)
// and 64 + 16 (l / 16) + [0, 16), but the B scale a product takes is the one
// in the lane group of its A element, i.e. of the element's natural block of
// 32: activations are quantised in natural blocks of 32, the scale of block
// b sits in lane group b, and each block's two 16-byte halves go where the
// pairing asks.  D: lane l holds rows 4 (l / 16) + i, column l % 16.
//
// Loads that cover half of a 128-byte line read at half the rate of whole
// lines (a probe: 16 rows x 64 B per instruction 2.6 TB/s, 8 rows x 128 B
// 4.6 TB/s).  So one instruction takes 8 weight rows x 256 elements (two
// 128-element chunks, one line per row): A row m is weight row m % 8 on
// chunk m / 8, B column n is token n % 8 on chunk n / 8, and the blocks of
// D where the two chunks agree hold each row's two half sums; the other
// two blocks are discarded.  Up to 8 tokens per launch.
//
// Work: a layer's row groups (8 rows of a matrix of one expert) are split
// over the workgroups, gate/up in whole multiples of 8 groups and down by
// cost (a unit's groups weigh more the more entries it has); a workgroup's
// groups go to its eight waves whole when it has a multiple of 8 of them,
// else by slices of K (each wave takes one slice of every group) whose sums
// meet in LDS through LDS float atomics.  A wave keeps kMfRing steps of
// weight loads in flight (one row group, two chunks, each; down 2 kMfRing
// where it loads a scale dword per step).
#pragma once

namespace moe {
namespace dec {

constexpr int kUnionBytes = (kXStage16 + kHStage4) * 16;
constexpr int kMfRing = 8;     // steps of loads in flight per wave
constexpr int kHParts = 3;     // e4m3 parts of h
constexpr int kZsBytes = 1024; // logits of the rank top-k (T * E <= 128, rows padded to 4)

// ---- byte offsets in the LDS union ------------------------------------------
// gate/up: BF16 x for the router at 0 (the layout of stage_x), the e4m3 parts
// of x after it, their scales, the rank logits; the gate/up sums reuse the
// BF16 stage once the router is done
__device__ __forceinline__ int mf_xq(const DecArgs& a) { return a.T * a.H * 2; }
__device__ __forceinline__ int mf_xsc(const DecArgs& a) { return a.T * a.H * 4; }
__device__ __forceinline__ int mf_zs(const DecArgs& a) {
  return (a.T * a.H * 4 + a.T * a.H / 16 + 15) & ~15;
}
// row groups of one gate/up batch: gate and up sums of 8 rows x T tokens
__device__ __forceinline__ int mf_gu_batch(const DecArgs& a) {
  const int n = a.H / 32;
  return n < kMfTab ? n : kMfTab;
}
// down: e4m3 parts of h of a unit's ne entries, then their scales
__device__ __forceinline__ int mf_hsc(const DecArgs& a, int ne) { return ne * a.I * kHParts; }

// LDS-only barrier: LDS writes done, every wave here; loads in flight stay
// in flight
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- e4m3 parts ---------------------------------------------------------------
// exponent e of a block's scale 2^e: largest |v| / 2^e <= 448 (the largest
// e4m3), kept where the later parts' scales (e - 4, e - 8) stay e8m0 values
__device__ __forceinline__ int part_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  int e = (int)((b >> 23) & 0xffu) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  e = e < -118 ? -118 : e;
  return e > 126 ? 126 : e;
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// two floats to e4m3 (RNE, OCP), into the low (HI false) or high 16 bits of old
template <bool HI>
__device__ __forceinline__ int to_e4m3x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// e4m3 bytes 0, 1 (HI false) or 2, 3 of w as floats
template <bool HI>
__device__ __forceinline__ v2f from_e4m3x2(int w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Split v[32] (already divided by 2^e) into P e4m3 parts: part p of element i
// in byte i of out[p][0..7]; v is left holding the last remainder.
template <int P>
__device__ __forceinline__ void split_parts(float v[32], uint32_t out[P][8]) {
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      int w = to_e4m3x2<false>(v[4 * d], v[4 * d + 1], 0);
      w = to_e4m3x2<true>(v[4 * d + 2], v[4 * d + 3], w);
      out[p][d] = (uint32_t)w;
      if (p + 1 < P) {
        const v2f lo = from_e4m3x2<false>(w), hi = from_e4m3x2<true>(w);
        v[4 * d] = (v[4 * d] - lo.x) * 16.f;
        v[4 * d + 1] = (v[4 * d + 1] - lo.y) * 16.f;
        v[4 * d + 2] = (v[4 * d + 2] - hi.x) * 16.f;
        v[4 * d + 3] = (v[4 * d + 3] - hi.y) * 16.f;
      }
    }
  }
}

// Write the P parts of natural block kb of chunk c, column col, into a B
// stage with np parts: its 16-element halves go to lane groups 2 (kb & 1) and
// 2 (kb & 1) + 1 at byte 16 (kb >> 1) of their 32; its scale exponent e (part
// p: e - 4p) to lane group kb
template <int P>
__device__ __forceinline__ void put_block(uint8_t* q, uint8_t* sc, int c, int kb, int col,
                                          int ncol, const uint32_t parts[P][8], int e) {
  const int off = 16 * (kb >> 1), g0 = 2 * (kb & 1);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int i0 = ((c * P + p) * 4 + g0) * ncol + col;
    const int i1 = ((c * P + p) * 4 + g0 + 1) * ncol + col;
    *reinterpret_cast<uint4*>(q + (i0 << 5) + off) =
        make_uint4(parts[p][0], parts[p][1], parts[p][2], parts[p][3]);
    *reinterpret_cast<uint4*>(q + (i1 << 5) + off) =
        make_uint4(parts[p][4], parts[p][5], parts[p][6], parts[p][7]);
    sc[((c * P + p) * 4 + kb) * ncol + col] = (uint8_t)(127 + e - 4 * p);
  }
}

__device__ __forceinline__ float bf16_f(uint32_t w, bool hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

// x of every token as two e4m3 parts in the B order (header comment): part
// p of chunk c, lane group g, token t is 32 bytes at
// xq + (((c * 2 + p) * 4 + g) * T + t) * 32, its scale byte at
// xsc[((c * 2 + p) * 4 + g) * T + t].  Read from global memory, so it runs
// beside the router's use of the BF16 stage.
__device__ __forceinline__ void stage_xq(const DecArgs& a, uint8_t* U) {
  const int T = a.T, H = a.H, C = H / 128;
  uint8_t* xq = U + mf_xq(a);
  uint8_t* xsc = U + mf_xsc(a);
  const int nb = T * C * 4;
  for (int b = threadIdx.x; b < nb; b += kT) {
    const int t = b / (C * 4), r = b - t * (C * 4), c = r >> 2, kb = r & 3;
    const uint4* src = reinterpret_cast<const uint4*>(a.x + (int64_t)t * H + c * 128 + 32 * kb);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = ldg16(src + i);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_f(ww[j], false);
        v[8 * i + 2 * j + 1] = bf16_f(ww[j], true);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int e = part_exp(amax);
    const float inv = pow2f(-e);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= inv;
    uint32_t q[2][8];
    split_parts<2>(v, q);
    put_block<2>(xq, xsc, c, kb, t, T, q, e);
  }
}

// ---- the matrix instruction -------------------------------------------------
__device__ __forceinline__ v4f mfma_fp4_fp8(uint4 a, uint32_t sa, const v8i& b, uint32_t sb,
                                            v4f c) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4, 0, 0, (int)sa, 0,
                                                          (int)sb);
}

// B fragments from a stage of np parts and ncol items: lane column n =
// lane % 16 is item n % 8 on chunk 2 cp + n / 8.  A column past the items
// reads the last item (its D column is discarded), so every lane loads and
// no register is cleared per step; the lane's offsets are fixed, the chunk
// pair's part is uniform.
struct BLane {
  uint32_t off;     // index of the lane's 32-byte block for chunk pair 0, part 0
  uint32_t step;    // blocks per part (4 * ncol); per chunk pair: 2 * np * step
};

__device__ __forceinline__ BLane b_lane(int np, int ncol) {
  const int lane = threadIdx.x & 63, h = (lane >> 3) & 1, g = lane >> 4;
  const int col = (lane & 7) < ncol ? (lane & 7) : ncol - 1;
  BLane o;
  o.step = (uint32_t)(4 * ncol);
  o.off = (uint32_t)((h * np * 4 + g) * ncol + col);
  return o;
}

__device__ __forceinline__ void b_frag(const uint8_t* q, const uint8_t* sc, const BLane& L, int cp,
                                       int p, int np, v8i& b, uint32_t& s) {
  const uint32_t i = (uint32_t)((2 * cp * np + p) * L.step) + L.off;
  b = *reinterpret_cast<const v8i*>(q + (i << 5));
  s = sc[i];
}

// The lane's part of an A operand: row row0 + lane % 8 of a matrix with K
// elements per row, 16 bytes of chunk 2 cp + (lane / 8) % 2 at block lane /
// 16 (one 128-byte line per row per instruction), and the dword of the row's
// scales holding that block's byte.  The lane's byte offsets are fixed; the
// row group's base and the chunk pair are uniform.
struct ALane {
  uint32_t code, scale;
};

__device__ __forceinline__ ALane a_lane(int K) {
  const int lane = threadIdx.x & 63, h = (lane >> 3) & 1, g = lane >> 4, r = lane & 7;
  ALane o;
  o.code = (uint32_t)(r * (K / 2) + h * 64 + g * 16);
  o.scale = (uint32_t)(r * (K / 32) + h * 4);
  return o;
}

// base of a row group of one matrix: its codes and its scales
struct MPtr {
  const uint8_t* code;
  const uint8_t* scale;
};

__device__ __forceinline__ MPtr m_ptr(const uint8_t* base, int64_t off_code, int64_t off_scale,
                                      int row0, int K) {
  MPtr p;
  p.code = base + off_code + (int64_t)row0 * (K / 2);
  p.scale = base + off_scale + (int64_t)row0 * (K / 32);
  return p;
}

__device__ __forceinline__ void a_load(const MPtr& p, const ALane& L, int cp, uint4& q,
                                       uint32_t& s) {
  q = ldg16(p.code + cp * 128 + L.code);
  s = *reinterpret_cast<const uint32_t*>(p.scale + cp * 8 + L.scale);
}

// the lane's scale byte of its A operand
__device__ __forceinline__ uint32_t a_scale(uint32_t w) {
  return (w >> (8 * ((threadIdx.x & 63) >> 4))) & 0xffu;
}

// D values of lane l that belong to a row: the diagonal blocks (A chunk
// equals B chunk), rows 4 ((l / 16) % 2) + i of the group, item l % 8
__device__ __forceinline__ bool d_diag() {
  const int lane = threadIdx.x & 63;
  return ((lane >> 5) & 1) == ((lane >> 3) & 1);
}
__device__ __forceinline__ int d_row8(int i) { return 4 * (((threadIdx.x & 63) >> 4) & 1) + i; }

// ---- work split of one batch over the waves -----------------------------------
// n row groups, C chunk pairs of K: S slices of K (a power of two, S * n a
// multiple of 8 when C allows) and wave w takes slice w % S of groups
// w / S, w / S + 8 / S, ..., one group at a time over its slice
struct MfSplit {
  int st, o;        // group stride and first group of this wave
  int cl, nc;       // first chunk pair of its slice and the slice's chunk pairs
  int cnt;          // its groups
};

__device__ __forceinline__ MfSplit mf_split(int n, int C) {
  int g8 = n & 7 ? (n & 3 ? (n & 1 ? 1 : 2) : 4) : 8;   // gcd(n, 8)
  int S = 8 / g8;
  while (S > C) S >>= 1;
  const int wave = uni((int)(threadIdx.x >> 6));
  MfSplit m;
  m.st = 8 / S;
  m.o = wave / S;
  const int s = wave % S;
  m.cl = s * C / S;
  m.nc = (s + 1) * C / S - m.cl;
  m.cnt = m.o < n ? (n - m.o + m.st - 1) / m.st : 0;
  return m;
}

// cursor over a wave's steps: its r-th group, chunk pair c; past the last
// step it stays there (the loads ahead then repeat the last step's)
struct MfCur {
  int r, c;
};

__device__ __forceinline__ bool cur_next(const MfSplit& m, MfCur& k) {
  if (k.c + 1 < m.cl + m.nc) {
    k.c = uni(k.c + 1);
    return false;
  }
  if (k.r + 1 < m.cnt) {
    k.r = uni(k.r + 1);
    k.c = m.cl;
    return true;                          // a new group
  }
  return false;
}

__device__ __forceinline__ int cur_group(const MfSplit& m, const MfCur& k) {
  return m.o + m.st * k.r;
}

// ---- gate/up ------------------------------------------------------------------
struct MfGuStep {
  uint4 g, u;
  uint32_t gs, us;
};

struct MfGuPtr {
  MPtr g, u;
};

__device__ __forceinline__ MfGuPtr gu_ptr(const DecArgs& a, const DecLds& S, int q) {
  const uint8_t* base = unit_base(a, uni(S.p.mf_slot[q]));
  const int row0 = uni(S.p.mf_row[q]);
  MfGuPtr p;
  p.g = m_ptr(base, a.off[0], a.off[1], row0, a.H);
  p.u = m_ptr(base, a.off[2], a.off[3], row0, a.H);
  return p;
}

// One batch of n gate/up row groups (table S.p.mf_*), sums into the LDS
// accumulators acc[((j * 2 + m) * 8 + row) * T + t], which start at zero.
// Every step issues the same loads (past the end they repeat the last), so
// that the waits for a step's data are counted, not a drain of every load
// in flight.
// Gate/up with the A scales of a row group loaded once per pass of kMfRing
// steps instead of one dword per step (the step's scale load cost as much as
// its code load: a timing variant without scale loads was 7 us faster per
// DeepSeek-shaped call at four tokens).  Lane l loads 16 scale bytes of row
// l % 8 at byte 16 (l / 8) (NS loads per row: H / 32 bytes), so a row's
// line comes whole; the dword a lane needs at step cp (2 cp + h of its row,
// h = (l / 8) % 2) sits in lane row + 8 ((cp / 2) % 8), register 2 (cp % 2)
// + h of load cp / 16, and ds_bpermute hands it over.  Needs each wave's
// groups to run whole passes (nc a multiple of kMfRing): a pass then lies in
// one group, and the loads of pass p + 1 go out at the first reload of pass
// p into the set pass p - 1 used (two sets, passes unrolled in pairs).
struct MfGuCode {
  uint4 g, u;
};

template <int NS>
struct MfGuScales {
  uint4 g[NS], u[NS];
};

template <int NS>
__device__ __forceinline__ void gu_batch_gs(const DecArgs& a, DecLds& S, uint8_t* U,
                                            const MfSplit& m, int nsteps, float* acc) {
  const int lane = threadIdx.x & 63, col = lane & 7;
  const int T = a.T, SB = a.H / 32;
  const uint8_t* xq = U + mf_xq(a);
  const uint8_t* xsc = U + mf_xsc(a);
  const ALane L = a_lane(a.H);
  const BLane BL = b_lane(2, T);
  uint32_t so[NS];                        // this lane's scale bytes (past the row: its start)
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int b = 128 * j + 16 * (lane >> 3);
    so[j] = (uint32_t)((lane & 7) * SB + (b < SB ? b : 0));
  }
  const int hb = (lane >> 3) & 1;
  MfCur lc{0, m.cl}, cc{0, m.cl};
  MfGuPtr lp = gu_ptr(a, S, cur_group(m, lc));
  auto load_scales = [&](MfGuScales<NS>& z) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      z.g[j] = ldg16(lp.g.scale + so[j]);
      z.u[j] = ldg16(lp.u.scale + so[j]);
    }
  };
  auto load_codes = [&](MfGuCode& c) {
    c.g = ldg16(lp.g.code + lc.c * 128 + L.code);
    c.u = ldg16(lp.u.code + lc.c * 128 + L.code);
    if (cur_next(m, lc)) lp = gu_ptr(a, S, cur_group(m, lc));
  };
  // the lane's scale byte at chunk pair cp from a set
  auto pick = [&](const uint4 (&w)[NS], int cp) -> uint32_t {
    const uint4 v = NS > 1 && cp >= 16 ? w[NS - 1] : w[0];
    const int src = ((lane & 7) + 8 * ((cp >> 1) & 7)) * 4;
    const uint32_t lo = (cp & 1) ? v.z : v.x, hi = (cp & 1) ? v.w : v.y;
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)lo);
    const uint32_t d1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)hi);
    return a_scale(hb ? d1 : d0);
  };
  MfGuScales<NS> z0, z1;
  load_scales(z0);
  MfGuCode ring[kMfRing];
#pragma unroll
  for (int i = 0; i < kMfRing; ++i) load_codes(ring[i]);
  v4f ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
  const bool mine = d_diag() && col < T;
  // one pass: steps p0 .. p0 + kMfRing - 1 with scale set z, the next
  // pass's set loaded into zn at its first reload
  auto pass = [&](int p0, const MfGuScales<NS>& z, MfGuScales<NS>& zn) {
#pragma unroll
    for (int i = 0; i < kMfRing; ++i) {
      if (p0 + i < nsteps) {
        v8i b0, b1;
        uint32_t s0b, s1b;
        b_frag(xq, xsc, BL, cc.c, 0, 2, b0, s0b);
        b_frag(xq, xsc, BL, cc.c, 1, 2, b1, s1b);
        const uint32_t sg = pick(z.g, cc.c), su = pick(z.u, cc.c);
        ag = mfma_fp4_fp8(ring[i].g, sg, b0, s0b, ag);
        ag = mfma_fp4_fp8(ring[i].g, sg, b1, s1b, ag);
        au = mfma_fp4_fp8(ring[i].u, su, b0, s0b, au);
        au = mfma_fp4_fp8(ring[i].u, su, b1, s1b, au);
        if (cc.c == m.cl + m.nc - 1) {      // the group's last step: add its sums
          const int q = cur_group(m, cc);
          if (mine) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = d_row8(r);
              atomicAdd(acc + ((q * 2 + 0) * 8 + row) * T + col, ag[r]);
              atomicAdd(acc + ((q * 2 + 1) * 8 + row) * T + col, au[r]);
            }
          }
          ag = au = v4f{0.f, 0.f, 0.f, 0.f};
        }
        cur_next(m, cc);
      }
      if (i == 0) load_scales(zn);           // pass p0 + kMfRing: the cursor is there
      load_codes(ring[i]);                   // step p0 + i + kMfRing
    }
  };
  for (int s0 = 0; s0 < nsteps; s0 += 2 * kMfRing) {
    pass(s0, z0, z1);
    if (s0 + kMfRing >= nsteps) break;
    pass(s0 + kMfRing, z1, z0);
  }
}

__device__ __forceinline__ void gu_batch(const DecArgs& a, DecLds& S, uint8_t* U, int n,
                                         float* acc) {
  const int lane = threadIdx.x & 63, col = lane & 7;
  const int T = a.T, C2 = a.H / 256;
  const uint8_t* xq = U + mf_xq(a);
  const uint8_t* xsc = U + mf_xsc(a);
  const MfSplit m = mf_split(n, C2);
  const int nsteps = m.cnt * m.nc;
  if (nsteps == 0) return;
  if (m.nc % kMfRing == 0 && a.H <= 4096) return gu_batch_gs<1>(a, S, U, m, nsteps, acc);
  if (m.nc % kMfRing == 0 && a.H <= 8192) return gu_batch_gs<2>(a, S, U, m, nsteps, acc);
  const ALane L = a_lane(a.H);
  const BLane BL = b_lane(2, T);
  MfCur lc{0, m.cl}, cc{0, m.cl};
  MfGuPtr lp = gu_ptr(a, S, cur_group(m, lc));
  MfGuStep ring[kMfRing];
#pragma unroll
  for (int i = 0; i < kMfRing; ++i) {
    a_load(lp.g, L, lc.c, ring[i].g, ring[i].gs);
    a_load(lp.u, L, lc.c, ring[i].u, ring[i].us);
    if (cur_next(m, lc)) lp = gu_ptr(a, S, cur_group(m, lc));
  }
  v4f ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
  const bool mine = d_diag() && col < T;
  for (int s0 = 0; s0 < nsteps; s0 += kMfRing) {
#pragma unroll
    for (int i = 0; i < kMfRing; ++i) {
      if (s0 + i < nsteps) {
        v8i b0, b1;
        uint32_t s0b, s1b;
        b_frag(xq, xsc, BL, cc.c, 0, 2, b0, s0b);
        b_frag(xq, xsc, BL, cc.c, 1, 2, b1, s1b);
        const uint32_t sg = a_scale(ring[i].gs), su = a_scale(ring[i].us);
        ag = mfma_fp4_fp8(ring[i].g, sg, b0, s0b, ag);
        ag = mfma_fp4_fp8(ring[i].g, sg, b1, s1b, ag);
        au = mfma_fp4_fp8(ring[i].u, su, b0, s0b, au);
        au = mfma_fp4_fp8(ring[i].u, su, b1, s1b, au);
        if (cc.c == m.cl + m.nc - 1) {      // the group's last step: add its sums
          const int q = cur_group(m, cc);
          if (mine) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = d_row8(r);
              atomicAdd(acc + ((q * 2 + 0) * 8 + row) * T + col, ag[r]);
              atomicAdd(acc + ((q * 2 + 1) * 8 + row) * T + col, au[r]);
            }
          }
          ag = au = v4f{0.f, 0.f, 0.f, 0.f};
        }
        cur_next(m, cc);
      }
      a_load(lp.g, L, lc.c, ring[i].g, ring[i].gs);   // step s0 + i + kMfRing
      a_load(lp.u, L, lc.c, ring[i].u, ring[i].us);
      if (cur_next(m, lc)) lp = gu_ptr(a, S, cur_group(m, lc));
    }
  }
}

// h = silu(g) * u of the batch's groups for each entry of their units
// (SHARED: the shared expert, all T tokens), tagged with the generation;
// the accumulators are cleared for the next batch
template <bool SHARED>
__device__ __forceinline__ void gu_out(const DecArgs& a, const DecLds& S, int n, float* acc) {
  const int T = a.T, I = a.I;
  for (int q = threadIdx.x; q < n * 8; q += kT) {
    const int j = q >> 3, row = q & 7;
    const int u = S.p.mf_unit[j];
    const int i = S.p.mf_row[j] + row;
    const int e0 = SHARED ? 0 : S.p.unit_start[u];
    const int ne = SHARED ? T : S.p.unit_start[u + 1] - e0;
    for (int e = 0; e < ne; ++e) {
      const int t = SHARED ? e : S.p.ent_tok[e0 + e];
      const int pair = SHARED ? a.T * a.k + e : S.p.ent_pair[e0 + e];
      const float gv = acc[((j * 2 + 0) * 8 + row) * T + t];
      const float uv = acc[((j * 2 + 1) * 8 + row) * T + t];
      const float h = gv / (1.0f + expf(-gv)) * uv;
      __hip_atomic_store(a.h + (int64_t)pair * I + i,
                         ((uint64_t)a.gen << 32) | __float_as_uint(h), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int t = 0; t < T; ++t) {
      acc[((j * 2 + 0) * 8 + row) * T + t] = 0.f;
      acc[((j * 2 + 1) * 8 + row) * T + t] = 0.f;
    }
  }
}

// Gate/up of row groups [g0, g1) of the flattened (unit, 8 rows of I) list
// (SHARED: groups of the shared expert), in batches.  Every wave of the
// workgroup calls it (it holds barriers).
template <bool SHARED>
__device__ __forceinline__ void mf_gateup(const DecArgs& a, DecLds& S, uint8_t* U, int g0,
                                          int g1) {
  float* acc = reinterpret_cast<float*>(U);
  const int GI = a.I / 8, NB = mf_gu_batch(a);
  for (int b0 = g0; b0 < g1; b0 += NB) {
    const int n = g1 - b0 < NB ? g1 - b0 : NB;
    for (int j = threadIdx.x; j < n; j += kT) {
      const int q = b0 + j;
      if (SHARED) {
        S.p.mf_slot[j] = -1;
        S.p.mf_row[j] = q * 8;
        S.p.mf_unit[j] = -1;
      } else {
        const int u = q / GI;
        S.p.mf_slot[j] = S.p.unit_slot[u];
        S.p.mf_row[j] = (q - u * GI) * 8;
        S.p.mf_unit[j] = u;
      }
    }
    lds_barrier();
    gu_batch(a, S, U, n, acc);
    lds_barrier();
    gu_out<SHARED>(a, S, n, acc);
    lds_barrier();
  }
}

// ---- down ---------------------------------------------------------------------
struct MfDnStep {
  uint4 q;
  uint32_t s;
};

__device__ __forceinline__ MPtr dn_ptr(const DecArgs& a, const DecLds& S, int q) {
  const uint8_t* base = unit_base(a, uni(S.p.mf_slot[q]));
  return m_ptr(base, a.off[4], a.off[5], uni(S.p.mf_row[q]), a.I);
}

// h of a unit's ne entries (from entry e0) as kHParts e4m3 parts in the B
// order (entries as columns, natural blocks as in stage_xq) at hq, its
// scales after them: values polled until they carry this launch's
// generation
__device__ __forceinline__ void stage_hq(const DecArgs& a, const DecLds& S, uint8_t* hq, int e0,
                                         int ne) {
  const int I = a.I, CI = I / 128;
  uint8_t* hsc = hq + mf_hsc(a, ne);
  const int nb = ne * CI * 4;
  for (int b = threadIdx.x; b < nb; b += kT) {
    const int e = b / (CI * 4), r = b - e * (CI * 4), c = r >> 2, kb = r & 3;
    const uint64_t* src = a.h + (int64_t)S.p.ent_pair[e0 + e] * I + c * 128 + 32 * kb;
    uint64_t w[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      w[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    for (;;) {
      bool all = true;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((unsigned)(w[i] >> 32) != a.gen) {
          all = false;
          w[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (all) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(a.hdr + kHError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = __uint_as_float((uint32_t)w[i]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    const int ex = part_exp(amax);
    const float inv = pow2f(-ex);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= inv;
    uint32_t q[kHParts][8];
    split_parts<kHParts>(v, q);
    put_block<kHParts>(hq, hsc, c, kb, e, ne, q, ex);
  }
}

// Down with a row group's A scales once per pass of kMfRing steps, as in
// gu_batch_gs (a ring of kMfRing steps, two scale sets; each wave's groups
// run whole passes).
template <int NS>
__device__ __forceinline__ void dn_batch_gs(const DecArgs& a, DecLds& S, uint8_t* U,
                                            const MfSplit& m, int nsteps, float* yacc) {
  const int lane = threadIdx.x & 63, col = lane & 7;
  const int T = a.T, SB = a.I / 32;
  const ALane L = a_lane(a.I);
  uint32_t so[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int b = 128 * j + 16 * (lane >> 3);
    so[j] = (uint32_t)((lane & 7) * SB + (b < SB ? b : 0));
  }
  const int hb = (lane >> 3) & 1;
  MfCur lc{0, m.cl}, cc{0, m.cl};
  MPtr lp = dn_ptr(a, S, cur_group(m, lc));
  auto load_scales = [&](uint4 (&z)[NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) z[j] = ldg16(lp.scale + so[j]);
  };
  auto load_codes = [&](uint4& q) {
    q = ldg16(lp.code + lc.c * 128 + L.code);
    if (cur_next(m, lc)) lp = dn_ptr(a, S, cur_group(m, lc));
  };
  auto pick = [&](const uint4 (&w)[NS], int cp) -> uint32_t {
    const uint4 v = NS > 1 && cp >= 16 ? w[NS - 1] : w[0];
    const int src = ((lane & 7) + 8 * ((cp >> 1) & 7)) * 4;
    const uint32_t lo = (cp & 1) ? v.z : v.x, hi = (cp & 1) ? v.w : v.y;
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)lo);
    const uint32_t d1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)hi);
    return a_scale(hb ? d1 : d0);
  };
  uint4 z0[NS], z1[NS];
  load_scales(z0);
  uint4 ring[kMfRing];
#pragma unroll
  for (int i = 0; i < kMfRing; ++i) load_codes(ring[i]);
  auto enter = [&](int q, const uint8_t*& hq, const uint8_t*& hsc, BLane& BL, int& ne) {
    ne = uni(S.p.unit_start[S.p.mf_unit[q] + 1] - S.p.unit_start[S.p.mf_unit[q]]);
    hq = U + uni(S.p.mf_hoff[q]);
    hsc = hq + mf_hsc(a, ne);
    BL = b_lane(kHParts, ne);
  };
  const uint8_t *hq, *hsc;
  BLane BL;
  int ne;
  enter(cur_group(m, cc), hq, hsc, BL, ne);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const bool diag = d_diag();
  auto pass = [&](int p0, const uint4 (&z)[NS], uint4 (&zn)[NS]) {
#pragma unroll
    for (int i = 0; i < kMfRing; ++i) {
      if (p0 + i < nsteps) {
        const uint32_t sa = pick(z, cc.c);
#pragma unroll
        for (int p = 0; p < kHParts; ++p) {
          v8i b;
          uint32_t sb;
          b_frag(hq, hsc, BL, cc.c, p, kHParts, b, sb);
          acc = mfma_fp4_fp8(ring[i], sa, b, sb, acc);
        }
        if (cc.c == m.cl + m.nc - 1) {
          const int q = cur_group(m, cc);
          if (diag && col < ne) {
#pragma unroll
            for (int r = 0; r < 4; ++r) atomicAdd(yacc + (q * 8 + d_row8(r)) * T + col, acc[r]);
          }
          acc = v4f{0.f, 0.f, 0.f, 0.f};
        }
        if (cur_next(m, cc)) enter(cur_group(m, cc), hq, hsc, BL, ne);
      }
      if (i == 0) load_scales(zn);
      load_codes(ring[i]);
    }
  };
  for (int s0 = 0; s0 < nsteps; s0 += 2 * kMfRing) {
    pass(s0, z0, z1);
    if (s0 + kMfRing >= nsteps) break;
    pass(s0 + kMfRing, z1, z0);
  }
}

// one batch of n down row groups (table S.p.mf_*: each group's unit, its h
// stage, its entry count): sums into yacc[(j * 8 + row) * T + e]; loads as
// in gu_batch
__device__ __forceinline__ void dn_batch(const DecArgs& a, DecLds& S, uint8_t* U, int n,
                                         float* yacc) {
  const int lane = threadIdx.x & 63, col = lane & 7;
  const int CI2 = a.I / 256, T = a.T;
  const MfSplit m = mf_split(n, CI2);
  const int nsteps = m.cnt * m.nc;
  if (nsteps == 0) return;
  if (m.nc % kMfRing == 0 && a.I <= 4096) return dn_batch_gs<1>(a, S, U, m, nsteps, yacc);
  if (m.nc % kMfRing == 0 && a.I <= 8192) return dn_batch_gs<2>(a, S, U, m, nsteps, yacc);
  const ALane L = a_lane(a.I);
  MfCur lc{0, m.cl}, cc{0, m.cl};
  MPtr lp = dn_ptr(a, S, cur_group(m, lc));
  MfDnStep ring[2 * kMfRing];
#pragma unroll
  for (int i = 0; i < 2 * kMfRing; ++i) {
    a_load(lp, L, lc.c, ring[i].q, ring[i].s);
    if (cur_next(m, lc)) lp = dn_ptr(a, S, cur_group(m, lc));
  }
  // the compute cursor's group: its h stage and entries
  auto enter = [&](int q, const uint8_t*& hq, const uint8_t*& hsc, BLane& BL, int& ne) {
    ne = uni(S.p.unit_start[S.p.mf_unit[q] + 1] - S.p.unit_start[S.p.mf_unit[q]]);
    hq = U + uni(S.p.mf_hoff[q]);
    hsc = hq + mf_hsc(a, ne);
    BL = b_lane(kHParts, ne);
  };
  const uint8_t *hq, *hsc;
  BLane BL;
  int ne;
  enter(cur_group(m, cc), hq, hsc, BL, ne);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const bool diag = d_diag();
  for (int s0 = 0; s0 < nsteps; s0 += 2 * kMfRing) {
#pragma unroll
    for (int i = 0; i < 2 * kMfRing; ++i) {
      if (s0 + i < nsteps) {
        const uint32_t sa = a_scale(ring[i].s);
#pragma unroll
        for (int p = 0; p < kHParts; ++p) {
          v8i b;
          uint32_t sb;
          b_frag(hq, hsc, BL, cc.c, p, kHParts, b, sb);
          acc = mfma_fp4_fp8(ring[i].q, sa, b, sb, acc);
        }
        if (cc.c == m.cl + m.nc - 1) {
          const int q = cur_group(m, cc);
          if (diag && col < ne) {
#pragma unroll
            for (int r = 0; r < 4; ++r) atomicAdd(yacc + (q * 8 + d_row8(r)) * T + col, acc[r]);
          }
          acc = v4f{0.f, 0.f, 0.f, 0.f};
        }
        if (cur_next(m, cc)) enter(cur_group(m, cc), hq, hsc, BL, ne);
      }
      a_load(lp, L, lc.c, ring[i].q, ring[i].s);
      if (cur_next(m, lc)) lp = dn_ptr(a, S, cur_group(m, lc));
    }
  }
}

// Down of row groups [g0, g1) of the flattened (unit, 8 rows of H) list:
// the h of every unit the range touches is staged at once (as many units
// as the LDS holds beside the y sums of one batch; a range touches one or
// two units at the pages' shapes), then the range's groups run in batches;
// results gate-weighted into y with fp32 atomics once every workgroup has
// cleared its slice of y.
__device__ __forceinline__ void mf_down(const DecArgs& a, DecLds& S, uint8_t* U, int g0, int g1,
                                        bool timing) {
  const int HG = a.H / 8, H = a.H, T = a.T;
  const int ybytes = kMfTab * 8 * T * 4;          // y sums of one batch (at most)
  bool y_clear = false;
  bool first = true;
  for (int s0 = g0; s0 < g1;) {
    // units [u0, u1) staged in this pass
    const int u0 = s0 / HG;
    int u1 = u0, off = 0;
    while (u1 * HG < g1) {
      const int ne = S.p.unit_start[u1 + 1] - S.p.unit_start[u1];
      const int sz = (mf_hsc(a, ne) + mf_hsc(a, ne) / 32 + 15) & ~15;
      if (u1 > u0 && off + sz + ybytes > kUnionBytes) break;
      off += sz;
      ++u1;
    }
    const int s1 = u1 * HG < g1 ? u1 * HG : g1;
    float* yacc = reinterpret_cast<float*>(U + off);
    const int NB = (kUnionBytes - off) / (8 * T * 4) < kMfTab ? (kUnionBytes - off) / (8 * T * 4)
                                                               : kMfTab;
    lds_barrier();                        // the previous stages are free
    {
      int o = 0;
      for (int u = u0; u < u1; ++u) {
        const int e0 = S.p.unit_start[u], ne = S.p.unit_start[u + 1] - e0;
        stage_hq(a, S, U + o, e0, ne);
        o += (mf_hsc(a, ne) + mf_hsc(a, ne) / 32 + 15) & ~15;
      }
    }
    for (int q = threadIdx.x; q < NB * 8 * T; q += kT) yacc[q] = 0.f;
    if (first) stamp(timing, a, 11);
    first = false;
    for (int b0 = s0; b0 < s1; b0 += NB) {
      const int n = s1 - b0 < NB ? s1 - b0 : NB;
      for (int j = threadIdx.x; j < n; j += kT) {
        const int gq = b0 + j, u = gq / HG;
        int o = 0;
        for (int v = u0; v < u; ++v) {
          const int ne = S.p.unit_start[v + 1] - S.p.unit_start[v];
          o += (mf_hsc(a, ne) + mf_hsc(a, ne) / 32 + 15) & ~15;
        }
        S.p.mf_slot[j] = S.p.unit_slot[u];
        S.p.mf_row[j] = (gq - u * HG) * 8;
        S.p.mf_unit[j] = u;
        S.p.mf_hoff[j] = o;
      }
      lds_barrier();
      dn_batch(a, S, U, n, yacc);
      lds_barrier();
      if (!y_clear) {
        const int lane = threadIdx.x & 63;
        if (threadIdx.x < 64) {
          const unsigned yz = lane < kNCtr ? __hip_atomic_load(a.hdr + kHYZero + lane * kLine,
                                                               __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT)
                                           : 0u;
          if (__builtin_amdgcn_readfirstlane((unsigned)wave_sum_dpp((float)yz)) < (unsigned)a.G)
            wait_count(a.hdr, a.hdr + kHYZero, (unsigned)a.G);
        }
        __syncthreads();
        y_clear = true;
      }
      for (int q = threadIdx.x; q < n * 8 * T; q += kT) {
        const int e = q % T, jr = q / T, j = jr >> 3;
        const int u = S.p.mf_unit[j], e0 = S.p.unit_start[u];
        if (e < S.p.unit_start[u + 1] - e0)
          unsafeAtomicAdd(a.y + (int64_t)S.p.ent_tok[e0 + e] * H + S.p.mf_row[j] + (jr & 7),
                          S.p.ent_gw[e0 + e] * yacc[q]);
        yacc[q] = 0.f;
      }
      // every thread is done with this batch's table (mf_unit, mf_row) before
      // the next batch's is written
      lds_barrier();
    }
    s0 = s1;
  }
  stamp(timing, a, 12);
}

// Down work split by cost.  A row group of a unit with ne entries costs
// about kDnA + kDnB * ne: its MFMA steps are the same for any ne (the B
// columns hold the entries), but its h stage, its B fragment reads (distinct
// columns instead of one broadcast column) and its y results grow with ne.
// On the DeepSeek-shaped layer at four tokens the shared expert's groups
// (ne = 4) took 1.31 times as long as single-entry ones; kDnA = 17, kDnB = 2
// gives 25 / 19 (cost_bound over the units' H / 8 groups).  Boundaries
// are rounded to whole multiples of 8 groups: a batch of a multiple of 8
// groups gives each wave whole groups (mf_split), anything else slices
// every group's K over the waves.  Against the even split of
// row groups: DeepSeek-shaped layer, 4 tokens 104 -> 99 us, 8 tokens 213 ->
// 192 us per launch.
constexpr int kDnA = 17, kDnB = 2;

__device__ __forceinline__ int mf_dn_bound(const DecArgs& a, const DecLds& S, int b, int G) {
  const int g = cost_bound(S.p, uni(S.p.n_units), a.H / 8, kDnA, kDnB, b, G);
  return uni((g + 4) & ~7);
}

// ---- the kernel ---------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(kT) void decode_mfma_kernel(DecArgs a) {
  __shared__ DecLds S;
  uint8_t* U = S.raw;
  const int wave = uni((int)(threadIdx.x >> 6));
  const int bid = blockIdx.x, G = a.G;
  const bool route = a.route != 0;
  const bool timing = a.hdr[kHTiming] != 0;
  const unsigned gen =
      __hip_atomic_load(a.hdr + kHGen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  a.gen = gen;
  stamp(timing, a, 0);

  // 1. router rows in flight, x staged twice (BF16 for the router, e4m3
  // parts for the matrix core), router dot products, y cleared
  RouterRow rw;
  const int item0 = bid + G * wave;
  if (route && item0 < router_items(a)) router_load(a, item0, 0, rw);
  stage_x<2>(a, S);
  stage_xq(a, U);
  __syncthreads();
  if (route) {
    router_items_run<2>(a, S, item0, rw, uni((int)gen));
    stamp(timing, a, 5);
  }
  {
    int64_t lo, hi;
    split((int64_t)a.T * a.H, G, bid, lo, hi);
    for (int64_t i = lo + threadIdx.x; i < hi; i += kT) coherent_store(a.y + i, 0.f);
  }
  lds_barrier();                          // the BF16 stage becomes the gate/up sums
  {
    float* acc = reinterpret_cast<float*>(U);
    const int n = mf_gu_batch(a) * 16 * a.T;   // gate and up, 8 rows, T tokens
    for (int i = threadIdx.x; i < n; i += kT) acc[i] = 0.f;
  }
  signal_done(a.hdr + kHYZero);
  stamp(timing, a, 8);

  // 2. the expert list
  build_units<M, kMaxCE, true>(a, S, route, timing, gen,
                               reinterpret_cast<float*>(U + mf_zs(a)));
  stamp(timing, a, 1);

  // 3. gate/up of every unit (the shared expert is the last one; in the
  // first phase its row groups would not spread evenly over the grid), in
  // whole multiples of 8 groups per workgroup (I / 8 is a multiple of 8):
  // each wave then takes whole groups, where any other count slices every
  // group's K over the waves and meets the slices in LDS atomics.  On the
  // DeepSeek-shaped layer this took 8 tokens from 192 to 160 us per launch
  // (at 4 tokens no change, at 2 tokens 66.8 -> 68.4 us: shares of 8 or 16
  // groups where the even split gave 13)
  {
    int64_t lo, hi;
    split((int64_t)S.p.n_units * (a.I / 64), G, bid, lo, hi);
    mf_gateup<false>(a, S, U, (int)lo * 8, (int)hi * 8);
  }
  stamp(timing, a, 7);

  // 4. down of every unit (h polled per value, no grid-wide wait), split
  // by cost rather than by row groups
  mf_down(a, S, U, mf_dn_bound(a, S, bid, G), mf_dn_bound(a, S, bid + 1, G), timing);
  stamp(timing, a, 3);
  finish_launch(a, gen);
}

// tokens one launch of the matrix-core decode takes (0: the shape has no
// such launch): at most 8 (B columns are 8 items x 2 chunks), and both the
// gate/up stages (BF16 x, its e4m3 parts and scales, the rank logits) and
// the down stages (h parts of one unit, sums of 8 row groups) must fit the
// LDS union
inline int mf_max_tokens(int H, int I) {
  if (H % 256 || I % 256) return 0;
  int t = 0;
  for (int T = 1; T <= 8; ++T) {
    const int gu = T * H * 4 + T * H / 16 + kZsBytes;
    const int dn = T * I * kHParts + T * I * kHParts / 32 + 16 + kMfTab * 8 * T * 4;
    if (gu > kUnionBytes || dn > kUnionBytes) break;
    t = T;
  }
  return t;
}

}  // namespace dec
}  // namespace moe

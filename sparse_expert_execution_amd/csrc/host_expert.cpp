// host_expert.cpp - the host side of the exact split: the expert FFNs of the
// (token, expert) pairs the GPU does not run, computed on the host cores
// straight from the pinned expert pool.
//
// A cache miss can stay where it lives and run on the host, whose partial sum
// is then merged exactly with the GPU's (explainx.ai guide, "Decode: decide
// whether to move an expert or compute where it lives"); the host side's rate
// is one of the two profiled bandwidths the q* split balances ("FreeToken
// 753b Model Explained", "Measure System Bandwidth").
//
// Same precision contract as moe_decode: x as given (BF16), fp32
// accumulation, h = silu(g) * u in fp32.  Work is split over a persistent
// pool of threads by rows: the gate/up rows of an expert, then its down rows
// (each thread owns whole output rows, so there are no atomics and the
// result does not depend on the thread count).  Row dots use AVX-512 or
// AVX2/FMA when the CPU has them: an MXFP4 or NVFP4 code is decoded by a
// permute over the sixteen signed e2m1 values (AVX-512) or over the eight
// magnitudes plus the sign bit (AVX2); an NVFP4 row scales each 16-element
// sum by its E4M3 byte and the row's total by the matrix's fp32 scale.
#include <immintrin.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "error.hpp"

namespace moe {
namespace {

// ---- a small persistent thread pool ---------------------------------------------
class Pool {
 public:
  explicit Pool(int n) {
    for (int i = 0; i < n; ++i) workers_.emplace_back([this] { loop(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(m_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }
  int size() const { return (int)workers_.size() + 1; }
  // run fn(task) for task in [0, n) on the pool and the calling thread
  void run(int n, const std::function<void(int)>& fn) {
    if (n <= 0) return;
    {
      std::lock_guard<std::mutex> g(m_);
      fn_ = &fn;
      n_ = n;
      next_.store(0);
      busy_ = (int)workers_.size();
      ++gen_;
    }
    cv_.notify_all();
    work();
    std::unique_lock<std::mutex> l(m_);
    done_.wait(l, [this] { return busy_ == 0; });
    fn_ = nullptr;
  }

 private:
  void work() {
    for (;;) {
      const int t = next_.fetch_add(1);
      if (t >= n_) break;
      (*fn_)(t);
    }
  }
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      {
        std::unique_lock<std::mutex> l(m_);
        cv_.wait(l, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
      }
      work();
      {
        std::lock_guard<std::mutex> g(m_);
        if (--busy_ == 0) done_.notify_all();
      }
    }
  }
  std::vector<std::thread> workers_;
  std::mutex m_;
  std::condition_variable cv_, done_;
  const std::function<void(int)>* fn_ = nullptr;
  int n_ = 0, busy_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
  std::atomic<int> next_{0};
};

std::mutex g_pool_m;
// held by a moe_host_experts call for as long as it uses the pool: calls from
// several host threads run one after another on it
std::mutex g_call_m;
Pool* g_pool = nullptr;
int g_pool_threads = 0;

Pool& pool(int threads) {
  std::lock_guard<std::mutex> g(g_pool_m);
  if (threads <= 0) {
    threads = (int)std::thread::hardware_concurrency();
    if (threads <= 0) threads = 1;
  }
  if (!g_pool || g_pool_threads != threads) {
    delete g_pool;
    g_pool = new Pool(threads - 1);
    g_pool_threads = threads;
  }
  return *g_pool;
}

// ---- formats ------------------------------------------------------------------------
inline float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline float e8m0(uint8_t s) {
  uint32_t u = s == 0 ? 0x00400000u : (s == 255 ? 0x7fc00000u : (uint32_t)s << 23);
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

const float kE2m1[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};

// OCP FP8 E4M3FN byte: sign, 4 exponent bits (bias 7), 3 mantissa bits;
// exponent 0 is subnormal (m / 8 * 2^-6).  The block scales written by the
// packer are non-negative and at most 448.
inline float e4m3(uint8_t s) {
  const int e = (s >> 3) & 15, m = s & 7;
  const float mag = e == 0 ? (float)m * 0x1p-9f : std::ldexp(1.0f + (float)m * 0.125f, e - 7);
  return (s & 0x80) ? -mag : mag;
}

// ---- row dots: a weight row against an fp32 vector of length K --------------------
float dot_mxfp4_scalar(const uint8_t* codes, const uint8_t* scales, const float* v, int K) {
  float acc = 0.f;
  for (int b = 0; b < K / 32; ++b) {
    float s = 0.f;
    for (int j = 0; j < 16; ++j) {
      const uint8_t byte = codes[b * 16 + j];
      const uint8_t lo = byte & 15, hi = byte >> 4;
      const float a = (lo & 8) ? -kE2m1[lo & 7] : kE2m1[lo & 7];
      const float c = (hi & 8) ? -kE2m1[hi & 7] : kE2m1[hi & 7];
      s += a * v[b * 32 + 2 * j] + c * v[b * 32 + 2 * j + 1];
    }
    acc += s * e8m0(scales[b]);
  }
  return acc;
}

// NVFP4 row: e2m1 codes, an E4M3 scale per 16 elements (the matrix's fp32
// scale is applied by the caller)
float dot_nvfp4_scalar(const uint8_t* codes, const uint8_t* scales, const float* v, int K) {
  float acc = 0.f;
  for (int b = 0; b < K / 16; ++b) {
    float s = 0.f;
    for (int j = 0; j < 8; ++j) {
      const uint8_t byte = codes[b * 8 + j];
      const uint8_t lo = byte & 15, hi = byte >> 4;
      const float a = (lo & 8) ? -kE2m1[lo & 7] : kE2m1[lo & 7];
      const float c = (hi & 8) ? -kE2m1[hi & 7] : kE2m1[hi & 7];
      s += a * v[b * 16 + 2 * j] + c * v[b * 16 + 2 * j + 1];
    }
    acc += s * e4m3(scales[b]);
  }
  return acc;
}

float dot_bf16_scalar(const uint16_t* w, const float* v, int K) {
  float acc = 0.f;
  for (int i = 0; i < K; ++i) acc += bf16_to_f32(w[i]) * v[i];
  return acc;
}

__attribute__((target("avx2,fma"))) inline float hsum256(__m256 v) {
  const __m128 lo = _mm256_castps256_ps128(v), hi = _mm256_extractf128_ps(v, 1);
  __m128 s = _mm_add_ps(lo, hi);
  s = _mm_add_ps(s, _mm_movehl_ps(s, s));
  s = _mm_add_ss(s, _mm_shuffle_ps(s, s, 1));
  return _mm_cvtss_f32(s);
}

// 8 codes (in the low bytes of c, element order) -> 8 floats
__attribute__((target("avx2,fma"))) inline __m256 decode8(__m128i c8, __m256 lut) {
  const __m256i c = _mm256_cvtepu8_epi32(c8);
  const __m256i mag = _mm256_and_si256(c, _mm256_set1_epi32(7));
  const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(c, _mm256_set1_epi32(8)), 28);
  return _mm256_xor_ps(_mm256_permutevar8x32_ps(lut, mag), _mm256_castsi256_ps(sgn));
}

__attribute__((target("avx2,fma"))) float dot_mxfp4_avx2(const uint8_t* codes,
                                                          const uint8_t* scales, const float* v,
                                                          int K) {
  const __m256 lut = _mm256_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f);
  const __m128i m15 = _mm_set1_epi8(15);
  __m256 acc = _mm256_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {
    const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + b * 16));
    const __m128i lo = _mm_and_si128(raw, m15);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m15);
    const __m128i c0 = _mm_unpacklo_epi8(lo, hi);   // codes 0..15
    const __m128i c1 = _mm_unpackhi_epi8(lo, hi);   // codes 16..31
    const float* x = v + b * 32;
    __m256 s = _mm256_mul_ps(decode8(c0, lut), _mm256_loadu_ps(x));
    s = _mm256_fmadd_ps(decode8(_mm_srli_si128(c0, 8), lut), _mm256_loadu_ps(x + 8), s);
    s = _mm256_fmadd_ps(decode8(c1, lut), _mm256_loadu_ps(x + 16), s);
    s = _mm256_fmadd_ps(decode8(_mm_srli_si128(c1, 8), lut), _mm256_loadu_ps(x + 24), s);
    acc = _mm256_fmadd_ps(s, _mm256_set1_ps(e8m0(scales[b])), acc);
  }
  return hsum256(acc);
}

__attribute__((target("avx2,fma"))) float dot_nvfp4_avx2(const uint8_t* codes,
                                                          const uint8_t* scales, const float* v,
                                                          int K) {
  const __m256 lut = _mm256_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f);
  const __m128i m15 = _mm_set1_epi8(15);
  __m256 acc = _mm256_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {          // two 16-element scale blocks
    const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + b * 16));
    const __m128i lo = _mm_and_si128(raw, m15);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m15);
    const __m128i c0 = _mm_unpacklo_epi8(lo, hi);   // codes 0..15
    const __m128i c1 = _mm_unpackhi_epi8(lo, hi);   // codes 16..31
    const float* x = v + b * 32;
    __m256 s0 = _mm256_mul_ps(decode8(c0, lut), _mm256_loadu_ps(x));
    s0 = _mm256_fmadd_ps(decode8(_mm_srli_si128(c0, 8), lut), _mm256_loadu_ps(x + 8), s0);
    __m256 s1 = _mm256_mul_ps(decode8(c1, lut), _mm256_loadu_ps(x + 16));
    s1 = _mm256_fmadd_ps(decode8(_mm_srli_si128(c1, 8), lut), _mm256_loadu_ps(x + 24), s1);
    acc = _mm256_fmadd_ps(s0, _mm256_set1_ps(e4m3(scales[2 * b])), acc);
    acc = _mm256_fmadd_ps(s1, _mm256_set1_ps(e4m3(scales[2 * b + 1])), acc);
  }
  float r = hsum256(acc);
  if (K % 32) r += dot_nvfp4_scalar(codes + (K / 32) * 16, scales + (K / 32) * 2,
                                    v + (K / 32) * 32, K % 32);
  return r;
}

__attribute__((target("avx2,fma"))) float dot_bf16_avx2(const uint16_t* w, const float* v,
                                                         int K) {
  __m256 acc0 = _mm256_setzero_ps(), acc1 = _mm256_setzero_ps();
  int i = 0;
  for (; i + 16 <= K; i += 16) {
    const __m256i a = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + i));
    const __m256i lo = _mm256_cvtepu16_epi32(_mm256_castsi256_si128(a));
    const __m256i hi = _mm256_cvtepu16_epi32(_mm256_extracti128_si256(a, 1));
    acc0 = _mm256_fmadd_ps(_mm256_castsi256_ps(_mm256_slli_epi32(lo, 16)),
                           _mm256_loadu_ps(v + i), acc0);
    acc1 = _mm256_fmadd_ps(_mm256_castsi256_ps(_mm256_slli_epi32(hi, 16)),
                           _mm256_loadu_ps(v + i + 8), acc1);
  }
  float s = hsum256(_mm256_add_ps(acc0, acc1));
  for (; i < K; ++i) s += bf16_to_f32(w[i]) * v[i];
  return s;
}

// AVX-512: the 16 signed e2m1 values in one register, a code is its own index
__attribute__((target("avx512f,avx512bw"))) float dot_mxfp4_avx512(const uint8_t* codes,
                                                                    const uint8_t* scales,
                                                                    const float* v, int K) {
  const __m512 lut = _mm512_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f, -0.f, -0.5f, -1.f,
                                    -1.5f, -2.f, -3.f, -4.f, -6.f);
  const __m128i m15 = _mm_set1_epi8(15);
  __m512 acc = _mm512_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {
    const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + b * 16));
    const __m128i lo = _mm_and_si128(raw, m15);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m15);
    const __m512 w0 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpacklo_epi8(lo, hi)), lut);
    const __m512 w1 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpackhi_epi8(lo, hi)), lut);
    const float* x = v + b * 32;
    const __m512 s = _mm512_fmadd_ps(w1, _mm512_loadu_ps(x + 16),
                                     _mm512_mul_ps(w0, _mm512_loadu_ps(x)));
    acc = _mm512_fmadd_ps(s, _mm512_set1_ps(e8m0(scales[b])), acc);
  }
  return _mm512_reduce_add_ps(acc);
}

__attribute__((target("avx512f,avx512bw"))) float dot_nvfp4_avx512(const uint8_t* codes,
                                                                    const uint8_t* scales,
                                                                    const float* v, int K) {
  const __m512 lut = _mm512_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f, -0.f, -0.5f, -1.f,
                                    -1.5f, -2.f, -3.f, -4.f, -6.f);
  const __m128i m15 = _mm_set1_epi8(15);
  __m512 acc = _mm512_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {          // two 16-element scale blocks
    const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + b * 16));
    const __m128i lo = _mm_and_si128(raw, m15);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m15);
    const __m512 w0 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpacklo_epi8(lo, hi)), lut);
    const __m512 w1 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpackhi_epi8(lo, hi)), lut);
    const float* x = v + b * 32;
    acc = _mm512_fmadd_ps(_mm512_mul_ps(w0, _mm512_loadu_ps(x)),
                          _mm512_set1_ps(e4m3(scales[2 * b])), acc);
    acc = _mm512_fmadd_ps(_mm512_mul_ps(w1, _mm512_loadu_ps(x + 16)),
                          _mm512_set1_ps(e4m3(scales[2 * b + 1])), acc);
  }
  float r = _mm512_reduce_add_ps(acc);
  if (K % 32) r += dot_nvfp4_scalar(codes + (K / 32) * 16, scales + (K / 32) * 2,
                                    v + (K / 32) * 32, K % 32);
  return r;
}

__attribute__((target("avx512f,avx512bw"))) float dot_bf16_avx512(const uint16_t* w,
                                                                   const float* v, int K) {
  __m512 acc = _mm512_setzero_ps();
  int i = 0;
  for (; i + 16 <= K; i += 16) {
    const __m512i a = _mm512_cvtepu16_epi32(
        _mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + i)));
    acc = _mm512_fmadd_ps(_mm512_castsi512_ps(_mm512_slli_epi32(a, 16)), _mm512_loadu_ps(v + i),
                          acc);
  }
  float s = _mm512_reduce_add_ps(acc);
  for (; i < K; ++i) s += bf16_to_f32(w[i]) * v[i];
  return s;
}

// MXFP4 row against a BF16 vector with BF16 dot products: every e2m1 value
// is exact in BF16 and so is x, so the products are exact and only the fp32
// sums round.  The 16 signed e2m1 values as BF16 bits, a code its index.
__attribute__((target("avx512f,avx512bw,avx512bf16"))) float dot_mxfp4_bf16dp(
    const uint8_t* codes, const uint8_t* scales, const uint16_t* xb, int K) {
  const __m512i lut = _mm512_setr_epi32(
      0x3F000000, 0x3FC03F80, 0x40404000, 0x40C04080,     // +0, 0.5, 1, 1.5, 2, 3, 4, 6
      (int)0xBF008000, (int)0xBFC0BF80, (int)0xC040C000, (int)0xC0C0C080,   // -0 .. -6
      0, 0, 0, 0, 0, 0, 0, 0);
  const __m128i m15 = _mm_set1_epi8(15);
  __m512 acc = _mm512_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {
    const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + b * 16));
    const __m128i lo = _mm_and_si128(raw, m15);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m15);
    const __m256i c = _mm256_set_m128i(_mm_unpackhi_epi8(lo, hi), _mm_unpacklo_epi8(lo, hi));
    const __m512i w = _mm512_permutexvar_epi16(_mm512_cvtepu8_epi16(c), lut);
    const __m512i x = _mm512_loadu_si512(xb + b * 32);
    const __m512 t = _mm512_dpbf16_ps(_mm512_setzero_ps(), (__m512bh)w, (__m512bh)x);
    acc = _mm512_fmadd_ps(t, _mm512_set1_ps(e8m0(scales[b])), acc);
  }
  return _mm512_reduce_add_ps(acc);
}

// Instruction-set level of the row dots: the best the CPU has, capped by
// the environment variable MOE_HOST_ISA (scalar, avx2, avx512, bf16) so that
// every path can be tested on one machine.  Read once per process.
int host_isa() {
  static const int v = [] {
    int best = 0;
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) best = 1;
    if (best && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw")) best = 2;
    if (best == 2 && __builtin_cpu_supports("avx512bf16")) best = 3;
    const char* cap = std::getenv("MOE_HOST_ISA");
    if (cap) {
      const int c = !std::strcmp(cap, "scalar") ? 0 : !std::strcmp(cap, "avx2") ? 1
                  : !std::strcmp(cap, "avx512") ? 2 : 3;
      if (c < best) best = c;
    }
    return best;
  }();
  return v;
}

bool have_avx512bf16() { return host_isa() >= 3; }
bool have_avx512() { return host_isa() >= 2; }
bool have_avx2() { return host_isa() >= 1; }

struct Layout {
  size_t off[6], bytes;
};

// dot of row `r` of matrix `m` (0 gate, 1 up, 2 down) with v
float row_dot(const moe_desc* d, const Layout& L, const uint8_t* blk, int m, int r,
              const float* v) {
  const int K = m < 2 ? d->hidden : d->inter;
  if (d->wtype == MOE_WTYPE_MXFP4) {
    const uint8_t* codes = blk + L.off[2 * m] + (size_t)r * (K / 2);
    const uint8_t* scales = blk + L.off[2 * m + 1] + (size_t)r * (K / 32);
    if (have_avx512()) return dot_mxfp4_avx512(codes, scales, v, K);
    if (have_avx2()) return dot_mxfp4_avx2(codes, scales, v, K);
    return dot_mxfp4_scalar(codes, scales, v, K);
  }
  if (d->wtype == MOE_WTYPE_NVFP4) {
    // codes [rows][K/2], E4M3 scales [rows][K/16]; the three fp32 matrix
    // scales follow the down scales
    const uint8_t* codes = blk + L.off[2 * m] + (size_t)r * (K / 2);
    const uint8_t* scales = blk + L.off[2 * m + 1] + (size_t)r * (K / 16);
    float g;
    std::memcpy(&g, blk + L.off[5] + (size_t)d->hidden * d->inter / 16 + 4 * m, 4);
    float acc;
    if (have_avx512()) acc = dot_nvfp4_avx512(codes, scales, v, K);
    else if (have_avx2()) acc = dot_nvfp4_avx2(codes, scales, v, K);
    else acc = dot_nvfp4_scalar(codes, scales, v, K);
    return acc * g;
  }
  const uint16_t* w = reinterpret_cast<const uint16_t*>(blk + L.off[m]) + (size_t)r * K;
  if (have_avx512()) return dot_bf16_avx512(w, v, K);
  if (have_avx2()) return dot_bf16_avx2(w, v, K);
  return dot_bf16_scalar(w, v, K);
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

int moe_host_experts(const moe_desc* desc, const void* x, int32_t T, const int32_t* ids,
                     const float* w, const uint8_t* include, const void* host_pool,
                     const int32_t* host_index, float* y, int32_t n_threads) {
  int st = check_desc(desc);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (T < 0) return set_error(MOE_EINVAL, "T < 0");
  if (!x || !ids || !w || !host_pool || !y) return set_error(MOE_EINVAL, "null pointer");
  if (desc->wtype != MOE_WTYPE_MXFP4 && desc->wtype != MOE_WTYPE_BF16 &&
      desc->wtype != MOE_WTYPE_NVFP4)
    return set_error(MOE_EUNSUPPORTED, "host experts run BF16, MXFP4 or NVFP4 weights");
  const int H = desc->hidden, I = desc->inter, E = desc->n_experts, k = desc->top_k;
  Layout L;
  layout(desc, L.off, &L.bytes);
  const uint8_t* pool_b = static_cast<const uint8_t*>(host_pool);

  // x in fp32, y cleared
  std::vector<float> xf((size_t)T * H);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16_to_f32(xb[i]);
  std::memset(y, 0, sizeof(float) * (size_t)T * H);

  // experts with their (token, weight) entries, in first-appearance order
  std::vector<int> order;
  std::vector<std::vector<std::pair<int, float>>> ent(E);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      const int p = t * k + j;
      if (include && !include[p]) continue;
      const int e = ids[p];
      if (e < 0 || e >= E) return set_error(MOE_EINVAL, "expert id %d out of range", e);
      if (ent[e].empty()) order.push_back(e);
      ent[e].push_back({t, w[p]});
    }
  }
  std::lock_guard<std::mutex> call_lock(g_call_m);
  Pool& P = pool(n_threads);
  std::vector<float> h;
  constexpr int kRows = 32;                     // rows per task
  for (int e : order) {
    const int idx = host_index ? host_index[e] : e;
    if (idx < 0) return set_error(MOE_EINVAL, "expert %d has no host block", e);
    const uint8_t* blk = pool_b + (size_t)idx * L.bytes;
    const auto& en = ent[e];
    const int n = (int)en.size();
    h.assign((size_t)n * I, 0.f);
    // gate/up rows -> h
    P.run((I + kRows - 1) / kRows, [&](int task) {
      const int r1 = std::min(I, (task + 1) * kRows);
      for (int r = task * kRows; r < r1; ++r) {
        for (int q = 0; q < n; ++q) {
          const float* xv = xf.data() + (size_t)en[q].first * H;
          float g, u;
          if (desc->wtype == MOE_WTYPE_MXFP4 && have_avx512bf16()) {
            // gate/up against x in BF16 (exact) with BF16 dot products
            const uint16_t* xr = xb + (size_t)en[q].first * H;
            g = dot_mxfp4_bf16dp(blk + L.off[0] + (size_t)r * (H / 2),
                                 blk + L.off[1] + (size_t)r * (H / 32), xr, H);
            u = dot_mxfp4_bf16dp(blk + L.off[2] + (size_t)r * (H / 2),
                                 blk + L.off[3] + (size_t)r * (H / 32), xr, H);
          } else {
            g = row_dot(desc, L, blk, 0, r, xv);
            u = row_dot(desc, L, blk, 1, r, xv);
          }
          h[(size_t)q * I + r] = g / (1.0f + std::exp(-g)) * u;
        }
      }
    });
    // down rows -> y (each task owns its output rows)
    P.run((H + kRows - 1) / kRows, [&](int task) {
      const int r1 = std::min(H, (task + 1) * kRows);
      for (int r = task * kRows; r < r1; ++r) {
        for (int q = 0; q < n; ++q) {
          const float o = row_dot(desc, L, blk, 2, r, h.data() + (size_t)q * I);
          y[(size_t)en[q].first * H + r] += en[q].second * o;
        }
      }
    });
  }
  return MOE_OK;
}

int moe_host_expert_rate(const moe_desc* desc, const void* host_pool, int32_t n_experts_timed,
                         int32_t reps, int32_t n_threads, double* bytes_per_s) {
  int st = check_desc(desc);
  if (st) return st;
  if (!host_pool || !bytes_per_s || n_experts_timed < 1 || reps < 1)
    return set_error(MOE_EINVAL, "bad rate probe arguments");
  if (n_experts_timed > desc->n_experts) n_experts_timed = desc->n_experts;
  Layout L;
  layout(desc, L.off, &L.bytes);
  const int H = desc->hidden, k = desc->top_k;
  std::vector<uint16_t> x((size_t)H, 0x3f80);   // ones
  std::vector<int32_t> ids(k, -1);
  std::vector<float> w(k, 1.f);
  std::vector<uint8_t> inc(k, 0);
  std::vector<float> y((size_t)H);
  double best = 0.0;
  for (int r = 0; r < reps; ++r) {
    const auto t0 = std::chrono::steady_clock::now();
    for (int e0 = 0; e0 < n_experts_timed; e0 += k) {
      int m = 0;
      for (int j = 0; j < k; ++j) {
        const int e = e0 + j;
        ids[j] = e < n_experts_timed ? e : 0;
        inc[j] = e < n_experts_timed;
        m += inc[j];
      }
      (void)m;
      st = moe_host_experts(desc, x.data(), 1, ids.data(), w.data(), inc.data(), host_pool,
                            nullptr, y.data(), n_threads);
      if (st) return st;
    }
    const double s =
        std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    const double rate = (double)n_experts_timed * (double)L.bytes / s;
    if (rate > best) best = rate;
  }
  *bytes_per_s = best;
  return MOE_OK;
}

}  // extern "C"

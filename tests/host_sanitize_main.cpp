// Driver for the sanitizer build of the HIP-free host sources (planner.cpp,
// host.cpp, host_expert.cpp): exercises the LRU planner (plans, rollbacks,
// resizes, bad arguments), q*, and the host expert kernel on BF16, MXFP4 and
// NVFP4 blocks of random bytes (thread counts 1 and 4 must agree bit for
// bit), so that AddressSanitizer and UndefinedBehaviorSanitizer see every
// path.  Numerics are checked against the oracle elsewhere; here the checks
// are memory safety, defined behaviour and the functions' own invariants.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "moe.h"

#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static int planner_paths(std::mt19937& rng) {
  moe_planner* p = nullptr;
  CHECK(moe_planner_create(&p, 2, 32, 8) == MOE_OK);
  CHECK(moe_planner_set_bandwidths(p, 51.5e9, 178e9) == MOE_OK);
  std::uniform_int_distribution<int> expert(0, 31), qd(-1, 6), coin(0, 9);
  std::uniform_real_distribution<float> wd(0.01f, 0.3f);
  moe_plan plan;
  for (int step = 0; step < 400; ++step) {
    const int n = 1 + step % 12;
    std::vector<int32_t> ids(n);
    std::vector<float> w(n);
    for (int i = 0; i < n; ++i) { ids[i] = expert(rng); w[i] = wd(rng); }
    const int layer = step % 2;
    CHECK(moe_planner_plan(p, layer, ids.data(), w.data(), n, qd(rng), &plan) == MOE_OK);
    CHECK(plan.n_hits + plan.n_misses == plan.n_selected);
    CHECK(plan.q + plan.n_host == plan.n_misses);
    std::vector<int32_t> table(32);
    CHECK(moe_planner_slot_table(p, layer, table.data()) == MOE_OK);
    int resident = 0;
    for (int e = 0; e < 32; ++e) resident += table[e] >= 0;
    CHECK(resident <= moe_planner_n_slots(p));
    if (coin(rng) == 0) CHECK(moe_planner_rollback(p) == MOE_OK);
    if (step == 150 || step == 250 || step == 330) {
      const int ns = step == 150 ? 3 : (step == 250 ? 12 : 8);
      std::vector<int32_t> old_of_new(ns);
      CHECK(moe_planner_resize(p, ns, old_of_new.data()) == MOE_OK);
      CHECK(moe_planner_n_slots(p) == ns);
    }
  }
  // bad arguments leave the state alone and set the error text
  int32_t bad = 99;
  float bw = 0.5f;
  CHECK(moe_planner_plan(p, 0, &bad, &bw, 1, 1, &plan) == MOE_EINVAL);
  CHECK(std::strlen(moe_last_error()) > 0);
  CHECK(moe_planner_plan(p, 5, &bad, &bw, 1, 1, &plan) != MOE_OK);
  std::vector<int32_t> old(4);
  CHECK(moe_planner_resize(p, 0, old.data()) != MOE_OK);
  moe_planner_destroy(p);
  // more distinct experts in one step than a plan holds
  CHECK(moe_planner_create(&p, 1, 1024, 16) == MOE_OK);
  std::vector<int32_t> many(MOE_PLAN_MAX + 8);
  std::vector<float> mw(many.size(), 0.1f);
  for (size_t i = 0; i < many.size(); ++i) many[i] = (int32_t)i;
  CHECK(moe_planner_plan(p, 0, many.data(), mw.data(), (int32_t)many.size(), 2, &plan) ==
        MOE_ECACHE);
  moe_planner_destroy(p);
  return 0;
}

static int qstar_paths() {
  for (int m = 0; m <= 16; ++m) {
    const int32_t q = moe_qstar(m, 51.5e9, 178e9);
    CHECK(q >= 0 && q <= m);
  }
  CHECK(moe_qstar(-1, 1.0, 1.0) == -1);
  CHECK(moe_qstar(4, 0.0, 1.0) == -1);
  CHECK(moe_qstar(4, 1.0, NAN) == -1);
  return 0;
}

// random expert blocks whose values stay finite
static void fill_pool(const moe_desc& d, std::vector<uint8_t>& pool, int n_blocks,
                      std::mt19937& rng) {
  size_t off[6], bytes;
  moe_expert_layout(&d, off, &bytes);
  pool.assign(bytes * n_blocks, 0);
  std::uniform_int_distribution<int> byte(0, 255), sc(118, 126), e4(0x20, 0x50);
  const size_t H = d.hidden, I = d.inter;
  for (int b = 0; b < n_blocks; ++b) {
    uint8_t* blk = pool.data() + b * bytes;
    if (d.wtype == MOE_WTYPE_BF16) {
      uint16_t* v = reinterpret_cast<uint16_t*>(blk);
      std::normal_distribution<float> nd(0.f, 0.02f);
      for (size_t i = 0; i < 3 * H * I; ++i) {
        const float f = nd(rng);
        uint32_t u;
        std::memcpy(&u, &f, 4);
        v[i] = (uint16_t)(u >> 16);
      }
      continue;
    }
    const bool nv = d.wtype == MOE_WTYPE_NVFP4;
    for (int m = 0; m < 3; ++m) {
      const size_t rows = m < 2 ? I : H, K = m < 2 ? H : I;
      for (size_t i = 0; i < rows * K / 2; ++i) blk[off[2 * m] + i] = (uint8_t)byte(rng);
      for (size_t i = 0; i < rows * K / (nv ? 16 : 32); ++i)
        blk[off[2 * m + 1] + i] = (uint8_t)(nv ? e4(rng) : sc(rng));
    }
    if (nv) {
      float g[3] = {0.01f, 0.02f, 0.005f};
      std::memcpy(blk + off[5] + H * I / 16, g, sizeof g);
    }
  }
}

static int host_expert_paths(std::mt19937& rng) {
  for (int wt : {MOE_WTYPE_BF16, MOE_WTYPE_MXFP4, MOE_WTYPE_NVFP4}) {
    moe_desc d = {256, 128, 8, 2, 0, 0, wt, MOE_WTYPE_BF16};
    const int T = 5, E = d.n_experts, k = d.top_k, H = d.hidden;
    std::vector<uint8_t> pool;
    fill_pool(d, pool, E, rng);
    std::vector<uint16_t> x((size_t)T * H);
    std::normal_distribution<float> nd(0.f, 1.f);
    for (auto& v : x) {
      const float f = nd(rng);
      uint32_t u;
      std::memcpy(&u, &f, 4);
      v = (uint16_t)(u >> 16);
    }
    std::vector<int32_t> ids((size_t)T * k);
    std::vector<float> w((size_t)T * k);
    std::vector<uint8_t> inc((size_t)T * k);
    std::vector<int32_t> index(E);
    for (int e = 0; e < E; ++e) index[e] = E - 1 - e;     // block order reversed
    for (int i = 0; i < T * k; ++i) {
      ids[i] = (i * 3 + 1) % E;
      w[i] = 0.1f * (1 + i % 3);
      inc[i] = (uint8_t)(i % 3 != 0);
    }
    std::vector<float> y1((size_t)T * H), y4((size_t)T * H);
    CHECK(moe_host_experts(&d, x.data(), T, ids.data(), w.data(), inc.data(), pool.data(),
                           index.data(), y1.data(), 1) == MOE_OK);
    CHECK(moe_host_experts(&d, x.data(), T, ids.data(), w.data(), inc.data(), pool.data(),
                           index.data(), y4.data(), 4) == MOE_OK);
    CHECK(std::memcmp(y1.data(), y4.data(), y1.size() * 4) == 0);
    for (float v : y1) CHECK(std::isfinite(v));
    // all pairs, identity index
    CHECK(moe_host_experts(&d, x.data(), T, ids.data(), w.data(), nullptr, pool.data(), nullptr,
                           y1.data(), 0) == MOE_OK);
    // an included expert without a block, an id out of range
    index[ids[1]] = -1;
    CHECK(moe_host_experts(&d, x.data(), T, ids.data(), w.data(), nullptr, pool.data(),
                           index.data(), y1.data(), 2) == MOE_EINVAL);
    ids[0] = E + 3;
    CHECK(moe_host_experts(&d, x.data(), T, ids.data(), w.data(), nullptr, pool.data(), nullptr,
                           y1.data(), 2) == MOE_EINVAL);
    double rate = 0;
    CHECK(moe_host_expert_rate(&d, pool.data(), 4, 1, 2, &rate) == MOE_OK);
    CHECK(rate > 0);
  }
  return 0;
}

int main() {
  std::mt19937 rng(7);
  if (planner_paths(rng)) return 1;
  if (qstar_paths()) return 1;
  if (host_expert_paths(rng)) return 1;
  std::printf("host sanitize driver: ok\n");
  return 0;
}

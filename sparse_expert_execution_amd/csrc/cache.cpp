// cache.cpp - expert cache in GPU memory filled from a pinned host pool, and
// the bandwidth probe that feeds the q* split.
//
// A miss can be copied over PCIe, run on the GPU and kept cached (explainx.ai
// guide, "Decode: decide whether to move an expert or compute where it
// lives"); the host pool is the source of truth and experts sit there in the
// same layout as in a device slot ("FreeToken 753b Model Explained", "How MoE
// Paging and Caching Work").  Fills run on a side stream with one
// hipMemcpyAsync per expert; events order them after the victim slot's last
// reader and before the compute stream's next use.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "../../include/moe.h"
#include "hip_error.hpp"
#include "kernels.hpp"
#include "planner.hpp"

using moe::hip_status;
using moe::set_error;

namespace moe {
namespace {

constexpr int kMaxUpdates = 64;
struct SlotUpdates {
  int n;
  int32_t idx[kMaxUpdates];
  int32_t val[kMaxUpdates];
};

__global__ void slot_update_kernel(int32_t* table, SlotUpdates u) {
  const int i = threadIdx.x;
  if (i < u.n) table[u.idx[i]] = u.val[i];
}

}  // namespace
}  // namespace moe

struct moe_cache {
  moe_planner* planner = nullptr;
  const uint8_t* host_pool = nullptr;
  uint8_t* dev_pool = nullptr;
  int32_t* dev_table = nullptr;
  int32_t n_layers = 0, n_experts = 0, n_slots = 0;
  size_t expert_bytes = 0;
  std::vector<hipEvent_t> slot_event;
  std::vector<char> slot_recorded;
  hipEvent_t fill_done = nullptr;
  int fail_fills = 0;
};

namespace {

int push_updates(moe_cache* c, const std::vector<std::pair<int32_t, int32_t>>& ups,
                 hipStream_t st) {
  for (size_t i = 0; i < ups.size(); i += moe::kMaxUpdates) {
    moe::SlotUpdates u;
    u.n = (int)std::min<size_t>(moe::kMaxUpdates, ups.size() - i);
    for (int j = 0; j < u.n; ++j) {
      u.idx[j] = ups[i + j].first;
      u.val[j] = ups[i + j].second;
    }
    hipLaunchKernelGGL(moe::slot_update_kernel, dim3(1), dim3(64), 0, st, c->dev_table, u);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return hip_status(err, "slot table update");
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_cache_create(moe_cache** out, const void* host_pool, int32_t n_layers, int32_t n_experts,
                     size_t expert_bytes, void* dev_slot_pool, int32_t n_slots,
                     int32_t* dev_slot_of_expert) {
  if (!out) return set_error(MOE_EINVAL, "null output");
  *out = nullptr;
  if (!host_pool || !dev_slot_pool || !dev_slot_of_expert || expert_bytes == 0 ||
      expert_bytes % 256)
    return set_error(MOE_EINVAL, "null pool/table or expert_bytes not a multiple of 256");
  moe_cache* c = new (std::nothrow) moe_cache;
  if (!c) return set_error(MOE_EINVAL, "out of host memory");
  int st = moe_planner_create(&c->planner, n_layers, n_experts, n_slots);
  if (st) {
    delete c;
    return st;
  }
  c->host_pool = static_cast<const uint8_t*>(host_pool);
  c->dev_pool = static_cast<uint8_t*>(dev_slot_pool);
  c->dev_table = dev_slot_of_expert;
  c->n_layers = n_layers;
  c->n_experts = n_experts;
  c->n_slots = n_slots;
  c->expert_bytes = expert_bytes;
  c->slot_event.assign(n_slots, nullptr);
  c->slot_recorded.assign(n_slots, 0);
  hipError_t err = hipSuccess;
  for (int s = 0; s < n_slots && err == hipSuccess; ++s)
    err = hipEventCreateWithFlags(&c->slot_event[s], hipEventDisableTiming);
  if (err == hipSuccess) err = hipEventCreateWithFlags(&c->fill_done, hipEventDisableTiming);
  if (err == hipSuccess)
    err = moe::launch_fill_i32(dev_slot_of_expert, -1, (int64_t)n_layers * n_experts, nullptr);
  if (err == hipSuccess) err = hipStreamSynchronize(nullptr);
  if (err != hipSuccess) {
    moe_cache_destroy(c);
    return hip_status(err, "moe_cache_create");
  }
  *out = c;
  return MOE_OK;
}

void moe_cache_destroy(moe_cache* c) {
  if (!c) return;
  for (hipEvent_t e : c->slot_event)
    if (e) (void)hipEventDestroy(e);
  if (c->fill_done) (void)hipEventDestroy(c->fill_done);
  moe_planner_destroy(c->planner);
  delete c;
}

int moe_cache_set_bandwidths(moe_cache* c, double b_pcie, double b_host) {
  if (!c) return set_error(MOE_EINVAL, "null cache");
  return moe_planner_set_bandwidths(c->planner, b_pcie, b_host);
}

const moe_planner* moe_cache_planner(const moe_cache* c) { return c ? c->planner : nullptr; }

int moe_cache_plan(moe_cache* c, int32_t layer, const int32_t* ids_host, const float* w_host,
                   int32_t n, int32_t q, moe_plan* plan) {
  moe::ApiRange range_("moe_cache_plan");
  if (!c) return set_error(MOE_EINVAL, "null cache");
  return moe::planner_plan(c->planner, layer, ids_host, w_host, n, q, plan);
}

int moe_cache_debug_fail_fills(moe_cache* c, int32_t n) {
  if (!c || n < 0) return set_error(MOE_EINVAL, "bad argument");
  c->fail_fills = n;
  return MOE_OK;
}

int cache_fill(moe_cache* c, const moe_plan* plan, void* side_stream, void* compute_stream) {
  moe::ApiRange range_("cache_fill");
  if (!c || !plan) return set_error(MOE_EINVAL, "null pointer");
  hipStream_t side = static_cast<hipStream_t>(side_stream);
  hipStream_t comp = static_cast<hipStream_t>(compute_stream);
  if (plan->layer < 0 || plan->layer >= c->n_layers || plan->q < 0 || plan->q > MOE_PLAN_MAX) {
    moe::planner_rollback(c->planner);
    return set_error(MOE_ECACHE, "invalid plan");
  }
  for (int i = 0; i < plan->q; ++i) {
    const int s = plan->fill_slot[i], e = plan->fill_expert[i];
    if (s < 0 || s >= c->n_slots || e < 0 || e >= c->n_experts ||
        moe::planner_slot_key(c->planner, s) != plan->layer * c->n_experts + e) {
      moe::planner_rollback(c->planner);
      return set_error(MOE_ECACHE, "plan does not match the cache state (fill %d)", i);
    }
  }
  if (c->fail_fills > 0) {
    --c->fail_fills;
    moe::planner_rollback(c->planner);
    return set_error(MOE_EHIP, "cache_fill: injected failure before any copy");
  }
  std::vector<std::pair<int32_t, int32_t>> ups;
  hipError_t err = hipSuccess;
  int issued = 0;
  for (int i = 0; i < plan->q && err == hipSuccess; ++i) {
    const int s = plan->fill_slot[i], e = plan->fill_expert[i];
    if (c->slot_recorded[s]) err = hipStreamWaitEvent(side, c->slot_event[s], 0);
    if (err != hipSuccess) break;
    const uint8_t* src =
        c->host_pool + ((size_t)plan->layer * c->n_experts + e) * c->expert_bytes;
    err = hipMemcpyAsync(c->dev_pool + (size_t)s * c->expert_bytes, src, c->expert_bytes,
                         hipMemcpyHostToDevice, side);
    if (err == hipSuccess) ++issued;
    if (plan->victim_layer[i] >= 0)
      ups.emplace_back(plan->victim_layer[i] * c->n_experts + plan->victim_expert[i], -1);
    ups.emplace_back(plan->layer * c->n_experts + e, s);
  }
  if (err == hipSuccess && plan->q > 0) err = hipEventRecord(c->fill_done, side);
  if (err == hipSuccess && plan->q > 0) err = hipStreamWaitEvent(comp, c->fill_done, 0);
  int st = MOE_OK;
  if (err != hipSuccess) {
    st = hip_status(err, "cache_fill");
  } else if (!ups.empty()) {
    st = push_updates(c, ups, comp);
  }
  if (st != MOE_OK) {
    // undo the plan; slots whose copy may have started no longer hold their
    // old expert, so they leave the cache
    std::string msg = moe::g_last_error;
    moe::planner_rollback(c->planner);
    std::vector<std::pair<int32_t, int32_t>> clear;
    for (int i = 0; i < issued + 1 && i < plan->q; ++i) {
      const int s = plan->fill_slot[i];
      const int32_t key = moe::planner_slot_key(c->planner, s);
      if (key >= 0) clear.emplace_back(key, -1);
      moe::planner_forget_slot(c->planner, s);
    }
    (void)push_updates(c, clear, comp);
    moe::g_last_error = msg;
    return st;
  }
  return MOE_OK;
}

int moe_cache_resize(moe_cache* c, void* dev_slot_pool, int32_t n_slots, void* compute_stream) {
  moe::ApiRange range_("moe_cache_resize");
  if (!c || !dev_slot_pool) return set_error(MOE_EINVAL, "null pointer");
  if (n_slots < 1) return set_error(MOE_EINVAL, "slot budget %d < 1", n_slots);
  uint8_t* np = static_cast<uint8_t*>(dev_slot_pool);
  const size_t eb = c->expert_bytes;
  if (np != c->dev_pool) {
    const uint8_t* a0 = c->dev_pool;
    const uint8_t* a1 = a0 + (size_t)c->n_slots * eb;
    const uint8_t* b1 = np + (size_t)n_slots * eb;
    if (np < a1 && a0 < b1)
      return set_error(MOE_EINVAL, "new slot pool overlaps the old one without being it");
  }
  hipStream_t comp = static_cast<hipStream_t>(compute_stream);
  const int32_t n_old = c->n_slots;
  std::vector<int32_t> old_key(n_old);
  for (int32_t s = 0; s < n_old; ++s) old_key[s] = moe::planner_slot_key(c->planner, s);
  // events of the new budget first, so that a failure leaves everything as it was
  std::vector<hipEvent_t> ev(n_slots, nullptr);
  hipError_t err = hipSuccess;
  for (int32_t s = n_old; s < n_slots && err == hipSuccess; ++s)
    err = hipEventCreateWithFlags(&ev[s], hipEventDisableTiming);
  if (err != hipSuccess) {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    return hip_status(err, "moe_cache_resize");
  }
  std::vector<int32_t> old_of_new(n_slots);
  int st = moe::planner_resize(c->planner, n_slots, old_of_new.data());
  if (st) {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    return st;
  }
  std::vector<int32_t> new_of_old(n_old, -1);
  for (int32_t d = 0; d < n_slots; ++d)
    if (old_of_new[d] >= 0) new_of_old[old_of_new[d]] = d;
  // survivors that change place: device-to-device copies on the compute
  // stream, after every earlier reader of the old slots
  for (int32_t d = 0; d < n_slots && err == hipSuccess; ++d) {
    const int32_t s = old_of_new[d];
    if (s < 0) continue;
    uint8_t* dst = np + (size_t)d * eb;
    const uint8_t* src = c->dev_pool + (size_t)s * eb;
    if (dst != src) err = hipMemcpyAsync(dst, src, eb, hipMemcpyDeviceToDevice, comp);
  }
  std::vector<std::pair<int32_t, int32_t>> ups;
  for (int32_t s = 0; s < n_old; ++s) {
    if (old_key[s] < 0) continue;
    if (new_of_old[s] < 0) ups.emplace_back(old_key[s], -1);
    else if (new_of_old[s] != s) ups.emplace_back(old_key[s], new_of_old[s]);
  }
  for (int32_t s = 0; s < n_old; ++s) {
    if (s < n_slots) ev[s] = c->slot_event[s];
    else (void)hipEventDestroy(c->slot_event[s]);
  }
  c->slot_event = std::move(ev);
  c->slot_recorded.assign(n_slots, 0);
  c->dev_pool = np;
  c->n_slots = n_slots;
  if (err == hipSuccess) st = push_updates(c, ups, comp);
  else st = hip_status(err, "moe_cache_resize copies");
  // every slot's last use is now this rebuild
  for (int32_t s = 0; s < n_slots && st == MOE_OK; ++s) {
    err = hipEventRecord(c->slot_event[s], comp);
    if (err != hipSuccess) st = hip_status(err, "moe_cache_resize");
    else c->slot_recorded[s] = 1;
  }
  return st;
}

int moe_cache_release(moe_cache* c, const moe_plan* plan, void* compute_stream) {
  moe::ApiRange range_("moe_cache_release");
  if (!c || !plan) return set_error(MOE_EINVAL, "null pointer");
  hipStream_t comp = static_cast<hipStream_t>(compute_stream);
  auto rec = [&](int s) -> int {
    if (s < 0 || s >= c->n_slots) return set_error(MOE_ECACHE, "slot %d out of range", s);
    hipError_t err = hipEventRecord(c->slot_event[s], comp);
    if (err != hipSuccess) return hip_status(err, "moe_cache_release");
    c->slot_recorded[s] = 1;
    return MOE_OK;
  };
  for (int i = 0; i < plan->n_hits; ++i) {
    int st = rec(plan->hit_slot[i]);
    if (st) return st;
  }
  for (int i = 0; i < plan->q; ++i) {
    int st = rec(plan->fill_slot[i]);
    if (st) return st;
  }
  return MOE_OK;
}

int moe_probe_bandwidths(const void* pinned_host, void* dev, size_t bytes, int32_t reps,
                         int32_t threads, void* stream, double* b_pcie, double* b_host) {
  if (!pinned_host || !dev || !b_pcie || !b_host || bytes < 4096 || reps < 1)
    return set_error(MOE_EINVAL, "bad probe arguments");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  if (err != hipSuccess) return hip_status(err, "probe events");
  double best = 0;
  for (int r = 0; r < reps + 1 && err == hipSuccess; ++r) {
    err = hipEventRecord(e0, st);
    if (err == hipSuccess) err = hipMemcpyAsync(dev, pinned_host, bytes, hipMemcpyHostToDevice, st);
    if (err == hipSuccess) err = hipEventRecord(e1, st);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float ms = 0;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
    if (err == hipSuccess && r > 0 && ms > 0) best = std::max(best, bytes / (ms * 1e-3));
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return hip_status(err, "probe copy");
  *b_pcie = best;

  // host streaming read: threads sum disjoint 64-bit words
  int nt = threads > 0 ? threads : (int)std::max(1u, std::thread::hardware_concurrency());
  const uint64_t* words = static_cast<const uint64_t*>(pinned_host);
  const size_t nw = bytes / 8;
  double hbest = 0;
  std::atomic<uint64_t> sink{0};
  for (int r = 0; r < reps + 1; ++r) {
    auto t0 = std::chrono::steady_clock::now();
    std::vector<std::thread> pool;
    for (int i = 0; i < nt; ++i) {
      pool.emplace_back([&, i]() {
        const size_t lo = nw * i / nt, hi = nw * (i + 1) / nt;
        uint64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
        size_t j = lo;
        for (; j + 4 <= hi; j += 4) {
          s0 += words[j]; s1 += words[j + 1]; s2 += words[j + 2]; s3 += words[j + 3];
        }
        for (; j < hi; ++j) s0 += words[j];
        sink += s0 + s1 + s2 + s3;
      });
    }
    for (auto& t : pool) t.join();
    const double s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    if (r > 0 && s > 0) hbest = std::max(hbest, bytes / s);
  }
  *b_host = hbest;
  return MOE_OK;
}

}  // extern "C"

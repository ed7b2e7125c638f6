// planner.cpp - the global LRU expert-cache planner.  Host only: no HIP
// calls, so it builds and is tested without a GPU.
//
// One cache of numbered slots is shared by every MoE layer and follows the
// router with least-recently-used replacement ("FreeToken 753b Model
// Explained", "How MoE Paging and Caching Work"; futuresignalnews.com,
// "2. Semantic-Aware Caching").  A miss is either filled into a slot or left
// to the host side; how many are filled is the q* split (explainx.ai guide,
// "Decode: decide whether to move an expert or compute where it lives").
// Tie-breaks and the choice of which misses to fill are not on the pages;
// the rules used are listed in include/moe.h next to moe_planner_plan.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe.h"
#include "planner.hpp"

using moe::set_error;

namespace moe {

struct PlannerState {
  std::vector<int32_t> slot_key;   // slot -> layer * E + expert, -1 = empty
  std::vector<uint64_t> stamp;     // slot -> last-use clock
  std::vector<int32_t> where;      // key -> slot, -1 = not resident
  uint64_t clock = 0;
};

}  // namespace moe

struct moe_planner {
  int32_t n_layers, n_experts, n_slots;
  double b_pcie = 0, b_host = 0;
  moe::PlannerState st, saved;
  bool have_saved = false;
  std::vector<float> weight;       // scratch [E]
  std::vector<int32_t> seen;       // scratch [E], -1 = not in step
};

namespace moe {

int planner_plan(moe_planner* p, int32_t layer, const int32_t* ids, const float* w, int32_t n,
                 int32_t q, moe_plan* plan) {
  if (!p || !plan || (n > 0 && (!ids || !w))) return set_error(MOE_EINVAL, "null pointer");
  if (layer < 0 || layer >= p->n_layers) return set_error(MOE_EINVAL, "layer %d out of range", layer);
  if (n < 0) return set_error(MOE_EINVAL, "n < 0");
  const int E = p->n_experts;
  // selected set: distinct ids, first-appearance order, summed weights
  std::vector<int32_t> sel;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = ids[i];
    if (e < 0 || e >= E) {
      for (int32_t s : sel) p->seen[s] = -1;
      return set_error(MOE_EINVAL, "expert id %d out of range", e);
    }
    if (p->seen[e] < 0) {
      p->seen[e] = (int32_t)sel.size();
      p->weight[e] = 0.f;
      sel.push_back(e);
    }
    p->weight[e] += w[i];
  }
  auto clear_seen = [&]() { for (int32_t s : sel) p->seen[s] = -1; };
  if ((int)sel.size() > MOE_PLAN_MAX) {
    clear_seen();
    return set_error(MOE_ECACHE, "%zu distinct experts exceed MOE_PLAN_MAX", sel.size());
  }
  std::vector<int32_t> misses_ranked;
  int nh = 0, nm = 0;
  for (int32_t e : sel) {
    if (p->st.where[layer * E + e] >= 0) ++nh;
    else misses_ranked.push_back(e), ++nm;
  }
  int32_t qq = q;
  if (qq < 0) {
    if (!(p->b_pcie > 0) || !(p->b_host > 0)) {
      clear_seen();
      return set_error(MOE_EINVAL, "q < 0 needs bandwidths (moe_planner_set_bandwidths)");
    }
    qq = moe_qstar(nm, p->b_pcie, p->b_host);
  }
  // state is modified from here on: keep a copy for rollback
  p->saved = p->st;
  p->have_saved = true;

  std::memset(plan, 0, sizeof(*plan));
  plan->layer = layer;
  plan->n_selected = (int32_t)sel.size();
  int hi = 0, mi = 0;
  for (size_t i = 0; i < sel.size(); ++i) {
    const int32_t e = sel[i];
    plan->selected[i] = e;
    const int32_t s = p->st.where[layer * E + e];
    if (s >= 0) {
      plan->hits[hi] = e;
      plan->hit_slot[hi] = s;
      ++hi;
      p->st.stamp[s] = ++p->st.clock;
    } else {
      plan->misses[mi++] = e;
    }
  }
  plan->n_hits = nh;
  plan->n_misses = nm;
  std::stable_sort(misses_ranked.begin(), misses_ranked.end(), [&](int32_t a, int32_t b) {
    if (p->weight[a] != p->weight[b]) return p->weight[a] > p->weight[b];
    return a < b;
  });
  const int cap = p->n_slots - nh;
  int qe = qq < 0 ? 0 : qq;
  if (qe > nm) qe = nm;
  if (qe > cap) qe = cap;
  if (qe < 0) qe = 0;
  for (int i = 0; i < qe; ++i) {
    const int32_t e = misses_ranked[i];
    int slot = -1;
    for (int s = 0; s < p->n_slots; ++s)
      if (p->st.slot_key[s] < 0) { slot = s; break; }
    int32_t vl = -1, ve = -1;
    if (slot < 0) {
      uint64_t best = UINT64_MAX;
      for (int s = 0; s < p->n_slots; ++s) {
        const int32_t key = p->st.slot_key[s];
        const bool in_step = (key / E == layer) && p->seen[key % E] >= 0;
        if (!in_step && p->st.stamp[s] < best) { best = p->st.stamp[s]; slot = s; }
      }
      const int32_t old = p->st.slot_key[slot];
      vl = old / E;
      ve = old % E;
      p->st.where[old] = -1;
    }
    p->st.slot_key[slot] = layer * E + e;
    p->st.where[layer * E + e] = slot;
    p->st.stamp[slot] = ++p->st.clock;
    plan->fill_expert[i] = e;
    plan->fill_slot[i] = slot;
    plan->victim_layer[i] = vl;
    plan->victim_expert[i] = ve;
  }
  plan->q = qe;
  plan->n_host = nm - qe;
  for (int i = qe; i < nm; ++i) plan->host_expert[i - qe] = misses_ranked[i];
  clear_seen();
  return MOE_OK;
}

int planner_rollback(moe_planner* p) {
  if (!p) return set_error(MOE_EINVAL, "null planner");
  if (!p->have_saved) return set_error(MOE_ECACHE, "nothing to roll back");
  p->st = p->saved;
  p->have_saved = false;
  return MOE_OK;
}

// Rebuild under n_new slots: the n_new most recently used residents survive
// (ties to the lower slot) with their recency; a survivor below n_new keeps
// its slot, the others move in old-slot order into the free slots below
// n_new, ascending.  old_of_new[d] = the old slot of new slot d's expert (-1:
// empty).
int planner_resize(moe_planner* p, int32_t n_new, int32_t* old_of_new) {
  if (!p || !old_of_new) return set_error(MOE_EINVAL, "null pointer");
  if (n_new < 1) return set_error(MOE_EINVAL, "slot budget %d < 1", n_new);
  std::vector<int32_t> res;
  for (int32_t s = 0; s < p->n_slots; ++s)
    if (p->st.slot_key[s] >= 0) res.push_back(s);
  std::stable_sort(res.begin(), res.end(), [&](int32_t a, int32_t b) {
    if (p->st.stamp[a] != p->st.stamp[b]) return p->st.stamp[a] > p->st.stamp[b];
    return a < b;
  });
  const size_t keep = std::min<size_t>(res.size(), (size_t)n_new);
  std::vector<char> used(n_new, 0);
  std::vector<int32_t> movers;
  for (int32_t d = 0; d < n_new; ++d) old_of_new[d] = -1;
  for (size_t i = 0; i < keep; ++i) {
    const int32_t s = res[i];
    if (s < n_new) {
      old_of_new[s] = s;
      used[s] = 1;
    } else {
      movers.push_back(s);
    }
  }
  std::sort(movers.begin(), movers.end());
  int32_t d = 0;
  for (int32_t s : movers) {
    while (used[d]) ++d;
    old_of_new[d] = s;
    used[d] = 1;
  }
  PlannerState ns;
  ns.slot_key.assign(n_new, -1);
  ns.stamp.assign(n_new, 0);
  ns.where.assign(p->st.where.size(), -1);
  ns.clock = p->st.clock;
  for (int32_t t = 0; t < n_new; ++t) {
    const int32_t s = old_of_new[t];
    if (s < 0) continue;
    ns.slot_key[t] = p->st.slot_key[s];
    ns.stamp[t] = p->st.stamp[s];
    ns.where[ns.slot_key[t]] = t;
  }
  p->st = std::move(ns);
  p->n_slots = n_new;
  p->have_saved = false;
  return MOE_OK;
}

void planner_forget_slot(moe_planner* p, int32_t slot) {
  const int32_t key = p->st.slot_key[slot];
  if (key >= 0) p->st.where[key] = -1;
  p->st.slot_key[slot] = -1;
  p->st.stamp[slot] = 0;
}

int32_t planner_slot_key(const moe_planner* p, int32_t slot) { return p->st.slot_key[slot]; }

}  // namespace moe

extern "C" {

int moe_planner_create(moe_planner** out, int32_t n_layers, int32_t n_experts, int32_t n_slots) {
  if (!out) return set_error(MOE_EINVAL, "null output");
  *out = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_slots < 1 ||
      (int64_t)n_layers * n_experts > (int64_t)1 << 30)
    return set_error(MOE_EINVAL, "bad planner shape L=%d E=%d slots=%d", n_layers, n_experts,
                     n_slots);
  moe_planner* p = new (std::nothrow) moe_planner;
  if (!p) return set_error(MOE_EINVAL, "out of host memory");
  p->n_layers = n_layers;
  p->n_experts = n_experts;
  p->n_slots = n_slots;
  p->st.slot_key.assign(n_slots, -1);
  p->st.stamp.assign(n_slots, 0);
  p->st.where.assign((size_t)n_layers * n_experts, -1);
  p->weight.assign(n_experts, 0.f);
  p->seen.assign(n_experts, -1);
  *out = p;
  return MOE_OK;
}

void moe_planner_destroy(moe_planner* p) { delete p; }

int moe_planner_set_bandwidths(moe_planner* p, double b_pcie, double b_host) {
  if (!p || !(b_pcie > 0) || !(b_host > 0)) return set_error(MOE_EINVAL, "bad bandwidths");
  p->b_pcie = b_pcie;
  p->b_host = b_host;
  return MOE_OK;
}

int moe_planner_plan(moe_planner* p, int32_t layer, const int32_t* ids, const float* w, int32_t n,
                     int32_t q, moe_plan* plan) {
  return moe::planner_plan(p, layer, ids, w, n, q, plan);
}

int moe_planner_rollback(moe_planner* p) { return moe::planner_rollback(p); }

int moe_planner_resize(moe_planner* p, int32_t n_slots, int32_t* old_of_new) {
  return moe::planner_resize(p, n_slots, old_of_new);
}

int32_t moe_planner_n_slots(const moe_planner* p) { return p ? p->n_slots : -1; }

int moe_planner_slot_table(const moe_planner* p, int32_t layer, int32_t* out) {
  if (!p || !out) return set_error(MOE_EINVAL, "null pointer");
  if (layer < 0 || layer >= p->n_layers) return set_error(MOE_EINVAL, "layer out of range");
  std::memcpy(out, p->st.where.data() + (size_t)layer * p->n_experts,
              sizeof(int32_t) * p->n_experts);
  return MOE_OK;
}

}  // extern "C"

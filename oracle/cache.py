"""Oracle: global LRU expert cache and the q* miss split (test infrastructure).

What the pages fix:
  * GPU memory holds a cache of experts with least-recently-used
    replacement, one cache shared by all MoE layers, whose contents follow
    the router ("FreeToken 753b Model Explained", table in "How MoE Paging
    and Caching Work"; futuresignalnews.com article, "2. Semantic-Aware
    Caching");
  * a miss is either copied over PCIe, run on the GPU and kept cached, or
    run on the CPU against the host copy; the cache may start cold
    (explainx.ai guide, "Decode: decide whether to move an expert or compute
    where it lives"; futuresignalnews.com, "3. Elastic Memory Management");
  * q* is the number of misses sent to the GPU, chosen from the profiled
    pinned-PCIe and host bandwidths so that both paths run at the same time
    (explainx.ai, "Decode: ..."; futuresignalnews.com, "1. Bandwidth-Adaptive
    Execution (The q* Policy)").  The formula is not printed.

Readings taken (parity unpinned against the pages; pinned only against a
textbook LRU and brute force):
  * a step's selected set S is the distinct experts of its tokens; a hit
    refreshes recency, hits are touched in S order;
  * misses are ranked by total gate weight (descending), ties to the lower
    expert id, and the first q are filled; unfilled misses are not inserted;
  * a fill takes the lowest-index empty slot, else the least recently used
    slot whose expert is not in S; a filled expert becomes most recent;
  * q is clamped to the slots that can take a fill (n_slots - hits);
  * q* = argmin over q in [0, m] of max(q / B_pcie, (m - q) / B_host), ties
    to the larger q (the expert size cancels).

Elastic budget: the GPU expert cache can be rebuilt under a revised slot
budget at a scheduler safe point, without restarting or reloading the host
pool (futuresignalnews.com, "3. Elastic Memory Management"; "FreeToken 753b
Model Explained", "How MoE Paging and Caching Work").  Readings taken (parity
unpinned against the pages): the n' most recently used residents survive
(ties to the lower slot) and keep their recency; a survivor whose slot is
below n' stays there, the others move, in old-slot order, into the free slots
below n' in ascending order; the rest are evicted.
"""

import numpy as np


def qstar(m, b_pcie, b_host):
    """Number of the m misses to fill into the GPU cache."""
    if m <= 0:
        return 0
    best_q, best_t = 0, None
    for q in range(m + 1):
        t = max(q / b_pcie, (m - q) / b_host)
        if best_t is None or t <= best_t:
            best_q, best_t = q, t
    return best_q


def selected_experts(ids, w):
    """Distinct experts of one step in first-appearance order, with the
    total gate weight each one carries."""
    ids = np.asarray(ids).reshape(-1)
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    order, weight = [], {}
    for e, g in zip(ids.tolist(), w.tolist()):
        if e not in weight:
            order.append(e)
            weight[e] = 0.0
        weight[e] += g
    return order, weight


class LRUCache:
    """Plain global LRU over (layer, expert) keys with numbered slots."""

    def __init__(self, n_slots):
        self.n_slots = n_slots
        self.slot_key = [None] * n_slots     # slot -> (layer, expert)
        self.stamp = [0] * n_slots           # last-use clock per slot
        self.where = {}                      # (layer, expert) -> slot
        self.clock = 0

    def step(self, layer, ids, w, q):
        """One decode step of one layer.  Returns the plan as a dict."""
        S, weight = selected_experts(ids, w)
        hits = [e for e in S if (layer, e) in self.where]
        misses = [e for e in S if (layer, e) not in self.where]
        for e in hits:
            self.clock += 1
            self.stamp[self.where[(layer, e)]] = self.clock
        ranked = sorted(misses, key=lambda e: (-weight[e], e))
        q_eff = max(0, min(q, len(misses), self.n_slots - len(hits)))
        in_step = set((layer, e) for e in S)
        fills, victims = [], []
        for e in ranked[:q_eff]:
            empty = [s for s in range(self.n_slots) if self.slot_key[s] is None]
            if empty:
                slot = empty[0]
                victims.append(-1)
            else:
                cands = [s for s in range(self.n_slots)
                         if self.slot_key[s] not in in_step]
                slot = min(cands, key=lambda s: (self.stamp[s], s))
                old = self.slot_key[slot]
                victims.append(old[1])
                del self.where[old]
            self.slot_key[slot] = (layer, e)
            self.where[(layer, e)] = slot
            self.clock += 1
            self.stamp[slot] = self.clock
            fills.append((e, slot))
        host = [e for e in ranked[q_eff:]]
        return {"selected": S, "hits": hits, "misses": misses, "q": q_eff,
                "fills": fills, "victims": victims, "host": host}

    def resize(self, n_new):
        """Rebuild under a budget of n_new slots.  Returns old_of_new: for
        each new slot, the old slot its expert comes from (-1: empty)."""
        resident = [s for s in range(self.n_slots) if self.slot_key[s] is not None]
        resident.sort(key=lambda s: (-self.stamp[s], s))
        keep = resident[:n_new]
        for s in resident[n_new:]:
            del self.where[self.slot_key[s]]
        stay = sorted(s for s in keep if s < n_new)
        movers = sorted(s for s in keep if s >= n_new)
        free = [d for d in range(n_new) if d not in set(stay)]
        old_of_new = [-1] * n_new
        for s in stay:
            old_of_new[s] = s
        for s, d in zip(movers, free):
            old_of_new[d] = s
        key = [None] * n_new
        stamp = [0] * n_new
        for d, s in enumerate(old_of_new):
            if s >= 0:
                key[d] = self.slot_key[s]
                stamp[d] = self.stamp[s]
                self.where[key[d]] = d
        self.slot_key, self.stamp, self.n_slots = key, stamp, n_new
        return old_of_new

    def slot_of_expert(self, layer, n_experts):
        out = np.full(n_experts, -1, dtype=np.int32)
        for (l, e), s in self.where.items():
            if l == layer:
                out[e] = s
        return out


def lru_sim(trace_ids, trace_w, n_slots, n_experts, q=None, b_pcie=None,
            b_host=None, layer=0, resize_at=None):
    """Run a single-layer trace through the cache.

    trace_ids [steps, T, k] (or [steps, k]); trace_w same shape.
    q: a fixed per-step fill count, or None to use q* from the bandwidths.
    resize_at: optional {step: n_slots}: rebuild under that budget before
    the step.
    Returns (list of per-step plans, [steps, E] slot table after each step).
    """
    trace_ids = np.asarray(trace_ids)
    trace_w = np.asarray(trace_w)
    cache = LRUCache(n_slots)
    plans, tables = [], []
    for s in range(trace_ids.shape[0]):
        if resize_at and s in resize_at:
            cache.resize(resize_at[s])
        S, _ = selected_experts(trace_ids[s], trace_w[s])
        m = sum((layer, e) not in cache.where for e in S)
        qs = qstar(m, b_pcie, b_host) if q is None else q
        plans.append(cache.step(layer, trace_ids[s], trace_w[s], qs))
        tables.append(cache.slot_of_expert(layer, n_experts))
    return plans, np.stack(tables)

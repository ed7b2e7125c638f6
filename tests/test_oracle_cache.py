"""Pins of the oracle's LRU expert cache and q* split (CPU only)."""

import math
from collections import OrderedDict

import numpy as np
import pytest

import synth
from oracle import cache


def _textbook_lru(trace_ids, trace_w, n_slots, resize_at=None):
    """OrderedDict LRU over whole steps: hits refresh in selection order,
    then misses (heaviest first) are inserted, evicting the least recently
    used entry that is not part of the current step.  resize_at {step: n}:
    before that step the capacity becomes n and the least recently used
    entries beyond it are dropped.  Returns per-step (hits, misses, resident
    set, victims)."""
    od = OrderedDict()
    out = []
    for s, (ids, w) in enumerate(zip(trace_ids, trace_w)):
        if resize_at and s in resize_at:
            n_slots = resize_at[s]
            while len(od) > n_slots:
                od.popitem(last=False)
        sel, weight = [], {}
        for e, g in zip(np.ravel(ids).tolist(), np.ravel(w).tolist()):
            if e not in weight:
                sel.append(e)
                weight[e] = 0.0
            weight[e] += g
        hits = [e for e in sel if e in od]
        misses = [e for e in sel if e not in od]
        for e in hits:
            od.move_to_end(e)
        victims = []
        for e in sorted(misses, key=lambda e: (-weight[e], e)):
            if len(od) >= n_slots:
                victim = next(v for v in od if v not in weight)
                del od[victim]
                victims.append(victim)
            od[e] = True
        out.append((hits, misses, set(od), victims))
    return out


def _trace(steps=512, E=256, k=8, seed=0):
    return synth.zipf_trace(E, k, steps, 1.1, 32, seed=seed)


def test_lru_matches_ordereddict_on_zipf_trace():
    ids, w = _trace()
    plans, table = cache.lru_sim(ids, w, 64, 256, q=8)
    ref = _textbook_lru(ids, w, 64)
    for s, (p, (hits, misses, resident, victims)) in enumerate(zip(plans, ref)):
        assert p["hits"] == hits, s
        assert p["misses"] == misses, s
        assert set(np.nonzero(table[s] >= 0)[0].tolist()) == resident, s
        assert [v for v in p["victims"] if v >= 0] == victims, s
    # slot table is a partial injection expert -> slot
    for s in range(table.shape[0]):
        used = table[s][table[s] >= 0]
        assert len(set(used.tolist())) == used.size and np.all(used < 64)


def test_lru_enough_slots_misses_equal_distinct():
    ids, w = _trace(steps=200, E=64)
    plans, _ = cache.lru_sim(ids, w, 64, 64, q=8)
    n_miss = sum(len(p["misses"]) for p in plans)
    assert n_miss == len(np.unique(ids))


def test_repeated_selection_hits_after_first_step():
    ids = np.tile(np.array([[5, 9, 2, 7]]), (10, 1))
    w = np.tile(np.array([[0.4, 0.3, 0.2, 0.1]]), (10, 1))
    plans, _ = cache.lru_sim(ids, w, 8, 16, q=4)
    assert len(plans[0]["misses"]) == 4
    assert all(len(p["hits"]) == 4 and not p["misses"] for p in plans[1:])


def test_no_fills_means_nothing_resident():
    ids, w = _trace(steps=40)
    plans, table = cache.lru_sim(ids, w, 64, 256, q=0)
    assert np.all(table == -1)
    assert all(len(p["host"]) == len(p["misses"]) == len(p["selected"]) for p in plans)


def test_fills_take_heaviest_misses_and_empty_slots_first():
    c = cache.LRUCache(4)
    p = c.step(0, [3, 1, 2], [0.1, 0.5, 0.3], q=2)
    assert p["fills"] == [(1, 0), (2, 1)] and p["host"] == [3]
    p = c.step(0, [7, 1], [0.2, 0.2], q=2)     # 1 hits; 7 fills slot 2
    assert p["hits"] == [1] and p["fills"] == [(7, 2)]


def test_victim_is_lru_outside_current_step():
    c = cache.LRUCache(2)
    c.step(0, [1, 2], [0.5, 0.5], q=2)     # slots: 1 -> 0, 2 -> 1
    c.step(0, [1], [1.0], q=1)             # 1 refreshed; 2 is LRU
    p = c.step(0, [3], [1.0], q=1)
    assert p["fills"] == [(3, 1)] and p["victims"] == [2]
    # 2 and 3 both selected; 1 is the only evictable slot
    p = c.step(0, [3, 2], [0.6, 0.4], q=1)
    assert p["fills"] == [(2, 0)] and p["victims"] == [1]


def test_cache_is_global_across_layers():
    c = cache.LRUCache(2)
    c.step(0, [4], [1.0], q=1)
    p = c.step(1, [4], [1.0], q=1)        # same expert id, other layer
    assert p["misses"] == [4] and p["victims"] == [-1]
    p = c.step(2, [4], [1.0], q=1)        # full: evicts the layer-0 copy
    assert p["victims"] == [4]
    assert c.slot_of_expert(0, 8)[4] == -1 and c.slot_of_expert(1, 8)[4] >= 0


def test_q_clamped_to_slots_free_of_current_step():
    c = cache.LRUCache(3)
    c.step(0, [0, 1], [0.5, 0.5], q=2)
    p = c.step(0, [0, 1, 2, 3, 4], [0.3, 0.3, 0.2, 0.1, 0.1], q=3)
    assert p["q"] == 1 and len(p["host"]) == 2


def test_qstar_closed_form_and_balance():
    for m in range(0, 17):
        for bp, bh in [(51.5, 178.0), (11.8, 90.0), (50, 50), (64, 8), (1, 1000)]:
            q = cache.qstar(m, bp, bh)
            cost = lambda q_: max(q_ / bp, (m - q_) / bh)
            assert all(cost(q) <= cost(q2) for q2 in range(m + 1))
            a = m * bp / (bp + bh)                 # continuous balance point
            assert q in (math.floor(a), math.ceil(a))


def test_qstar_ties_go_to_more_fills():
    assert cache.qstar(3, 1.0, 1.0) == 2
    assert cache.qstar(4, 1.0, 1.0) == 2
    assert cache.qstar(0, 5.0, 1.0) == 0


def test_qstar_with_page_bandwidths():
    # 51.5 GB/s pinned PCIe and 178 GB/s host expert-kernel bandwidth
    # (explainx.ai guide, resource table): 8 misses -> 2 filled, 6 on the CPU
    assert cache.qstar(8, 51.5, 178.0) == 2


def test_resize_matches_ordereddict_on_zipf_trace():
    """Elastic budget 64 -> 32 -> 96 mid-trace: the survivors of a rebuild are
    the most recently used experts, and the cache then behaves as a textbook
    LRU of the new capacity."""
    ids, w = _trace()
    at = {170: 32, 340: 96}
    plans, table = cache.lru_sim(ids, w, 64, 256, q=8, resize_at=at)
    ref = _textbook_lru(ids, w, 64, resize_at=at)
    for s, (p, (hits, misses, resident, victims)) in enumerate(zip(plans, ref)):
        assert p["hits"] == hits, s
        assert p["misses"] == misses, s
        assert set(np.nonzero(table[s] >= 0)[0].tolist()) == resident, s
    for s in range(table.shape[0]):
        cap = 64 if s < 170 else (32 if s < 340 else 96)
        used = table[s][table[s] >= 0]
        assert len(set(used.tolist())) == used.size and np.all(used < cap), s


def test_resize_growth_moves_nothing():
    c = cache.LRUCache(4)
    c.step(0, [1, 2, 3], [0.5, 0.3, 0.2], q=3)
    before = (list(c.slot_key), list(c.stamp))
    m = c.resize(6)
    assert m == [0, 1, 2, -1, -1, -1]
    assert c.slot_key[:4] == before[0] and c.stamp[:4] == before[1]
    assert c.slot_key[4:] == [None, None]


def test_resize_shrink_placement():
    """Survivors below the new budget stay; the others fill the free slots
    below it in ascending order, taken in old-slot order."""
    c = cache.LRUCache(6)
    c.step(0, [10, 11, 12, 13, 14, 15], [6, 5, 4, 3, 2, 1], q=6)   # slots 0..5
    c.step(0, [15, 13, 11], [1, 1, 1], q=0)                           # touch 5, 3, 1
    m = c.resize(3)
    # most recent: 11 (slot 1), 13 (slot 3), 15 (slot 5); 1 stays, 3 -> 0, 5 -> 2
    assert m == [3, 1, 5]
    assert c.where == {(0, 13): 0, (0, 11): 1, (0, 15): 2}
    m = c.resize(1)
    assert m == [1] and c.where == {(0, 11): 0}     # 11 now sits in slot 1

"""C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-only logic (argument checks, workspace sizes, q*, the LRU planner)
matches the oracle.  No GPU compute call is made here."""

import ctypes
import os
import re

import numpy as np
import pytest

import synth
from conftest import ROOT
from oracle import cache as ocache

_lib_mod = pytest.importorskip("sparse_expert_execution_amd._lib")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib_mod.LIB_PATH):
        pytest.fail("libmoe.so not built: run python -m sparse_expert_execution_amd.build")
    return _lib_mod.lib()


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b((?:moe|cache)_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported(L):
    declared = _declared()
    assert len(declared) >= 25
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(_lib_mod.EXPORTS)
    assert L.moe_abi_version() == 1


def test_exported_symbols_are_c_names():
    out = os.popen(f"nm -D --defined-only {_lib_mod.LIB_PATH}").read()
    exported = set(re.findall(r" T (\w+)", out))
    assert _declared() <= exported


def _desc(**kw):
    base = dict(hidden=256, inter=128, n_experts=8, top_k=2, has_shared=0, renorm_topk=0,
                wtype=_lib_mod.WTYPE_MXFP4, router_wtype=_lib_mod.WTYPE_F32)
    base.update(kw)
    return _lib_mod.MoeDesc(**base)


def test_layout_sizes(L):
    off = (ctypes.c_size_t * 6)()
    n = ctypes.c_size_t()
    d = _desc(hidden=4096, inter=2048, n_experts=256, top_k=6)
    assert L.moe_expert_layout(ctypes.byref(d), off, ctypes.byref(n)) == 0
    assert n.value == 13_369_344
    assert list(off) == [0, 4194304, 4456448, 8650752, 8912896, 13107200]
    d = _desc(hidden=2048, inter=768, n_experts=128, top_k=8, wtype=_lib_mod.WTYPE_BF16)
    assert L.moe_expert_layout(ctypes.byref(d), off, ctypes.byref(n)) == 0
    assert n.value == 9_437_184 and list(off)[:3] == [0, 3145728, 6291456]


@pytest.mark.parametrize("field,value,status", [
    ("hidden", 100, -1), ("inter", 0, -1), ("top_k", 9, -1), ("top_k", 0, -1),
    ("n_experts", 2000, -1), ("wtype", 7, -2), ("router_wtype", 2, -2), ("has_shared", 3, -1),
])
def test_bad_descriptors_rejected(L, field, value, status):
    d = _desc(**{field: value})
    off = (ctypes.c_size_t * 6)()
    n = ctypes.c_size_t()
    assert L.moe_expert_layout(ctypes.byref(d), off, ctypes.byref(n)) == status
    assert L.moe_last_error()


def test_null_and_size_errors_before_any_device_work(L):
    d = _desc()
    P = ctypes.c_void_p
    fake = P(4096)
    # null output pointers
    assert L.moe_route(ctypes.byref(d), fake, fake, 4, None, fake, fake, 1 << 20, None) == -1
    assert L.moe_decode(ctypes.byref(d), fake, 4, fake, fake, None, None, None, fake, fake,
                        1 << 20, None) == -1
    # workspace too small
    assert L.moe_route(ctypes.byref(d), fake, fake, 4, fake, fake, fake, 8, None) == -4
    assert L.moe_decode(ctypes.byref(d), fake, 4, fake, fake, None, fake, None, fake, fake, 8,
                        None) == -4
    # T beyond the decode limit
    assert L.moe_decode(ctypes.byref(d), fake, 65, fake, fake, None, fake, None, fake, fake,
                        1 << 30, None) == -1
    # shared flag mismatch
    assert L.moe_decode(ctypes.byref(d), fake, 1, fake, fake, None, fake, fake, fake, fake,
                        1 << 20, None) == -1
    # prefill needs MXFP4
    db = _desc(wtype=_lib_mod.WTYPE_BF16)
    assert L.moe_prefill(ctypes.byref(db), fake, 4, fake, fake, None, fake, None, fake, fake,
                         1 << 30, None) == -2
    # T == 0 is a no-op
    assert L.moe_decode(ctypes.byref(d), None, 0, None, None, None, None, None, None, None, 0,
                        None) == 0
    assert L.moe_quantize_mxfp4(fake, 4, 40, 40, fake, fake, None) == -1


def test_workspace_sizes(L):
    d = _desc(hidden=4096, inter=2048, n_experts=256, top_k=6, has_shared=1)
    assert L.moe_workspace_bytes(ctypes.byref(d), 16, 1) >= 256 + 16 * 256 * 4
    # prefill: MXFP4 x and h, the sort and the per-pair outputs
    pre = L.moe_workspace_bytes(ctypes.byref(d), 4096, 2)
    assert pre >= 4096 * 4096 * 17 // 32 + 4096 * 7 * 2048 * 17 // 32 + 4096 * 7 * 4096 * 4
    assert L.moe_workspace_bytes(ctypes.byref(d), 4, 0) >= 256 + 4 * 256 * 4
    assert L.moe_workspace_bytes(ctypes.byref(d), 4, 9) == 0


@pytest.mark.parametrize("shape,wtype,want", [
    ((2048, 768), 1, 16),      # BF16: 16, x of 16 tokens fits the 120 KB stage
    ((4096, 1024), 1, 15),     # BF16: 120 KB / (2 H) tokens
    ((800, 96), 2, 16),        # MXFP4, H not a multiple of 128: the vector kernel
    ((4096, 2048), 2, 8),      # MXFP4 on the matrix core: BF16 x, its two
    ((6144, 2048), 2, 5),      #   e4m3 parts and scales in 144 KB of LDS
    ((4096, 128), 2, 15),      # MXFP4 with I not a multiple of 256: the vector kernel
    ((512, 256), 2, 8),
    ((4096, 2048), 3, 15),     # NVFP4: the vector kernel
])
def test_decode_launch_tokens(L, shape, wtype, want):
    """Per-launch token cap of the decode (the split of a larger batch)."""
    H, I = shape
    d = _desc(hidden=H, inter=I, n_experts=256, top_k=6, has_shared=1, wtype=wtype)
    assert L.moe_decode_launch_tokens(ctypes.byref(d)) == want
    bad = _desc(hidden=H, inter=I + 1, n_experts=256, top_k=6, has_shared=1, wtype=wtype)
    assert L.moe_decode_launch_tokens(ctypes.byref(bad)) < 0


def test_qstar_matches_oracle(L):
    for m in range(0, 20):
        for bp, bh in [(51.5, 178.0), (11.8, 90.0), (50, 50), (64, 8), (1, 1000), (3, 7)]:
            assert L.moe_qstar(m, bp, bh) == ocache.qstar(m, bp, bh)
    assert L.moe_qstar(-1, 1.0, 1.0) == -1
    assert L.moe_qstar(3, 0.0, 1.0) == -1


def _run_planner(ids, w, n_slots, E, q=None, bw=None, layers=None):
    from sparse_expert_execution_amd import ops
    n_layers = 1 if layers is None else max(layers) + 1
    p = ops.Planner(n_layers, E, n_slots)
    if bw:
        p.set_bandwidths(*bw)
    plans, tables = [], []
    for s in range(ids.shape[0]):
        layer = 0 if layers is None else layers[s]
        pl = p.plan(layer, ids[s], w[s], -1 if q is None else q)
        plans.append(ops.plan_dict(pl))
        tables.append(p.slot_table(layer))
    return plans, np.stack(tables)


@pytest.mark.parametrize("q,bw", [(8, None), (3, None), (None, (51.5, 178.0)),
                                  (None, (40.0, 40.0))])
def test_planner_matches_oracle_lru_on_zipf_trace(q, bw):
    ids, w = synth.zipf_trace(256, 8, 512, 1.1, 32)
    got, table = _run_planner(ids, w, 64, 256, q=q, bw=bw)
    kw = {"q": q} if q is not None else {"b_pcie": bw[0], "b_host": bw[1]}
    ref, ref_table = ocache.lru_sim(ids, w, 64, 256, **kw)
    assert np.array_equal(table, ref_table)
    for g, r in zip(got, ref):
        assert g["selected"] == r["selected"]
        assert g["hits"] == r["hits"] and g["misses"] == r["misses"]
        assert g["q"] == r["q"] and g["fills"] == r["fills"] and g["host"] == r["host"]
        assert [v[1] if v[0] >= 0 else -1 for v in g["victims"]] == r["victims"]


def test_planner_resize_matches_oracle_on_zipf_trace():
    """Elastic budget 64 -> 32 -> 96 -> 8 mid-trace, across two layers: the
    planner's tables and move maps equal the oracle's after every step."""
    from sparse_expert_execution_amd import ops
    ids, w = synth.zipf_trace(256, 8, 400, 1.1, 32)
    at = {100: 32, 200: 96, 300: 8}
    p = ops.Planner(2, 256, 64)
    p.set_bandwidths(51.5, 178.0)
    c = ocache.LRUCache(64)
    for s in range(ids.shape[0]):
        if s in at:
            assert list(p.resize(at[s])) == c.resize(at[s])
            assert p.n_slots == at[s]
        layer = s % 2
        S, _ = ocache.selected_experts(ids[s], w[s])
        m = sum((layer, e) not in c.where for e in S)
        r = c.step(layer, ids[s], w[s], ocache.qstar(m, 51.5, 178.0))
        g = ops.plan_dict(p.plan(layer, ids[s], w[s], -1))
        assert g["hits"] == r["hits"] and g["fills"] == r["fills"], s
        for l in range(2):
            assert np.array_equal(p.slot_table(l), c.slot_of_expert(l, 256)), s


def test_planner_resize_errors():
    from sparse_expert_execution_amd import ops
    p = ops.Planner(1, 8, 4)
    with pytest.raises(_lib_mod.MoeError):
        p.resize(0)
    p.plan(0, np.array([1, 2], np.int32), np.array([0.5, 0.5], np.float32), 2)
    p.resize(2)
    with pytest.raises(_lib_mod.MoeError):      # a rebuild drops the rollback level
        p.rollback()


def test_planner_global_across_layers_matches_oracle():
    rng = np.random.default_rng(4)
    steps, E = 300, 16
    ids = np.stack([rng.choice(E, size=4, replace=False) for _ in range(steps)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, size=(steps, 4)).astype(np.float32)
    layers = rng.integers(0, 3, size=steps)
    got, _ = _run_planner(ids, w, 6, E, q=3, layers=list(layers))
    c = ocache.LRUCache(6)
    for s in range(steps):
        r = c.step(int(layers[s]), ids[s], w[s], 3)
        g = got[s]
        assert g["hits"] == r["hits"] and g["fills"] == r["fills"]
        assert [v[1] if v[0] >= 0 else -1 for v in g["victims"]] == r["victims"]


def test_planner_errors_and_rollback():
    from sparse_expert_execution_amd import ops
    p = ops.Planner(2, 8, 4)
    p.plan(0, [1, 2], [0.5, 0.5], 2)
    before = p.slot_table(0).copy()
    with pytest.raises(_lib_mod.MoeError) as ei:
        p.plan(0, [1, 9], [0.5, 0.5], 2)          # id out of range
    assert ei.value.status == -1
    assert np.array_equal(p.slot_table(0), before)
    with pytest.raises(_lib_mod.MoeError):
        p.plan(5, [1], [1.0], 1)                   # layer out of range
    with pytest.raises(_lib_mod.MoeError):
        p.plan(0, [1], [1.0], -1)                  # q* without bandwidths
    p.plan(0, [3, 4], [0.5, 0.5], 2)
    assert sorted(np.nonzero(p.slot_table(0) >= 0)[0].tolist()) == [1, 2, 3, 4]
    p.rollback()
    assert np.array_equal(p.slot_table(0), before)
    with pytest.raises(_lib_mod.MoeError):
        p.rollback()                               # only one level


def test_layer_stream_argument_checks():
    """moe_layer_stream_create rejects bad arguments before any HIP call."""
    L = _lib_mod.lib()
    out = ctypes.c_void_p()
    host = ctypes.create_string_buffer(1024)
    dev = ctypes.create_string_buffer(1024)
    assert L.moe_layer_stream_create(None, host, 2, 512, dev, None) == _lib_mod.MOE_EINVAL
    assert L.moe_layer_stream_create(ctypes.byref(out), None, 2, 512, dev, None) == \
        _lib_mod.MOE_EINVAL
    assert L.moe_layer_stream_create(ctypes.byref(out), host, 0, 512, dev, None) == \
        _lib_mod.MOE_EINVAL
    assert L.moe_layer_stream_create(ctypes.byref(out), host, 2, 0, dev, None) == \
        _lib_mod.MOE_EINVAL
    # overlapping buffers
    base = ctypes.addressof(dev)
    assert L.moe_layer_stream_create(ctypes.byref(out), host, 2, 512, ctypes.c_void_p(base),
                                     ctypes.c_void_p(base + 256)) == _lib_mod.MOE_EINVAL
    assert not out.value

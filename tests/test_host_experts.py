"""The host side of the exact split (moe_host_experts) against the fp64 oracle,
on the CPU.  Expert blocks are assembled here from seeded fp32 draws with the
oracle's own BF16 / MXFP4 / NVFP4 encoders, in the documented block layout
(gate codes, gate scales, up codes, up scales, down codes, down scales, and
for NVFP4 the three fp32 matrix scales; BF16: gate, up, down), so nothing on
the input or expected side comes from the library.
"""

import os

import numpy as np
import pytest
import torch

import synth
from conftest import ROOT
from oracle import formats, layer as olayer

_lib_mod = pytest.importorskip("sparse_expert_execution_amd._lib")

TOL = 1e-4          # fp32 accumulation against fp64


@pytest.fixture(scope="module")
def ops():
    if not os.path.exists(_lib_mod.LIB_PATH):
        pytest.fail("libmoe.so not built: run python -m sparse_expert_execution_amd.build")
    from sparse_expert_execution_amd import ops as o
    return o


def _block(mats, wtype):
    """One expert block in the documented layout, plus the exact fp64 values."""
    parts, exact, gs = [], [], []
    for m in mats:
        a = m.numpy()
        if wtype == "bf16":
            bits = formats.bf16_round(a)
            parts.append(bits.astype(np.uint16).view(np.uint8).ravel())
            exact.append(formats.bf16_decode(bits))
        elif wtype == "nvfp4":
            codes, scales, g = formats.nvfp4_encode(a)
            parts += [codes.ravel(), scales.ravel()]
            gs.append(g)
            exact.append(formats.nvfp4_decode(codes, scales, g))
        else:
            codes, scales = formats.mxfp4_encode(a)
            parts += [codes.ravel(), scales.ravel()]
            exact.append(formats.mxfp4_decode(codes, scales))
    if wtype == "nvfp4":            # the three fp32 matrix scales after the down scales
        parts.append(np.array(gs + [0.0], dtype=np.float32).view(np.uint8))
    raw = np.concatenate(parts)
    pad = (-raw.size) % 256
    return np.concatenate([raw, np.zeros(pad, np.uint8)]), tuple(exact)


def _pool(name, wtype, experts):
    blocks, exact = [], {}
    for e in experts:
        b, ex = _block(synth.expert_weights(name, 0, e, device="cpu", as_dtype=torch.float32),
                       wtype)
        blocks.append(b)
        exact[e] = ex
    return np.stack(blocks), exact


def _desc(ops, name, wtype):
    s = synth.SHAPES[name]
    return ops.make_desc(s["hidden"], s["inter"], s["n_experts"], s["top_k"], wtype=wtype,
                         router_wtype="bf16")


def _route(name, T, seed=0):
    s = synth.SHAPES[name]
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(s["n_experts"], size=s["top_k"], replace=False)
                    for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 0.5, size=ids.shape).astype(np.float32)
    return ids, w


def _run(ops, desc, x, ids, w, pool, include=None, host_index=None, threads=0):
    T, H = x.shape
    y = torch.full((T, H), float("nan"), dtype=torch.float32)
    inc = None if include is None else torch.from_numpy(include.astype(np.uint8))
    hi = None if host_index is None else torch.from_numpy(host_index.astype(np.int32))
    ops.host_experts(desc, x, torch.from_numpy(ids), torch.from_numpy(w),
                     torch.from_numpy(pool.ravel()), y, include=inc, host_index=hi,
                     threads=threads)
    return y.numpy().astype(np.float64)


def _expect(x, ids, w, exact, include=None):
    xs = formats.bf16_decode(x.view(torch.int16).numpy().view(np.uint16))
    return olayer.combine(xs, ids, w, exact, include=include)


@pytest.mark.parametrize("name,wtype,T", [("tiny", "bf16", 4), ("tiny", "mxfp4", 4),
                                          ("tiny", "nvfp4", 4), ("ragged_decode", "nvfp4", 5),
                                          ("ragged_decode", "mxfp4", 5),
                                          ("ragged_prefill", "mxfp4", 9),
                                          ("small_cache", "mxfp4", 1)])
def test_host_experts_match_oracle(ops, name, wtype, T):
    s = synth.SHAPES[name]
    desc = _desc(ops, name, wtype)
    ids, w = _route(name, T)
    pool, exact = _pool(name, wtype, range(s["n_experts"]))
    _, eb = ops.expert_layout(desc)
    assert pool.shape[1] == eb                     # documented layout, same size
    x = synth.tokens(name, 0, T, device="cpu")
    got = _run(ops, desc, x, ids, w, pool)
    ref = _expect(x, ids, w, exact)
    assert olayer.row_rel_error(got, ref) < TOL


def test_host_experts_qwen_full_size(ops):
    name = "qwen_bf16_decode"
    desc = _desc(ops, name, "bf16")
    ids, w = _route(name, 1, seed=3)
    experts = [int(e) for e in ids[0]]
    blocks, exact = _pool(name, "bf16", experts)
    index = np.full(synth.SHAPES[name]["n_experts"], -1, np.int32)
    index[experts] = np.arange(len(experts))
    x = synth.tokens(name, 0, 1, device="cpu")
    got = _run(ops, desc, x, ids, w, blocks, host_index=index)
    assert olayer.row_rel_error(got, _expect(x, ids, w, exact)) < TOL


def test_host_experts_subset_merges_with_complement(ops):
    """include mask: the host partial over one subset plus the partial over
    the complement is the full layer (the exact split)."""
    name = "ragged_prefill"
    s = synth.SHAPES[name]
    desc = _desc(ops, name, "mxfp4")
    ids, w = _route(name, 7, seed=5)
    pool, exact = _pool(name, "mxfp4", range(s["n_experts"]))
    x = synth.tokens(name, 0, 7, device="cpu")
    rng = np.random.default_rng(9)
    inc = rng.random(ids.shape) < 0.5
    a = _run(ops, desc, x, ids, w, pool, include=inc)
    b = _run(ops, desc, x, ids, w, pool, include=~inc)
    full = _expect(x, ids, w, exact)
    assert olayer.row_rel_error(a, _expect(x, ids, w, exact, include=inc)) < TOL
    assert olayer.row_rel_error(a + b, full) < TOL


def test_host_experts_thread_count_invariant(ops):
    name = "ragged_decode"
    s = synth.SHAPES[name]
    desc = _desc(ops, name, "mxfp4")
    ids, w = _route(name, 6, seed=2)
    pool, _ = _pool(name, "mxfp4", range(s["n_experts"]))
    x = synth.tokens(name, 0, 6, device="cpu")
    y1 = _run(ops, desc, x, ids, w, pool, threads=1)
    y4 = _run(ops, desc, x, ids, w, pool, threads=4)
    assert np.array_equal(y1, y4)


def test_host_experts_errors(ops):
    name = "small_cache"
    desc = _desc(ops, name, "mxfp4")
    ids, w = _route(name, 1)
    pool, _ = _pool(name, "mxfp4", range(2))
    index = np.full(synth.SHAPES[name]["n_experts"], -1, np.int32)
    x = synth.tokens(name, 0, 1, device="cpu")
    with pytest.raises(_lib_mod.MoeError) as ei:
        _run(ops, desc, x, ids, w, pool, host_index=index)   # expert without a block
    assert ei.value.status == -1
    bad = ids.copy()
    bad[0, 0] = 999
    with pytest.raises(_lib_mod.MoeError):
        _run(ops, desc, x, bad, w, pool)


def test_host_expert_rate_positive(ops):
    name = "small_cache"
    desc = _desc(ops, name, "mxfp4")
    pool, _ = _pool(name, "mxfp4", range(4))
    r = ops.host_expert_rate(desc, torch.from_numpy(pool.ravel()), n_experts=4, reps=2)
    assert r > 0


@pytest.mark.parametrize("isa", ["scalar", "avx2", "avx512"])
def test_host_experts_every_isa_path(isa):
    """The row-dot paths a CPU without AVX512-BF16 (or AVX-512, or AVX2) would
    take, forced through MOE_HOST_ISA in a fresh process (the level is read
    once per process): the oracle comparisons above must hold on each."""
    import subprocess
    import sys
    env = dict(os.environ, MOE_HOST_ISA=isa)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                        "test_host_experts.py"), "-q", "-k", "match_oracle",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert " passed" in r.stdout

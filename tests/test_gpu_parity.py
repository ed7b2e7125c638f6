"""GPU parity: every HIP entry point against the fp64 oracle, through the C ABI.

Bars: bit-exact for MXFP4 codes, dequantised values, top-k ids (where the
oracle's probability gap between ranks k and k+1 exceeds 1e-4), slot tables
and merges; per-token max-abs error / max-abs reference <= 1e-2 for layer
outputs (fp32 accumulation on the GPU).
"""

import sys

import numpy as np
import pytest
import torch

import synth
from helpers import GpuLayer, bf16_to_f64, desc_for, oracle_combine, oracle_router
from oracle import cache as ocache
from oracle import formats, layer as olayer

pytestmark = pytest.mark.gpu

TOL = 1e-2
GAP = 1e-4


def _say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ops():
    from sparse_expert_execution_amd import ops as _ops
    _ops._lib.lib()
    return _ops


# ---------------------------------------------------------------- formats
def test_dequant_bit_exact_all_codes_and_scales(ops):
    _say("dequant all bytes x scales")
    scales = [0, 1, 100, 120, 127, 134, 254]
    codes = np.tile(np.arange(256, dtype=np.uint8).reshape(16, 16), (len(scales), 1))
    sc = np.repeat(np.array(scales, dtype=np.uint8), 16)
    d_codes = torch.from_numpy(codes).cuda()
    d_sc = torch.from_numpy(sc).cuda()
    out = torch.empty(codes.shape[0] * 32, dtype=torch.float32, device="cuda")
    ops.dequant_mxfp4(d_codes, d_sc, out)
    torch.cuda.synchronize()
    ref = formats.mxfp4_decode(codes.reshape(-1, 16), sc.reshape(-1, 1)).reshape(-1)
    with np.errstate(over="ignore"):
        ref32 = ref.astype(np.float32)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref32.view(np.uint32))


@pytest.mark.parametrize("wtype", ["mxfp4", "nvfp4"])
def test_dot_fp4_bit_exact_all_codes_and_scales(ops, wtype):
    """The decode gate/up rows' block step (FP4 -> BF16 convert, fp32 dot with
    BF16 x, then the block scale): with x one-hot at each of the 32 positions
    the result is one element's value, bit for bit the oracle's decode, over
    every code byte and a range of scale bytes; with random x it is the fp64
    dot within fp32 summation error."""
    _say("dot fp4", wtype)
    codes = np.tile(np.arange(256, dtype=np.uint8).reshape(16, 16), (8, 1))
    nb = codes.shape[0]
    if wtype == "mxfp4":
        scales = np.repeat(np.array([0, 1, 100, 120, 127, 134, 200, 254], dtype=np.uint8), 16)
        ref = formats.mxfp4_decode(codes, scales.reshape(-1, 1))
        sc_dev = torch.from_numpy(scales).cuda()
    else:
        # E4M3 scale bytes: subnormal, small, unit, large, the largest (448)
        pairs = np.array([[1, 7], [8, 56], [56, 57], [100, 126], [120, 64], [0x3f, 0x40],
                          [2, 0x7e], [0x30, 0x31]], dtype=np.uint8)
        scales = np.repeat(pairs, 16, axis=0)
        ref = formats.nvfp4_decode(codes, scales, np.float32(1.0))
        sc_dev = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    one_hot = np.zeros((32, 32), dtype=np.uint16)
    one_hot[np.arange(32), np.arange(32)] = 0x3F80            # bf16 1.0
    x = torch.from_numpy(one_hot.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty((nb, 32), dtype=torch.float32, device="cuda")
    ops.dot_fp4(wtype, torch.from_numpy(codes).cuda(), sc_dev, x, out)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):
        ref32 = ref.astype(np.float32)
    # a dot product starts from +0, so a -0 element comes out as +0
    ref32 = ref32 + np.float32(0.0)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref32.view(np.uint32))
    rng = np.random.default_rng(12)
    xr = torch.randn((5, 32), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    out = torch.empty((nb, 5), dtype=torch.float32, device="cuda")
    ops.dot_fp4(wtype, torch.from_numpy(codes).cuda(), sc_dev, xr.cuda(), out)
    torch.cuda.synchronize()
    dot = ref @ bf16_to_f64(xr).T
    scale = np.abs(ref) @ np.abs(bf16_to_f64(xr)).T
    got = out.cpu().numpy().astype(np.float64)
    finite = scale < 1e38                  # no fp32 overflow on the way
    assert np.all(np.abs(got - dot)[finite] <= 64 * 2.0 ** -24 * scale[finite] + 1e-45)
    del rng


def _encode_cases():
    rng = np.random.default_rng(1)
    rows = [rng.standard_normal(256) * 0.02, rng.standard_normal(256),
            rng.standard_normal(256) * 1e-30, rng.standard_normal(256) * 1e30,
            np.zeros(256), -np.zeros(256)]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) * 2.0 ** -3
    ties[0] = 4.0 * 2.0 ** -3            # block max at 4 * 2^X pins the scale
    rows.append(np.concatenate([ties, -ties, ties * 2 ** 20, -ties * 2 ** -100,
                                ties * 3, ties * 7.9, ties * 1e-3, ties]))
    sub = rng.standard_normal(256) * 2.0 ** -140   # fp32 denormals
    rows.append(sub)
    return np.stack(rows).astype(np.float32)


def test_quantize_bit_exact(ops):
    _say("quantize edge + random rows")
    src = _encode_cases()
    rng = np.random.default_rng(2)
    big = (rng.standard_normal((300, 4096)) * 0.02).astype(np.float32)
    for a in (src, big):
        d = torch.from_numpy(a).cuda()
        c = torch.empty((a.shape[0], a.shape[1] // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((a.shape[0], a.shape[1] // 32), dtype=torch.uint8, device="cuda")
        ops.quantize_mxfp4(d, c, s)
        torch.cuda.synchronize()
        rc, rs = formats.mxfp4_encode(a.astype(np.float64))
        assert np.array_equal(s.cpu().numpy(), rs)
        assert np.array_equal(c.cpu().numpy(), rc)


def _nvfp4_sections(ops, desc, blk):
    """(codes, scales, g) of gate, up and down from a packed NVFP4 block."""
    off, _ = ops.expert_layout(desc)
    H, I = desc.hidden, desc.inter
    b = blk.cpu().numpy()
    gs = b[off[5] + H * I // 16:off[5] + H * I // 16 + 12].view(np.float32)
    out = []
    for m, (rows, K) in enumerate([(I, H), (I, H), (H, I)]):
        c = b[off[2 * m]:off[2 * m] + rows * K // 2].reshape(rows, K // 2)
        sc = b[off[2 * m + 1]:off[2 * m + 1] + rows * K // 16].reshape(rows, K // 16)
        out.append((c, sc, gs[m]))
    return out


def test_nvfp4_pack_bit_exact(ops):
    """moe_pack_expert with NVFP4 weights against the oracle encoder: codes,
    E4M3 scales and the fp32 matrix scales, byte for byte (edge-case rows in
    the gate matrix, synthetic experts of two shapes)."""
    _say("nvfp4 pack")
    rng = np.random.default_rng(13)
    cases = []
    gate = (rng.standard_normal((128, 256)) * 0.02).astype(np.float32)
    edge = _encode_cases()
    gate[:edge.shape[0]] = edge[:, :256]
    gate[-1, :16] = 0.0                                   # an all-zero block
    cases.append(("tiny", [torch.from_numpy(gate).cuda(),
                           torch.from_numpy((rng.standard_normal((128, 256)) * 3).astype(
                               np.float32)).cuda(),
                           torch.from_numpy((rng.standard_normal((256, 128)) * 1e-3).astype(
                               np.float32)).cuda()]))
    cases.append(("dsv4_mxfp4_decode",
                  list(synth.expert_weights("dsv4_mxfp4_decode", 0, 5, device="cuda",
                                            as_dtype=torch.float32))))
    for name, mats in cases:
        desc = desc_for(name, "nvfp4")
        _, eb = ops.expert_layout(desc)
        blk = torch.zeros(eb, dtype=torch.uint8, device="cuda")
        ops.pack_expert(desc, blk, *mats)
        torch.cuda.synchronize()
        for m, (c, sc, g) in zip(mats, _nvfp4_sections(ops, desc, blk)):
            rc, rs, rg = formats.nvfp4_encode(m.cpu().numpy())
            assert np.float32(g).tobytes() == np.float32(rg).tobytes(), name
            assert np.array_equal(sc, rs), name
            assert np.array_equal(c, rc), name


def test_wave_scan_dpp(ops):
    """The DPP inclusive wave scan the decode expert list uses, against a
    prefix sum: counts, signed values, and values with every row boundary
    set."""
    _say("wave scan")
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.integers(0, 9, 64 * 16), rng.integers(-1000, 1000, 64 * 16),
                           np.where(np.arange(64 * 4) % 16 == 15, 1 << 20, 1)]).astype(np.int32)
    inp = torch.from_numpy(vals).cuda()
    out = torch.empty_like(inp)
    ops.wave_scan(inp, out)
    torch.cuda.synchronize()
    ref = np.cumsum(vals.reshape(-1, 64).astype(np.int64), axis=1).astype(np.int32).ravel()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_merge_exact(ops):
    _say("merge")
    rng = np.random.default_rng(3)
    for n in (1, 7, 4096 * 16 + 3):
        a = rng.standard_normal(n).astype(np.float32)
        b = rng.standard_normal(n).astype(np.float32)
        da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        y = torch.empty_like(da)
        ops.merge_partials(da, db, y)
        ops.merge_partials(da, db, da)          # aliasing y == a
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), a + b)
        assert np.array_equal(da.cpu().numpy(), a + b)


# ------------------------------------------------------------ MFMA layout
@pytest.mark.parametrize("scale_mode", ["unit", "random"])
def test_mfma_fp4_tile_layout(ops, scale_mode):
    _say("mfma tile", scale_mode)
    rng = np.random.default_rng(4)
    ac = rng.integers(0, 256, size=(16, 64), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(16, 64), dtype=np.uint8)
    if scale_mode == "unit":
        a_s = np.full((16, 4), 127, dtype=np.uint8)
        b_s = np.full((16, 4), 127, dtype=np.uint8)
    else:
        a_s = rng.integers(120, 135, size=(16, 4), dtype=np.uint8)
        b_s = rng.integers(120, 135, size=(16, 4), dtype=np.uint8)
    out = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    ops.mfma_fp4_tile(*(torch.from_numpy(v).cuda() for v in (ac, a_s, bc, b_s)), out)
    torch.cuda.synchronize()
    A = formats.mxfp4_decode(ac, a_s)
    B = formats.mxfp4_decode(bc, b_s)
    ref = A @ B.T
    got = out.cpu().numpy().astype(np.float64)
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref)) / scale
    hint = {"transposed": np.max(np.abs(got - ref.T)) / scale}
    assert err < 1e-6, f"mfma layout mismatch err={err} hints={hint}"


# ----------------------------------------------------------------- router
def _check_topk(r, gi, gw, k, renorm=False):
    """GPU top-k against the oracle's routing r.  Tokens whose fp64 gap
    between ranks k and k+1 exceeds GAP must match exactly; every token,
    including the near-tied ones, must hold k distinct ids in descending
    probability (within GAP), every expert clearly above the k-th probability
    and none clearly below it, with weights equal to the oracle's p at the
    GPU's ids (renormalised when asked)."""
    clear = r["gap"] > GAP
    assert np.array_equal(gi[clear], r["ids"][clear])
    assert np.allclose(gw[clear], r["w"][clear], rtol=1e-4, atol=1e-7)
    for t in range(gi.shape[0]):
        p = r["p"][t]
        sel = gi[t]
        assert np.all((sel >= 0) & (sel < p.size)), t
        assert np.unique(sel).size == k, ("repeated id", t, sel)
        ps = p[sel]
        assert np.all(ps[:-1] >= ps[1:] - GAP), ("not descending", t, ps)
        kth = np.sort(p)[::-1][k - 1]
        assert np.all(ps >= kth - GAP), ("below the k-th", t)
        must = np.nonzero(p > kth + GAP)[0]
        assert np.all(np.isin(must, sel)), ("missed a clear top-k expert", t)
        ref_w = ps / ps.sum() if renorm else ps
        assert np.allclose(gw[t], ref_w, rtol=1e-4, atol=1e-7), ("weights", t)


def _check_route(ops, name, T, renorm=False, layer=0):
    s = synth.SHAPES[name]
    from helpers import desc_for
    desc = desc_for(name, renorm=renorm)
    wr = synth.router_weights(name, layer, device="cuda")
    x = synth.tokens(name, layer, T, device="cuda")
    ids = torch.empty((T, s["top_k"]), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s["top_k"]), dtype=torch.float32, device="cuda")
    ws = ops.workspace(desc, T, 0)
    ops.route(desc, x, wr, ids, w, ws)
    torch.cuda.synchronize()
    r = olayer.route(bf16_to_f64(x), oracle_router(name, layer), s["top_k"], renorm=renorm)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    _check_topk(r, gi, gw, s["top_k"], renorm)
    return gi


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 100), ("qwen_bf16_decode", 1),
                                    ("qwen_bf16_decode", 8), ("dsv4_mxfp4_decode", 1),
                                    ("dsv4_mxfp4_decode", 16), ("dsv4_mxfp4_decode", 300),
                                    ("glm_cache_decode", 3), ("ragged_decode", 64),
                                    ("qwen_bf16_decode", 130), ("ragged_decode", 200),
                                    ("dsv4_mxfp4_prefill", 4096), ("many_experts", 1),
                                    ("many_experts", 16), ("many_experts", 100)])
def test_route_topk_exact(ops, name, T):
    _say("route", name, T)
    _check_route(ops, name, T)


def test_route_renorm(ops):
    _say("route renorm")
    _check_route(ops, "qwen_bf16_decode", 8, renorm=True)


# ----------------------------------------------------------------- decode
def _run_decode(ops, L, x, ids, w, slot_of=None, fn="decode"):
    T = x.shape[0]
    y = torch.full((T, L.s["hidden"]), float("nan"), dtype=torch.float32, device="cuda")
    mode = 1 if fn == "decode" else 2
    ws = ops.workspace(L.desc, T, mode)
    getattr(ops, fn)(L.desc, x, ids, w, L.pool, y, ws, slot_of=slot_of, shared=L.shared)
    torch.cuda.synchronize()
    if fn == "decode":
        assert ops.decode_status(ws) == 0, "a wait inside the decode kernel expired"
    return y.cpu().numpy().astype(np.float64)


def _oracle_out(L, x, ids, w, tokens=None, include=None, prefill=False, with_shared=True):
    s = L.s
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    xs = bf16_to_f64(x)[tok]
    ids_t, w_t = ids[tok], w[tok].astype(np.float64)
    inc = None if include is None else include[tok]
    shared_id = s["n_experts"] if (s["shared"] and with_shared) else None
    return oracle_combine(L.name, L.layer, L.wtype, xs, ids_t, w_t, shared_id=shared_id,
                          prefill=prefill, include=inc)


def _route_gpu(ops, L, x):
    T = x.shape[0]
    k = L.s["top_k"]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ops.route(L.desc, x, L.w_router, ids, w, ops.workspace(L.desc, T, 0))
    return ids, w


@pytest.mark.parametrize("wtype", ["bf16", "mxfp4"])
@pytest.mark.parametrize("T", [1, 4])
def test_decode_tiny(ops, wtype, T):
    _say("decode tiny", wtype, T)
    L = GpuLayer("tiny", wtype=wtype)
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w)
    ref = _oracle_out(L, x, ids.cpu().numpy(), w.cpu().numpy())
    assert olayer.row_rel_error(y, ref) < TOL


@pytest.mark.parametrize("T", [1, 5, 33, 64])
def test_decode_ragged_shapes(ops, T):
    _say("decode ragged", T)
    L = GpuLayer("ragged_decode")
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w)
    ref = _oracle_out(L, x, ids.cpu().numpy(), w.cpu().numpy())
    assert olayer.row_rel_error(y, ref) < TOL


@pytest.mark.parametrize("name", ["ragged_decode", "mfma_decode"])
def test_decode_partial_over_resident_subset(ops, name):
    """Non-resident experts are skipped; the two partial sums merge exactly."""
    _say("decode partial + merge", name)
    L = GpuLayer(name)
    T, E = 9, L.s["n_experts"]
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    rng = np.random.default_rng(5)
    resident = rng.random(E) < 0.5
    slot_of = torch.from_numpy(np.where(resident, np.arange(E), -1).astype(np.int32)).cuda()
    y_gpu = _run_decode(ops, L, x, ids, w, slot_of=slot_of)
    hi, hw = ids.cpu().numpy(), w.cpu().numpy()
    inc = resident[hi]
    ref_gpu = _oracle_out(L, x, hi, hw, include=inc)
    assert olayer.row_rel_error(y_gpu, ref_gpu) < TOL
    # host side: the other subset (oracle), merged on the GPU
    ref_host = _oracle_out(L, x, hi, hw, include=~inc, with_shared=False)
    a = torch.from_numpy(y_gpu.astype(np.float32)).cuda()
    b = torch.from_numpy(ref_host.astype(np.float32)).cuda()
    out = torch.empty_like(a)
    ops.merge_partials(a, b, out)
    torch.cuda.synchronize()
    full = _oracle_out(L, x, hi, hw)
    assert olayer.row_rel_error(out.cpu().numpy(), full) < TOL


@pytest.mark.parametrize("T", [1, 8])
def test_decode_qwen_full_layer(ops, T):
    _say("decode qwen full", T)
    L = GpuLayer("qwen_bf16_decode", layer=3)
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w)
    ref = _oracle_out(L, x, ids.cpu().numpy(), w.cpu().numpy())
    assert olayer.row_rel_error(y, ref) < TOL


@pytest.mark.parametrize("T,sample", [(1, [0]), (4, [0, 1, 2, 3]),
                                      (16, [0, 2, 5, 7, 8, 11, 13, 15])])
def test_decode_dsv4_full_layer_sampled(ops, T, sample):
    _say("decode dsv4 full", T)
    L = GpuLayer("dsv4_mxfp4_decode", layer=7)
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w)
    assert np.all(np.isfinite(y))
    ref = _oracle_out(L, x, ids.cpu().numpy(), w.cpu().numpy(), tokens=sample)
    assert olayer.row_rel_error(y[sample], ref) < TOL


@pytest.mark.parametrize("name,sample", [("mfma_decode", None),
                                         ("dsv4_mxfp4_decode", [0, 5, 7])])
def test_decode_mfma_crowded_experts(ops, name, sample):
    """Matrix-core decode of 8 tokens whose experts are shared unevenly (units
    of 8, 5, 3 and 1 entries besides the shared expert's 8): the down row
    groups are split over the grid by cost, which these entry counts skew."""
    _say("decode crowded experts", name)
    L = GpuLayer(name, layer=2 if name == "dsv4_mxfp4_decode" else 0)
    T, E, k = 8, L.s["n_experts"], L.s["top_k"]
    x = L.tokens(T)
    hi = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        row = [0, 1, 2 if t < 5 else 3]              # 8, 8, 5 and 3 entries
        row += [4 + (t * (k - 3) + j) % (E - 4) for j in range(k - 3)]
        hi[t] = row[:k]
    assert all(len(set(r)) == k for r in hi.tolist())
    hw = np.random.default_rng(11).uniform(0.02, 0.3, size=(T, k)).astype(np.float32)
    ids = torch.from_numpy(hi).cuda()
    w = torch.from_numpy(hw).cuda()
    y = _run_decode(ops, L, x, ids, w)
    assert np.all(np.isfinite(y))
    ref = _oracle_out(L, x, hi, hw.astype(np.float64), tokens=sample)
    got = y if sample is None else y[sample]
    assert olayer.row_rel_error(got, ref) < TOL


def _route_decode(ops, L, x, slot_of=None, ws=None):
    T, k, H = x.shape[0], L.s["top_k"], L.s["hidden"]
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = ops.workspace(L.desc, T, 1)
    ops.route_decode(L.desc, x, L.w_router, ids, w, L.pool, y, ws, slot_of=slot_of,
                     shared=L.shared)
    torch.cuda.synchronize()
    assert ops.decode_status(ws) == 0, "a wait inside the decode kernel expired"
    return ids, w, y, ws


def _launches(L, T):
    """Kernel launches of one decode call: T split evenly into launches of at
    most moe_decode_launch_tokens tokens (its values are pinned on the host
    in test_abi_host)."""
    from sparse_expert_execution_amd import ops as _ops
    per = _ops.decode_launch_tokens(L.desc)
    return (T + per - 1) // per


def _counters_clear(ws, launches):
    """Decode header after `launches` launches on a fresh workspace: every
    count back at zero (exit groups at word 96, the gate/up and exit lines
    from word 128), the launch generation (word 0) advanced once per launch."""
    hdr = ws[:8192].view(torch.int32)
    return torch.count_nonzero(hdr[96:1152]).item() == 0 and hdr[0].item() == launches


def _check_ids(L, x, gi, gw, renorm=False):
    r = olayer.route(bf16_to_f64(x), oracle_router(L.name, L.layer), L.s["top_k"],
                     renorm=renorm)
    _check_topk(r, gi, gw, L.s["top_k"], renorm)


@pytest.mark.parametrize("name,T,wtype", [("tiny", 1, "bf16"), ("tiny", 4, "mxfp4"),
                                          ("qwen_bf16_decode", 1, None),
                                          ("qwen_bf16_decode", 4, None),
                                          ("qwen_bf16_decode", 16, None),
                                          ("ragged_decode", 3, None),
                                          ("ragged_decode", 9, None),
                                          ("glm_cache_decode", 1, None),
                                          ("tiny", 4, "nvfp4"),
                                          ("ragged_decode", 9, "nvfp4"),
                                          ("qwen_bf16_decode", 4, "nvfp4"),
                                          ("many_experts", 1, None),
                                          ("many_experts", 5, None),
                                          ("many_experts", 16, None),
                                          ("mfma_decode", 1, None),
                                          ("mfma_decode", 3, None),
                                          ("mfma_decode", 8, None),
                                          ("mfma_decode", 11, None)])
def test_route_decode(ops, name, T, wtype):
    """Router + experts + combine in one call (one persistent kernel per
    launch of up to moe_decode_launch_tokens tokens)."""
    _say("route_decode", name, T, wtype)
    L = GpuLayer(name, wtype=wtype)
    x = L.tokens(T)
    ids, w, y, ws = _route_decode(ops, L, x)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    _check_ids(L, x, gi, gw)
    ref = _oracle_out(L, x, gi, gw)
    assert olayer.row_rel_error(y.cpu().numpy(), ref) < TOL
    # the counts are re-armed
    assert _counters_clear(ws, _launches(L, T))
    # a second call on the same workspace: same routing, same output up to
    # the order of the fp32 atomic adds
    ids2, w2, y2, _ = _route_decode(ops, L, x, ws=ws)
    assert torch.equal(ids, ids2)
    assert olayer.row_rel_error(y2.cpu().numpy(), y.cpu().numpy().astype(np.float64)) < 1e-5
    # then fewer tokens on that workspace: the logits left by the earlier
    # launches (other rows, older generation) must not be taken
    if T > 1:
        xs = x[1:].contiguous()
        ids3, w3, y3, _ = _route_decode(ops, L, xs, ws=ws)
        assert torch.equal(ids3, ids[1:])
        assert olayer.row_rel_error(y3.cpu().numpy(), ref[1:]) < TOL
        assert _counters_clear(ws, 2 * _launches(L, T) + _launches(L, T - 1))


@pytest.mark.parametrize("name,T,wtype", [("tiny", 4, "bf16"), ("qwen_bf16_decode", 1, None),
                                          ("qwen_bf16_decode", 16, None),
                                          ("ragged_decode", 9, None),
                                          ("mfma_decode", 5, None)])
def test_route_decode_renorm(ops, name, T, wtype):
    """Renormalised top-k weights in the one-kernel path: the rank and the
    wave-arg-max top-k, the one-wave and the workgroup expert list."""
    _say("route_decode renorm", name, T)
    L = GpuLayer(name, wtype=wtype, renorm=True)
    x = L.tokens(T)
    ids, w, y, _ = _route_decode(ops, L, x)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    _check_ids(L, x, gi, gw, renorm=True)
    assert np.allclose(gw.sum(axis=1), 1.0, atol=1e-6)
    ref = _oracle_out(L, x, gi, gw)
    assert olayer.row_rel_error(y.cpu().numpy(), ref) < TOL


@pytest.mark.parametrize("T,sample", [(1, [0]), (4, [0, 1, 2, 3]), (16, [1, 4, 6, 9, 10, 12, 14, 15])])
def test_route_decode_dsv4_full_sampled(ops, T, sample):
    _say("route_decode dsv4", T)
    L = GpuLayer("dsv4_mxfp4_decode", layer=11)
    x = L.tokens(T)
    ids, w, y, ws = _route_decode(ops, L, x)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    _check_ids(L, x, gi, gw)
    ref = _oracle_out(L, x, gi, gw, tokens=sample)
    assert olayer.row_rel_error(y.cpu().numpy()[sample], ref) < TOL
    assert _counters_clear(ws, _launches(L, T))


@pytest.mark.parametrize("T,sample", [(2, [0, 1]), (5, [0, 4])])
def test_route_decode_glm_matrix_core_sampled(ops, T, sample):
    """GLM-shaped layer (H 6144: two 16-byte scale loads per row in the
    matrix-core gate/up) on the matrix-core decode, sampled tokens."""
    _say("route_decode glm matrix core", T)
    L = GpuLayer("glm_cache_decode", layer=0)
    x = L.tokens(T)
    ids, w, y, ws = _route_decode(ops, L, x)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    _check_ids(L, x, gi, gw)
    ref = _oracle_out(L, x, gi, gw, tokens=sample)
    # repeated calls: the down phase runs two batches per pass here, whose
    # table hand-over between batches once let y results land on wrong rows
    # in about one call in sixty
    for rep in range(20):
        if rep:
            ids, w, y, ws = _route_decode(ops, L, x)
            assert np.array_equal(ids.cpu().numpy(), gi)
        got = y.cpu().numpy()[sample]
        err = olayer.row_rel_error(got, ref)
        if err >= TOL:
            bad = np.argwhere(np.abs(got - ref) > TOL * np.abs(ref).max(axis=1, keepdims=True))
            _say("glm mismatch: call", rep, "bad (token, column) count", len(bad),
                 "first", bad[:24].tolist())
        assert err < TOL
        assert _counters_clear(ws, _launches(L, T))


def test_route_decode_dsv4_nvfp4_sampled(ops):
    """DeepSeek-shaped layer with NVFP4 experts (and the shared expert), one
    token: router + experts + combine against the oracle."""
    _say("route_decode dsv4 nvfp4")
    L = GpuLayer("dsv4_mxfp4_decode", layer=3, wtype="nvfp4")
    x = L.tokens(1)
    ids, w, y, ws = _route_decode(ops, L, x)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    _check_ids(L, x, gi, gw)
    ref = _oracle_out(L, x, gi, gw)
    assert olayer.row_rel_error(y.cpu().numpy(), ref) < TOL


@pytest.mark.parametrize("name,T,partial", [("tiny", 4, False), ("ragged_prefill", 1, False),
                                            ("ragged_prefill", 77, False),
                                            ("ragged_prefill", 700, True),
                                            ("mixed_prefill", 400, False)])
def test_prefill_nvfp4(ops, name, T, partial):
    """Prefill with NVFP4 experts (BF16 matrix cores, x as given, h rounded to
    BF16): ragged shapes, multi-tile experts and partial residency against
    the oracle's BF16-h contract."""
    _say("prefill nvfp4", name, T, partial)
    L = GpuLayer(name, wtype="nvfp4")
    E = L.s["n_experts"]
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    slot_of, resident = None, np.ones(E, dtype=bool)
    if partial:
        resident = np.arange(E) % 4 != 2
        slot_of = torch.from_numpy(np.where(resident, np.arange(E), -1).astype(np.int32)).cuda()
    y = _run_decode(ops, L, x, ids, w, slot_of=slot_of, fn="prefill")
    hi, hw = ids.cpu().numpy(), w.cpu().numpy()
    ref = _oracle_out(L, x, hi, hw, include=resident[hi] if partial else None, prefill="bf16")
    assert olayer.row_rel_error(y, ref) < TOL


def test_prefill_nvfp4_dsv4_sampled(ops):
    """DeepSeek-shaped layer with NVFP4 experts at T = 4096: tokens at the
    first and last rows of expert segments against the oracle."""
    _say("prefill nvfp4 dsv4 4096")
    L = GpuLayer("dsv4_mxfp4_prefill", wtype="nvfp4")
    T = 4096
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w, fn="prefill")
    assert np.all(np.isfinite(y))
    hi, hw = ids.cpu().numpy(), w.cpu().numpy()
    sample = _segment_sample(hi, L.s["n_experts"])
    ref = _oracle_out(L, x, hi, hw, tokens=sample, prefill="bf16")
    assert olayer.row_rel_error(y[sample], ref) < TOL


def test_route_decode_partial_subset(ops):
    _say("route_decode partial")
    L = GpuLayer("ragged_decode")
    T, E = 4, L.s["n_experts"]
    x = L.tokens(T, stream=3)
    resident = np.arange(E) % 4 != 1
    slot_of = torch.from_numpy(np.where(resident, np.arange(E), -1).astype(np.int32)).cuda()
    ids, w, y, _ = _route_decode(ops, L, x, slot_of=slot_of)
    gi, gw = ids.cpu().numpy(), w.cpu().numpy()
    ref = _oracle_out(L, x, gi, gw, include=resident[gi])
    assert olayer.row_rel_error(y.cpu().numpy(), ref) < TOL


# ---------------------------------------------------------------- prefill
@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 300), ("ragged_prefill", 1),
                                    ("ragged_prefill", 77), ("ragged_prefill", 700),
                                    ("mixed_prefill", 150), ("mixed_prefill", 400),
                                    ("deep_prefill", 1), ("deep_prefill", 50),
                                    ("deep_prefill", 300)])
def test_prefill_small(ops, name, T):
    _say("prefill", name, T)
    L = GpuLayer(name, wtype="mxfp4")
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w, fn="prefill")
    ref = _oracle_out(L, x, ids.cpu().numpy(), w.cpu().numpy(), prefill=True)
    assert olayer.row_rel_error(y, ref) < TOL


@pytest.mark.parametrize("name,T,partial", [("tiny", 300, False), ("ragged_prefill", 700, True),
                                            ("ragged_prefill", 1, False),
                                            ("dsv4_mxfp4_prefill", 4096, False)])
def test_prefill_sort_integers(ops, name, T, partial):
    """The prefill expert sort, bit for bit against a host stable sort: the
    segment starts, the 128-row tile list and the sorted pair ids (resident
    routed pairs by expert, then the shared expert's), non-resident pairs
    left out."""
    _say("prefill sort", name, T, partial)
    L = GpuLayer(name, wtype="mxfp4")
    s = L.s
    E, k = s["n_experts"], s["top_k"]
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    resident = np.arange(E) % 3 != 0 if partial else np.ones(E, dtype=bool)
    slot_of = None
    if partial:
        slot_of = torch.from_numpy(np.where(resident, np.arange(E), -1).astype(np.int32)).cuda()
    y = torch.empty((T, s["hidden"]), dtype=torch.float32, device="cuda")
    ws = ops.workspace(L.desc, T, 2)
    ops.prefill(L.desc, x, ids, w, L.pool, y, ws, slot_of=slot_of, shared=L.shared)
    torch.cuda.synchronize()
    seg, tiles, pairs = (v.cpu().numpy() for v in ops.prefill_sort_view(L.desc, T, ws))
    hi = ids.cpu().numpy().reshape(-1)
    bins = np.where(resident[hi], hi, -1)
    if s["shared"]:
        bins = np.concatenate([bins, np.full(T, E)])
    order = np.argsort(np.where(bins < 0, E + 1, bins), kind="stable")
    kept = order[bins[order] >= 0]
    counts = np.bincount(bins[bins >= 0], minlength=E + 1)
    starts = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(seg[:E + 2], starts)
    assert np.array_equal(pairs[:kept.size], kept)
    ref_tiles = [(b, starts[b] + r) for b in range(E + 1) for r in range(0, counts[b], 128)]
    assert tiles[0] == len(ref_tiles)
    assert np.array_equal(tiles[1:1 + 2 * len(ref_tiles)].reshape(-1, 2),
                          np.array(ref_tiles, dtype=np.int64).reshape(-1, 2))


def test_prefill_partial_subset(ops):
    _say("prefill partial")
    L = GpuLayer("ragged_prefill")
    T, E = 200, L.s["n_experts"]
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    resident = np.arange(E) % 3 != 0
    slot_of = torch.from_numpy(np.where(resident, np.arange(E), -1).astype(np.int32)).cuda()
    y = _run_decode(ops, L, x, ids, w, slot_of=slot_of, fn="prefill")
    hi, hw = ids.cpu().numpy(), w.cpu().numpy()
    ref = _oracle_out(L, x, hi, hw, include=resident[hi], prefill=True)
    assert olayer.row_rel_error(y, ref) < TOL


@pytest.mark.parametrize("buffers", [1, 2])
def test_prefill_layer_stream(ops, buffers):
    """Full-layer streaming from a pinned pool (one or two device buffers):
    every layer's prefill through the streamed buffer equals the prefill over
    its resident pool bit for bit, and the oracle."""
    _say("prefill layer stream", buffers)
    name = "ragged_prefill"
    s = synth.SHAPES[name]
    n_layers, T, E, H = 4, 48, s["n_experts"], s["hidden"]
    Ls = [GpuLayer(name, layer=l) for l in range(n_layers)]
    eb = Ls[0].expert_bytes
    lb = (E + (1 if s["shared"] else 0)) * eb
    host = torch.empty(n_layers * lb, dtype=torch.uint8).pin_memory()
    for l, L in enumerate(Ls):
        host[l * lb:l * lb + E * eb].copy_(L.pool.cpu())
        if s["shared"]:
            host[l * lb + E * eb:(l + 1) * lb].copy_(L.shared.cpu())
    bufs = [torch.empty(lb, dtype=torch.uint8, device="cuda") for _ in range(buffers)]
    ls = ops.LayerStream(host, n_layers, lb, bufs)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    outs = []
    for l, L in enumerate(Ls):
        x = L.tokens(T)
        ids, w = _route_gpu(ops, L, x)
        buf = ls.acquire(l, copy, comp)
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        ops.prefill(L.desc, x, ids, w, buf[:E * eb], y, ops.workspace(L.desc, T, 2),
                    shared=buf[E * eb:] if s["shared"] else None)
        ls.release(l, comp)
        outs.append((x, ids, w, y))
    torch.cuda.synchronize()
    for l, (x, ids, w, y) in enumerate(outs):
        L = Ls[l]
        got = y.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, _run_decode(ops, L, x, ids, w, fn="prefill")), l
        ref = _oracle_out(L, x, ids.cpu().numpy(), w.cpu().numpy(), prefill=True)
        assert olayer.row_rel_error(got, ref) < TOL, l
    # a buffer whose layer has not been released cannot take another layer
    ls.acquire(0, copy, comp)
    with pytest.raises(ops._lib.MoeError):
        ls.acquire(buffers, copy, comp)
    ls.release(0, comp)
    torch.cuda.synchronize()


def _segment_sample(ids, E, n_experts=4):
    """Tokens at the first and last rows of expert segments of the prefill
    sort: token 0 and T-1 (the shared expert's segment, and the rows of the
    first and last tiles), and the first and last token routed to the lowest
    routed expert, the highest one, the one with the most tokens and the one
    with the fewest."""
    T = ids.shape[0]
    counts = np.bincount(ids.ravel(), minlength=E)
    hit = np.nonzero(counts)[0]
    fewest = int(hit[np.argmin(counts[hit])])
    picks = [int(hit[0]), int(hit[-1]), int(np.argmax(counts)), fewest][:n_experts]
    toks = {0, T - 1}
    for e in picks:
        rows = np.nonzero((ids == e).any(axis=1))[0]
        toks.update((int(rows[0]), int(rows[-1])))
    return sorted(toks)


@pytest.mark.parametrize("T", [4096, 8192, 16384])
def test_prefill_dsv4_full_layer_sampled(ops, T):
    """DeepSeek-shaped layer at the pages' prefill sizes (every expert hit):
    tokens at the first and last rows of several expert segments against the
    oracle's prefill contract."""
    _say("prefill dsv4", T)
    L = GpuLayer("dsv4_mxfp4_prefill")
    x = L.tokens(T)
    ids, w = _route_gpu(ops, L, x)
    y = _run_decode(ops, L, x, ids, w, fn="prefill")
    assert np.all(np.isfinite(y))
    hi, hw = ids.cpu().numpy(), w.cpu().numpy()
    sample = _segment_sample(hi, L.s["n_experts"])
    assert len(sample) >= 8
    _say("prefill dsv4", T, "oracle on tokens", sample)
    ref = _oracle_out(L, x, hi, hw, tokens=sample, prefill=True)
    assert olayer.row_rel_error(y[sample], ref) < TOL


# ------------------------------------------------------------ expert cache
def test_cache_trace_fills_tables_and_merge(ops):
    """Zipf trace through the GPU cache: slot tables equal the oracle LRU step
    by step, and GPU partial (resident + filled) + host partial (oracle) merge
    to the full layer output."""
    _say("cache trace")
    name = "small_cache"
    s = synth.SHAPES[name]
    E, k, slots, steps = s["n_experts"], s["top_k"], s["slots"], 40
    layers = s["layers"]
    Ls = [GpuLayer(name, layer=l) for l in range(layers)]
    eb = Ls[0].expert_bytes
    host_pool = torch.empty(layers * E * eb, dtype=torch.uint8).pin_memory()
    for l in range(layers):
        host_pool[l * E * eb:(l + 1) * E * eb].copy_(Ls[l].pool.cpu())
    dev_pool = torch.zeros(slots * eb, dtype=torch.uint8, device="cuda")
    table = torch.zeros((layers, E), dtype=torch.int32, device="cuda")
    cache = ops.ExpertCache(host_pool, layers, E, eb, dev_pool, slots, table)
    side = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ids_tr, w_tr = synth.zipf_trace(E, k, steps, s["zipf"], s["drift"])
    oc = ocache.LRUCache(slots)
    rng = np.random.default_rng(6)
    for st in range(steps):
        layer = int(rng.integers(0, layers))
        q = int(rng.integers(0, k + 1))
        ids_np, w_np = ids_tr[st:st + 1], w_tr[st:st + 1]
        plan = cache.plan(layer, ids_np, w_np, q)
        ref_plan = oc.step(layer, ids_np, w_np, q)
        pd = ops.plan_dict(plan)
        assert pd["fills"] == ref_plan["fills"] and pd["hits"] == ref_plan["hits"], st
        cache.fill(plan, side, comp)
        L = Ls[layer]
        x = L.tokens(1, stream=st)
        ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
        w = torch.from_numpy(w_np.astype(np.float32)).cuda()
        y = torch.empty((1, s["hidden"]), dtype=torch.float32, device="cuda")
        ws = ops.workspace(L.desc, 1, 1)
        ops.decode(L.desc, x, ids, w, dev_pool, y, ws, slot_of=table[layer])
        cache.release(plan, comp)
        resident_after = oc.slot_of_expert(layer, E) >= 0
        inc = resident_after[ids_np]
        y_host = _oracle_out(L, x, ids_np, w_np, include=~inc)
        yh = torch.from_numpy(y_host.astype(np.float32)).cuda()
        ops.merge_partials(y, yh, y)
        torch.cuda.synchronize()
        got_table = table.cpu().numpy()
        for l in range(layers):
            assert np.array_equal(got_table[l], oc.slot_of_expert(l, E)), (st, l)
        full = _oracle_out(L, x, ids_np, w_np)
        assert olayer.row_rel_error(y.cpu().numpy(), full) < TOL, st


def test_cache_elastic_rebuild_keeps_outputs(ops):
    """Elastic budget mid-trace: shrink in place to half the slots, then grow
    into a new, larger pool.  After every step the device slot table equals
    the oracle LRU (with the same rebuilds) and GPU partial + host partial
    still merge to the full layer, so the moved experts arrived intact."""
    _say("cache elastic rebuild")
    name = "small_cache"
    s = synth.SHAPES[name]
    E, k, slots, steps = s["n_experts"], s["top_k"], s["slots"], 36
    layers = s["layers"]
    Ls = [GpuLayer(name, layer=l) for l in range(layers)]
    eb = Ls[0].expert_bytes
    host_pool = torch.empty(layers * E * eb, dtype=torch.uint8).pin_memory()
    for l in range(layers):
        host_pool[l * E * eb:(l + 1) * E * eb].copy_(Ls[l].pool.cpu())
    pools = [torch.zeros(slots * eb, dtype=torch.uint8, device="cuda")]
    table = torch.zeros((layers, E), dtype=torch.int32, device="cuda")
    cache = ops.ExpertCache(host_pool, layers, E, eb, pools[0], slots, table)
    side = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ids_tr, w_tr = synth.zipf_trace(E, k, steps, s["zipf"], s["drift"], seed=8)
    oc = ocache.LRUCache(slots)
    rebuild = {12: ("same", slots // 2), 24: ("new", 2 * slots)}
    rng = np.random.default_rng(9)
    for st in range(steps):
        if st in rebuild:
            kind, n = rebuild[st]
            if kind == "new":
                pools.append(torch.zeros(n * eb, dtype=torch.uint8, device="cuda"))
            cache.resize(pools[-1], n, comp)
            oc.resize(n)
        layer = int(rng.integers(0, layers))
        ids_np, w_np = ids_tr[st:st + 1], w_tr[st:st + 1]
        q = int(rng.integers(1, k + 1))
        plan = cache.plan(layer, ids_np, w_np, q)
        ref_plan = oc.step(layer, ids_np, w_np, q)
        pd = ops.plan_dict(plan)
        assert pd["fills"] == ref_plan["fills"] and pd["hits"] == ref_plan["hits"], st
        cache.fill(plan, side, comp)
        L = Ls[layer]
        x = L.tokens(1, stream=st)
        ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
        w = torch.from_numpy(w_np.astype(np.float32)).cuda()
        y = torch.empty((1, s["hidden"]), dtype=torch.float32, device="cuda")
        ws = ops.workspace(L.desc, 1, 1)
        ops.decode(L.desc, x, ids, w, pools[-1], y, ws, slot_of=table[layer])
        cache.release(plan, comp)
        inc = (oc.slot_of_expert(layer, E) >= 0)[ids_np]
        yh = torch.from_numpy(_oracle_out(L, x, ids_np, w_np, include=~inc)
                              .astype(np.float32)).cuda()
        ops.merge_partials(y, yh, y)
        torch.cuda.synchronize()
        got_table = table.cpu().numpy()
        for l in range(layers):
            assert np.array_equal(got_table[l], oc.slot_of_expert(l, E)), (st, l)
        full = _oracle_out(L, x, ids_np, w_np)
        assert olayer.row_rel_error(y.cpu().numpy(), full) < TOL, st


@pytest.mark.parametrize("wtype", ["mxfp4", "nvfp4"])
def test_cache_trace_with_host_experts_merges_to_full_layer(ops, wtype):
    """The whole split: GPU partial over resident + filled experts, host
    partial over the other misses from moe_host_experts reading the pinned
    pool, merged on the GPU, equals the full layer (oracle)."""
    _say("cache trace + host experts", wtype)
    name = "small_cache"
    s = synth.SHAPES[name]
    E, k, slots, steps = s["n_experts"], s["top_k"], s["slots"], 24
    L = GpuLayer(name, wtype=wtype)
    eb = L.expert_bytes
    host_pool = torch.empty(E * eb, dtype=torch.uint8).pin_memory()
    host_pool.copy_(L.pool.cpu())
    dev_pool = torch.zeros(slots * eb, dtype=torch.uint8, device="cuda")
    table = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    cache = ops.ExpertCache(host_pool, 1, E, eb, dev_pool, slots, table)
    side = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ids_tr, w_tr = synth.zipf_trace(E, k, steps, s["zipf"], s["drift"], seed=3)
    y_host = torch.empty((1, s["hidden"]), dtype=torch.float32).pin_memory()
    for st in range(steps):
        ids_np, w_np = ids_tr[st:st + 1], w_tr[st:st + 1]
        plan = cache.plan(0, ids_np, w_np, 2)
        cache.fill(plan, side, comp)
        x = L.tokens(1, stream=st)
        ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
        w = torch.from_numpy(w_np.astype(np.float32)).cuda()
        y = torch.empty((1, s["hidden"]), dtype=torch.float32, device="cuda")
        ws = ops.workspace(L.desc, 1, 1)
        ops.decode(L.desc, x, ids, w, dev_pool, y, ws, slot_of=table[0])
        cache.release(plan, comp)
        host = set(ops.plan_dict(plan)["host"])
        inc = np.array([[int(e) in host for e in ids_np[0]]], dtype=np.uint8)
        ops.host_experts(L.desc, x.cpu(), torch.from_numpy(ids_np.astype(np.int32)),
                         torch.from_numpy(w_np.astype(np.float32)), host_pool, y_host,
                         include=torch.from_numpy(inc))
        ops.merge_partials(y, y_host.cuda(non_blocking=True), y)
        torch.cuda.synchronize()
        full = _oracle_out(L, x, ids_np, w_np)
        assert olayer.row_rel_error(y.cpu().numpy(), full) < TOL, st


def test_cache_glm_scale_steps_against_oracle(ops):
    """GLM-scale expert cache (6144 x 2048 MXFP4 experts, 256 in a pinned
    host pool, 64 slots) over the first 36 steps of the drifting Zipf trace
    with q from the planner's q* rule: the device slot table equals the
    oracle LRU after every step, and at the first (cold) and last step the
    GPU partial (resident + filled experts) plus the host expert kernel's
    partial (the other misses) merged on the GPU equals the oracle's full
    layer."""
    _say("cache glm scale")
    name = "glm_cache_decode"
    s = synth.SHAPES[name]
    E, k, slots, H = s["n_experts"], s["top_k"], s["slots"], s["hidden"]
    steps = 36
    L = GpuLayer(name)
    eb = L.expert_bytes
    host_pool = torch.empty(E * eb, dtype=torch.uint8).pin_memory()
    host_pool.copy_(L.pool.cpu())
    dev_pool = torch.zeros(slots * eb, dtype=torch.uint8, device="cuda")
    del L.pool
    torch.cuda.empty_cache()
    table = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    cache = ops.ExpertCache(host_pool, 1, E, eb, dev_pool, slots, table)
    b_pcie, b_host = 50e9, 178e9                       # fixed rates: q* = 2 of 8 misses
    cache.set_bandwidths(b_pcie, b_host)
    side = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ids_tr, w_tr = synth.zipf_trace(E, k, steps, s["zipf"], s["drift"])
    oc = ocache.LRUCache(slots)
    xs = L.tokens(steps)
    y_host = torch.empty((1, H), dtype=torch.float32).pin_memory()
    ws = ops.workspace(L.desc, 1, 1)
    checked = 0
    for st in range(steps):
        ids_np, w_np = ids_tr[st:st + 1], w_tr[st:st + 1]
        plan = cache.plan(0, ids_np, w_np, -1)
        S, _ = ocache.selected_experts(ids_np, w_np)
        m = sum((0, int(e)) not in oc.where for e in S)
        ref_plan = oc.step(0, ids_np, w_np, ocache.qstar(m, b_pcie, b_host))
        pd = ops.plan_dict(plan)
        assert pd["fills"] == ref_plan["fills"] and pd["hits"] == ref_plan["hits"], st
        cache.fill(plan, side, comp)
        x = xs[st:st + 1]
        ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
        w = torch.from_numpy(w_np.astype(np.float32)).cuda()
        y = torch.empty((1, H), dtype=torch.float32, device="cuda")
        ops.decode(L.desc, x, ids, w, dev_pool, y, ws, slot_of=table[0])
        cache.release(plan, comp)
        host = set(pd["host"])
        inc = np.array([[int(e) in host for e in ids_np[0]]], dtype=np.uint8)
        ops.host_experts(L.desc, x.cpu(), torch.from_numpy(ids_np.astype(np.int32)),
                         torch.from_numpy(w_np.astype(np.float32)), host_pool, y_host,
                         include=torch.from_numpy(inc))
        ops.merge_partials(y, y_host.cuda(non_blocking=True), y)
        torch.cuda.synchronize()
        assert np.array_equal(table.cpu().numpy()[0], oc.slot_of_expert(0, E)), st
        if st in (0, steps - 1):
            _say("cache glm scale: oracle at step", st, "hits", pd["hits"], "q", plan.q)
            full = _oracle_out(L, x, ids_np, w_np)
            assert olayer.row_rel_error(y.cpu().numpy(), full) < TOL, st
            checked += 1
    assert ops.decode_status(ws) == 0
    assert checked == 2


def test_cache_victim_fill_waits_for_last_use(ops):
    """Stream order of a victim fill: a decode reads four slots behind a long
    matrix product on the compute stream; the next step evicts exactly those
    slots and fills them on the side stream.  The copies must wait for the
    decode (the slots' last-use events), so the decode still sees the
    experts it was planned with: its y equals the oracle's for them, and the
    later step's y equals the oracle's for the new experts."""
    _say("cache victim ordering")
    name = "small_cache"
    s = synth.SHAPES[name]
    E, k, H = s["n_experts"], s["top_k"], s["hidden"]
    L = GpuLayer(name)
    eb = L.expert_bytes
    host_pool = torch.empty(E * eb, dtype=torch.uint8).pin_memory()
    host_pool.copy_(L.pool.cpu())
    slots = k
    dev_pool = torch.zeros(slots * eb, dtype=torch.uint8, device="cuda")
    table = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    cache = ops.ExpertCache(host_pool, 1, E, eb, dev_pool, slots, table)
    side = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    a = torch.randn((4096, 4096), device="cuda")
    b = torch.randn((4096, 4096), device="cuda")
    x = L.tokens(2)
    steps = [(np.array([[0, 1, 2, 3]]), np.array([[0.4, 0.3, 0.2, 0.1]], np.float32)),
             (np.array([[4, 5, 6, 7]]), np.array([[0.35, 0.3, 0.2, 0.15]], np.float32))]
    ys = []
    ws = ops.workspace(L.desc, 1, 1)
    for i, (ids_np, w_np) in enumerate(steps):
        plan = cache.plan(0, ids_np, w_np, k)
        if i == 1:
            victims = sorted(v for v in ops.plan_dict(plan)["victims"])
            assert victims == [(0, 0), (0, 1), (0, 2), (0, 3)]
        cache.fill(plan, side, comp)
        if i == 0:
            c = a
            for _ in range(8):                  # tens of ms of work ahead of the decode
                c = torch.mm(c, b).div_(64.0)
        y = torch.empty((1, H), dtype=torch.float32, device="cuda")
        ops.decode(L.desc, x[i:i + 1], torch.from_numpy(ids_np.astype(np.int32)).cuda(),
                   torch.from_numpy(w_np).cuda(), dev_pool, y, ws, slot_of=table[0])
        cache.release(plan, comp)
        ys.append(y)
    torch.cuda.synchronize()
    assert ops.decode_status(ws) == 0
    for i, (ids_np, w_np) in enumerate(steps):
        ref = _oracle_out(L, x[i:i + 1], ids_np, w_np)
        assert olayer.row_rel_error(ys[i].cpu().numpy(), ref) < TOL, i


def test_cache_injected_fill_failure_rolls_back(ops):
    _say("cache injected failure")
    name = "small_cache"
    s = synth.SHAPES[name]
    E, slots = s["n_experts"], s["slots"]
    L = GpuLayer(name)
    eb = L.expert_bytes
    host_pool = torch.empty(E * eb, dtype=torch.uint8).pin_memory()
    host_pool.copy_(L.pool.cpu())
    dev_pool = torch.zeros(slots * eb, dtype=torch.uint8, device="cuda")
    table = torch.zeros((1, E), dtype=torch.int32, device="cuda")
    cache = ops.ExpertCache(host_pool, 1, E, eb, dev_pool, slots, table)
    side = torch.cuda.Stream()
    p = cache.plan(0, [1, 2, 3], [0.5, 0.3, 0.2], 3)
    cache.fill(p, side)
    cache.release(p)
    before = cache.slot_table(0).copy()
    cache.debug_fail_fills(1)
    p = cache.plan(0, [4, 5], [0.6, 0.4], 2)
    with pytest.raises(ops._lib.MoeError) as ei:
        cache.fill(p, side)
    assert ei.value.status == ops._lib.MOE_EHIP
    assert np.array_equal(cache.slot_table(0), before)
    torch.cuda.synchronize()
    assert np.array_equal(table.cpu().numpy()[0], before)
    # the cache keeps working after the failure
    p = cache.plan(0, [4, 5], [0.6, 0.4], 2)
    cache.fill(p, side)
    cache.release(p)
    torch.cuda.synchronize()
    assert np.array_equal(table.cpu().numpy()[0], cache.slot_table(0))


def test_bandwidth_probe_and_qstar(ops):
    _say("probe")
    host = torch.empty(64 << 20, dtype=torch.uint8).pin_memory()
    dev = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    bp, bh = ops.probe_bandwidths(host, dev, reps=2)
    _say(f"B_pcie={bp / 1e9:.1f} GB/s B_host={bh / 1e9:.1f} GB/s")
    assert 1e9 < bp < 1e12 and 1e9 < bh < 1e13
    q = ops.qstar(8, bp, bh)
    assert q == ocache.qstar(8, bp, bh)

"""Pins of the oracle's router, expert FFN, combine and merge (CPU only)."""

import itertools

import numpy as np
import pytest
import torch

import synth
from oracle import formats, layer


def _tiny(seed=0):
    name = "tiny"
    s = synth.SHAPES[name]
    x = synth.tokens(name, 0, 4, seed=seed).float().double().numpy()
    wr = synth.router_weights(name, 0, seed=seed).double().numpy()
    experts = [tuple(m.double().numpy() for m in synth.expert_weights(name, 0, e, seed=seed))
               for e in range(s["n_experts"])]
    return s, x, wr, experts


def _torch_ffn(x, wg, wu, wd):
    """Textbook SwiGLU with PyTorch-CPU fp64 ops (independent of the oracle)."""
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T) @ wd.T).numpy()


def test_softmax_matches_torch():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((16, 257)) * 5
    ref = torch.softmax(torch.from_numpy(z), dim=-1).numpy()
    assert np.allclose(layer.softmax(z), ref, rtol=1e-13, atol=0)


def test_route_is_stable_argsort_and_sums_to_one():
    s, x, wr, _ = _tiny()
    r = layer.route(x, wr, s["top_k"])
    assert np.allclose(r["p"].sum(axis=1), 1.0, atol=1e-14)
    for t in range(x.shape[0]):
        order = np.argsort(-r["p"][t], kind="stable")
        assert list(r["ids"][t]) == list(order[: s["top_k"]])
        assert np.array_equal(r["w"][t], r["p"][t, r["ids"][t]])


def test_route_brute_force_best_subset():
    s, x, wr, _ = _tiny()
    k, E = s["top_k"], s["n_experts"]
    r = layer.route(x, wr, k)
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(E), k),
                   key=lambda c: sum(r["p"][t, list(c)]))
        assert set(best) == set(r["ids"][t].tolist())
        assert r["gap"][t] > 0


def test_route_ties_lower_id_and_descending():
    # experts 1 and 3 get identical logits, larger than the rest
    H, E = 4, 6
    wr = np.zeros((E, H))
    wr[1, 0] = wr[3, 0] = 2.0
    wr[5, 0] = 1.0
    x = np.array([[1.0, 0, 0, 0]])
    r = layer.route(x, wr, 3)
    assert r["ids"][0].tolist() == [1, 3, 5]
    assert r["gap"][0] > 0
    r2 = layer.route(x, wr, 1)
    assert r2["ids"][0].tolist() == [1] and r2["gap"][0] == 0.0


def test_route_renorm():
    s, x, wr, _ = _tiny()
    r = layer.route(x, wr, 3, renorm=True)
    assert np.allclose(r["w"].sum(axis=1), 1.0, atol=1e-14)


def test_sparse_gather_equals_dense_masked_mixture():
    s, x, wr, experts = _tiny()
    y, r = layer.moe_layer(x, wr, experts, s["top_k"])
    T, E = x.shape[0], s["n_experts"]
    gate = np.zeros((T, E))
    for t in range(T):
        gate[t, r["ids"][t]] = r["w"][t]
    dense = sum(gate[:, e:e + 1] * _torch_ffn(x, *experts[e]) for e in range(E))
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-15)


def test_k1_renorm_is_single_textbook_swiglu():
    s, x, wr, experts = _tiny()
    y, r = layer.moe_layer(x, wr, experts, 1, renorm=True)
    for t in range(x.shape[0]):
        e = int(r["ids"][t, 0])
        ref = _torch_ffn(x[t:t + 1], *experts[e])[0]
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-15)


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    got = layer.silu(z)
    assert got[0] == 0.0
    assert abs(got[1] - 0.7310585786300049) < 1e-15
    assert abs(got[2] + 0.2689414213699951) < 1e-15
    assert abs(got[3] - 40.0) < 1e-12 and abs(got[4]) < 1e-15


def test_zero_input_gives_zero_output():
    s, x, wr, experts = _tiny()
    y, _ = layer.moe_layer(np.zeros_like(x), wr, experts, s["top_k"],
                           shared=experts[0])
    assert np.all(y == 0)


def test_shared_expert_adds_weight_one():
    s, x, wr, experts = _tiny()
    y0, r = layer.moe_layer(x, wr, experts, s["top_k"])
    y1, _ = layer.moe_layer(x, wr, experts, s["top_k"], shared=experts[5])
    assert np.allclose(y1 - y0, _torch_ffn(x, *experts[5]), rtol=1e-11, atol=1e-15)


def test_every_partition_merges_exactly():
    s, x, wr, experts = _tiny()
    T, k = x.shape[0], s["top_k"]
    r = layer.route(x, wr, k)
    full = layer.combine(x, r["ids"], r["w"], experts, shared=experts[1])
    n = T * k
    for bits in range(2 ** n):
        mask = np.array([(bits >> i) & 1 for i in range(n)], dtype=bool).reshape(T, k)
        a = layer.combine(x, r["ids"], r["w"], experts, shared=experts[1], include=mask)
        b = layer.combine(x, r["ids"], r["w"], experts, shared=None, include=~mask)
        y = layer.merge(a, b)
        assert layer.row_rel_error(y, full) < 1e-12


def test_prefill_quantises_x_along_hidden_blocks():
    # x already on the MXFP4 grid (every block's max is 4 * 2^X): prefill x
    # quantisation is the identity, so the gate/up inputs equal decode's.
    s, _, _, experts = _tiny()
    rng = np.random.default_rng(5)
    H = s["hidden"]
    codes = rng.integers(0, 16, size=(3, H), dtype=np.uint8)
    codes[:, ::32] = 6
    scales = rng.integers(110, 130, size=(3, H // 32), dtype=np.uint8)
    x = formats.mxfp4_decode(formats.pack_nibbles(codes), scales)
    assert np.array_equal(layer.mx_roundtrip(x), x)
    # one huge element zeroes its own block only
    x2 = x.copy()
    x2[0, 40] = 1e6
    q = layer.mx_roundtrip(x2)
    assert np.array_equal(q[0, :32], x[0, :32])
    assert np.all(q[0, 32:64][np.arange(32) != 8] == 0)
    assert np.array_equal(q[0, 64:], x[0, 64:])


def test_prefill_contract_close_to_decode():
    s, x, wr, experts = _tiny()
    y_dec, r = layer.moe_layer(x, wr, experts, s["top_k"])
    y_pre = layer.combine(x, r["ids"], r["w"], experts, prefill=True)
    # MXFP4 x and h: a few-percent perturbation, not a different function
    rel = layer.row_rel_error(y_pre, y_dec)
    assert 1e-4 < rel < 0.5


def test_row_rel_error_definition():
    ref = np.array([[1.0, -4.0], [0.0, 0.0]])
    got = np.array([[1.5, -4.0], [0.0, 0.1]])
    assert layer.row_rel_error(got, ref) == pytest.approx(0.125)

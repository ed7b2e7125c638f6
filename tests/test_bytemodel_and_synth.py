"""Byte model against the pages' figures; generator determinism (CPU only)."""

import json
import os

import numpy as np
import torch

import synth
from conftest import GOLDEN
from sparse_expert_execution_amd import bytemodel as bm

with open(os.path.join(GOLDEN, "page_figures.json")) as f:
    PAGES = json.load(f)


def test_dsv4_expert_set_roughly_140GB():
    r = PAGES["dsv4_routing"]
    per_expert = bm.expert_bytes(4096, 2048, "mxfp4")
    assert per_expert == 13_369_344
    total = r["experts_per_layer"] * per_expert * r["layers"]
    assert abs(total / 1e9 - PAGES["dsv4_fp4_expert_set_GB_roughly"]["value"]) / 140 < 0.06
    # routed active parameters stay below the ~13B active the pages give
    active = r["active_per_token"] * 3 * 4096 * 2048 * r["layers"]
    assert 6e9 < active < r["active_params_B"] * 1e9


def test_glm_checkpoint_size():
    g = PAGES["glm_checkpoint"]
    # NVFP4: 4-bit code + one 8-bit scale per 16 elements = 4.5 bits/param
    gb = g["total_params_B"] * 1e9 * 4.5 / 8 / 1e9
    assert abs(gb - g["nvfp4_checkpoint_GB"]) / g["nvfp4_checkpoint_GB"] < 0.03


def test_prefill_chunk_is_link_bound():
    p = PAGES["prefill_chunk"]
    t = p["expert_pool_GB"] / p["link_GB_per_s"]
    assert p["seconds_low"] <= t <= p["seconds_high"] + 0.005


def test_expert_bytes_all_formats():
    assert bm.expert_bytes(2048, 768, "bf16") == 9_437_184
    assert bm.expert_bytes(6144, 2048, "mxfp4") == 20_054_016
    assert bm.expert_bytes(256, 128, "f32") == 393_216
    assert bm.expert_bytes(256, 128, "mxfp4") == 52_224


def test_decode_bytes_qwen_t1():
    b = bm.decode_call_bytes(2048, 768, 128, "bf16", 1, 8)
    assert b == 8 * 9_437_184 + 128 * 2048 * 2 + 2048 * 6


def test_expected_distinct():
    assert abs(bm.expected_distinct(128, 8, 8) - 51.62) < 0.01
    assert abs(bm.expected_distinct(256, 6, 16) - 80.84) < 0.01


def test_prefill_flops_per_token():
    assert bm.expert_flops(4096, 2048, 7) == 352_321_536


def test_synth_is_deterministic_and_keyed():
    a = synth.expert_weights("tiny", 0, 3)
    b = synth.expert_weights("tiny", 0, 3)
    c = synth.expert_weights("tiny", 0, 4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    x = synth.tokens("tiny", 0, 4)
    assert x.dtype == torch.bfloat16 and x.shape == (4, 256)
    assert torch.equal(x, synth.tokens("tiny", 0, 4))
    wq = synth.expert_weights("qwen_bf16_decode", 0, 0)
    assert wq[0].dtype == torch.bfloat16 and wq[2].shape == (2048, 768)


def test_synth_distribution():
    g, u, d = synth.expert_weights("dsv4_mxfp4_decode", 0, 0)
    assert abs(g.std().item() - 0.02) < 2e-4 and abs(g.mean().item()) < 2e-4


def test_zipf_trace_shape_and_drift():
    ids, w = synth.zipf_trace(256, 8, 512, 1.1, 32)
    assert ids.shape == (512, 8) and w.shape == (512, 8)
    for s in range(512):
        assert len(set(ids[s].tolist())) == 8
        assert np.all(np.diff(w[s]) <= 0)
    ids2, _ = synth.zipf_trace(256, 8, 512, 1.1, 32)
    assert np.array_equal(ids, ids2)
    # popularity is skewed: the 64 most frequent experts carry most picks
    counts = np.bincount(ids[:32].ravel(), minlength=256)
    assert np.sort(counts)[::-1][:64].sum() > 0.6 * counts.sum()

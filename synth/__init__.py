"""Seeded synthetic inputs for the routed MoE layer.

This module is shared by the oracle side (tests) and the GPU side (tests,
benchmark).  It holds NO arithmetic of the method: no routing, no softmax,
no quantisation, no FFN.  It only draws random numbers of the right shapes
and distributions, deterministically from a seed, with PyTorch's generators
(CPU or GPU), and names the workload shapes.

Distributions (the workload recipe): weights and router ~ N(0, 0.02),
tokens x ~ N(0, 1) cast to BF16 (PyTorch's cast, round to nearest even);
BF16-weight layers cast N(0, 0.02) fp32 draws to BF16 the same way.
Expert-cache traces draw expert ids from a Zipf(alpha) popularity over a
rank -> expert permutation that is redrawn every ``drift`` steps, k distinct
experts per step (sampling without replacement), and gate weights
U(0.02, 0.2) sorted descending.

Every tensor is drawn from its own generator seeded by a 63-bit value derived
from (workload, layer, expert, matrix, ...) with numpy's SeedSequence, so
one expert can be regenerated on its own, on the device it was first drawn
on, with identical values.  A CPU draw and a GPU draw of the same keys are
NOT equal (different generators); tests compare sides on one draw.
"""

import numpy as np
import torch

# Workload shapes.  wtype: 'f32' (tiny layer), 'bf16' or 'mxfp4'.
SHAPES = {
    "tiny": dict(hidden=256, inter=128, n_experts=8, top_k=2, shared=False,
                 wtype="f32", tokens=(4,), layers=1),
    "qwen_bf16_decode": dict(hidden=2048, inter=768, n_experts=128, top_k=8,
                             shared=False, wtype="bf16", tokens=(1, 8),
                             layers=48),
    "dsv4_mxfp4_decode": dict(hidden=4096, inter=2048, n_experts=256, top_k=6,
                              shared=True, wtype="mxfp4", tokens=(1, 4, 16),
                              layers=43),
    "dsv4_mxfp4_prefill": dict(hidden=4096, inter=2048, n_experts=256, top_k=6,
                               shared=True, wtype="mxfp4",
                               tokens=(4096, 8192, 16384), layers=1),
    # small shapes with ragged tails (fewer than 64 vectors per row, partial
    # tiles, odd expert counts) used by the parity tests
    "ragged_decode": dict(hidden=800, inter=96, n_experts=20, top_k=3, shared=True,
                          wtype="mxfp4", tokens=(1, 5, 33, 64), layers=1),
    "ragged_prefill": dict(hidden=512, inter=256, n_experts=13, top_k=4,
                           shared=True, wtype="mxfp4", tokens=(1, 77, 700),
                           layers=1),
    # the largest expert count one decode launch takes (1024: 16 logits per
    # lane in the wave top-k); H = 4096 so that the router's logits spread
    # enough for most tokens' k-th and (k+1)-th probabilities to be apart
    "many_experts": dict(hidden=4096, inter=128, n_experts=1024, top_k=8, shared=False,
                         wtype="mxfp4", tokens=(1, 5, 16), layers=1),
    # prefill with K = H not a multiple of 512 (the narrow GEMM scheme) and
    # K = I one (the wide scheme)
    "mixed_prefill": dict(hidden=640, inter=1024, n_experts=9, top_k=3, shared=True,
                          wtype="mxfp4", tokens=(150, 400), layers=1),
    # prefill with both K (H = 2048, I = 1024) on the wide GEMM scheme and a
    # shared expert spanning three 128-row tiles at T = 300
    "deep_prefill": dict(hidden=2048, inter=1024, n_experts=10, top_k=3, shared=True,
                         wtype="mxfp4", tokens=(50, 300), layers=1),
    # decode on the matrix-core MXFP4 path (H, I multiples of 256) at sizes
    # the oracle takes whole: 8 tokens per launch, 11 split into two
    "mfma_decode": dict(hidden=512, inter=256, n_experts=12, top_k=3, shared=True,
                        wtype="mxfp4", tokens=(1, 3, 8, 11), layers=1),
    "small_cache": dict(hidden=256, inter=128, n_experts=32, top_k=4,
                        shared=False, wtype="mxfp4", tokens=(1,), layers=2,
                        slots=8, steps=64, zipf=1.1, drift=16),
    "glm_cache_decode": dict(hidden=6144, inter=2048, n_experts=256, top_k=8,
                             shared=False, wtype="mxfp4", tokens=(1,), layers=1,
                             slots=64, steps=512, zipf=1.1, drift=32),
}

WEIGHT_STD = 0.02

_MATRIX = {"router": 0, "gate": 1, "up": 2, "down": 3, "x": 4, "trace": 5}


def seed_of(*keys):
    """63-bit seed from a tuple of ints / strings (stable across runs)."""
    ints = []
    for k in keys:
        if isinstance(k, str):
            ints.extend(int(b) for b in k.encode())
            ints.append(0xFFFF)
        else:
            ints.append(int(k) & 0xFFFFFFFF)
    ss = np.random.SeedSequence(ints)
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std, seed, device="cpu"):
    """fp32 N(0, std^2) tensor of the given shape from one seeded draw."""
    g = _gen(device, seed)
    out = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        out.mul_(std)
    return out


def router_weights(name, layer, device="cpu", seed=0, as_dtype=None):
    """W_r [E, H]: fp32 for the tiny layer, else BF16 (or ``as_dtype``)."""
    s = SHAPES[name]
    w = normal((s["n_experts"], s["hidden"]), WEIGHT_STD,
               seed_of(name, seed, layer, _MATRIX["router"]), device)
    dt = as_dtype or (torch.float32 if s["wtype"] == "f32" else torch.bfloat16)
    return w.to(dt)


def expert_weights(name, layer, expert, device="cpu", seed=0, as_dtype=None):
    """(gate [I, H], up [I, H], down [H, I]) of one expert.

    expert == n_experts names the shared expert.  Values are fp32 draws; for
    BF16-weight workloads they are cast to BF16 unless ``as_dtype`` says
    otherwise.  MXFP4 workloads return fp32 (each side quantises itself).
    """
    s = SHAPES[name]
    H, I = s["hidden"], s["inter"]
    out = []
    for mat, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = normal(shape, WEIGHT_STD,
                   seed_of(name, seed, layer, expert, _MATRIX[mat]), device)
        dt = as_dtype
        if dt is None:
            dt = torch.bfloat16 if s["wtype"] == "bf16" else torch.float32
        out.append(w.to(dt))
    return tuple(out)


def tokens(name, layer, T, device="cpu", seed=0, stream=0):
    """x [T, H] BF16 with x ~ N(0, 1)."""
    s = SHAPES[name]
    x = normal((T, s["hidden"]), 1.0,
               seed_of(name, seed, layer, _MATRIX["x"], T, stream), device)
    return x.to(torch.bfloat16)


def zipf_trace(n_experts, k, steps, alpha, drift, seed=0):
    """Expert-cache decode trace, one token per step.

    Returns ids [steps, k] int32 (ordered by descending gate weight) and
    w [steps, k] float32.
    """
    rng = np.random.Generator(np.random.PCG64(seed_of("trace", seed)))
    pop = np.arange(1, n_experts + 1, dtype=np.float64) ** (-alpha)
    pop /= pop.sum()
    ids = np.empty((steps, k), dtype=np.int32)
    w = np.empty((steps, k), dtype=np.float32)
    perm = None
    for s in range(steps):
        if s % drift == 0:
            perm = rng.permutation(n_experts)
        ranks = rng.choice(n_experts, size=k, replace=False, p=pop)
        ids[s] = perm[ranks]
        w[s] = np.sort(rng.uniform(0.02, 0.2, size=k))[::-1]
    return ids, w

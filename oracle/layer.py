"""Oracle: the routed MoE layer in fp64 (test infrastructure only).

What the pages fix: each token, in each MoE layer, is routed to a few of many
experts and only those experts run ("FreeToken 753b Model Explained", section
"FreeToken 753b Model Explained": six of 256 experts per layer for the
DeepSeek-V4-Flash shape); the layer output is a sum of per-expert partial
results, and the partial sums of two disjoint expert subsets (GPU-side and
CPU-side) recombine exactly, with no approximation and no change to the
router (explainx.ai guide, section "Decode: decide whether to move an expert
or compute where it lives"; futuresignalnews.com article, section
"1. Bandwidth-Adaptive Execution (The q* Policy)").

What the pages leave open, and the reading taken here:
  * gate: softmax over all E router logits, then the top k probabilities;
    ties go to the lower expert id; output order is descending probability;
    the k weights are the probabilities themselves, or divided by their sum
    when ``renorm`` is set;
  * expert: SwiGLU, o = W_d (silu(W_g x) * (W_u x)), silu(z) = z/(1+e^-z),
    no biases, no clamp;
  * shared expert (when present): always runs, weight 1, same shape;
  * prefill precision contract, MXFP4 experts: the gate/up product uses x
    quantised to MXFP4 along H and the down product uses h quantised to
    MXFP4 along I (the scaled FP4 matrix instructions take MXFP4 on both
    sides); NVFP4 experts: x as given (BF16) and h rounded to BF16 (nearest
    even) before the down product (the BF16 matrix instructions take e2m1
    times its E4M3 block scale exactly); decode uses x as given and h
    unrounded.

Pins (tests/test_oracle_layer.py): stable-argsort special case and
brute-force best k-subset on the tiny layer; probabilities sum to one; the
sparse gather equals the dense masked mixture evaluated over every expert;
k = 1 with renormalisation equals one textbook SwiGLU computed with
PyTorch-CPU's silu; x = 0 gives y = 0; every 2-way partition of the selected
(token, expert) pairs merges back to the full output.
"""

import numpy as np

from . import formats


def softmax(z):
    """Row-wise softmax over the last axis, max-subtracted, fp64."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def route(x, w_router, k, renorm=False):
    """Router: logits, softmax, top-k.

    x        [T, H] fp64 token activations
    w_router [E, H] fp64 router weights
    Returns dict with
      ids   [T, k] int32, descending probability, ties -> lower id
      w     [T, k] fp64 gate weights
      p     [T, E] fp64 probabilities
      z     [T, E] fp64 logits
      gap   [T] fp64  p_(k) - p_(k+1) (inf when k == E)
    """
    x = np.asarray(x, dtype=np.float64)
    w_router = np.asarray(w_router, dtype=np.float64)
    E = w_router.shape[0]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    z = x @ w_router.T
    p = softmax(z)
    T = x.shape[0]
    ids = np.empty((T, k), dtype=np.int32)
    gap = np.full(T, np.inf)
    expert = np.arange(E)
    for t in range(T):
        # sort by descending p, then ascending id
        order = np.lexsort((expert, -p[t]))
        ids[t] = order[:k]
        if k < E:
            gap[t] = p[t, order[k - 1]] - p[t, order[k]]
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        w = w / np.sum(w, axis=1, keepdims=True)
    return {"ids": ids, "w": w, "p": p, "z": z, "gap": gap}


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def mx_roundtrip(a):
    """Quantise fp64 rows to MXFP4 along the last axis and decode again."""
    codes, scales = formats.mxfp4_encode(a)
    return formats.mxfp4_decode(codes, scales)


def bf16_roundtrip(a):
    """Round fp64 values to BF16 (nearest even) through their fp32 value, and
    decode again."""
    return formats.bf16_decode(formats.bf16_round(np.asarray(a, dtype=np.float32)))


def expert_ffn(x, w_gate, w_up, w_down, prefill=False):
    """One SwiGLU expert on the rows of x.

    x [n, H]; w_gate, w_up [I, H]; w_down [H, I]; all fp64 values.
    prefill: False (decode contract), True or "mxfp4" (MXFP4 x and h), or
    "bf16" (x as given, h rounded to BF16).
    Returns o [n, H] fp64 (and h [n, I] for inspection).
    """
    if prefill not in (False, True, "mxfp4", "bf16"):
        raise ValueError(f"unknown precision contract {prefill!r}")
    mx = prefill is True or prefill == "mxfp4"
    x = np.asarray(x, dtype=np.float64)
    xin = mx_roundtrip(x) if mx else x
    g = xin @ np.asarray(w_gate, dtype=np.float64).T
    u = xin @ np.asarray(w_up, dtype=np.float64).T
    h = silu(g) * u
    if mx:
        hin = mx_roundtrip(h)
    elif prefill == "bf16":
        hin = bf16_roundtrip(h)
    else:
        hin = h
    o = hin @ np.asarray(w_down, dtype=np.float64).T
    return o, h


def combine(x, ids, w, experts, shared=None, prefill=False, include=None):
    """Weighted combine over the selected experts.

    x       [T, H] fp64
    ids     [T, k] expert ids; w [T, k] gate weights
    experts mapping / list: experts[e] = (w_gate, w_up, w_down) as fp64
    shared  (w_gate, w_up, w_down) of the shared expert, or None
    include optional [T, k] bool mask: only these pairs contribute (a partial
            sum); the shared expert contributes iff ``shared`` is given
    Returns y [T, H] fp64.

    Each expert runs once on the rows of every token routed to it; a token's
    output is the sum over its k experts of weight * expert output, plus the
    shared expert's output with weight 1.
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, k = ids.shape
    H = x.shape[1]
    if include is None:
        include = np.ones((T, k), dtype=bool)
    y = np.zeros((T, H), dtype=np.float64)
    for e in np.unique(ids):
        rows, slots = np.nonzero((ids == e) & include)
        if rows.size == 0:
            continue
        o, _ = expert_ffn(x[rows], *experts[int(e)], prefill=prefill)
        for r, (t, j) in enumerate(zip(rows, slots)):
            y[t] += w[t, j] * o[r]
    if shared is not None:
        o, _ = expert_ffn(x, *shared, prefill=prefill)
        y += o
    return y


def moe_layer(x, w_router, experts, k, shared=None, renorm=False,
              prefill=False):
    """Full layer: route then combine.  Returns (y [T, H], route dict)."""
    r = route(x, w_router, k, renorm=renorm)
    y = combine(x, r["ids"], r["w"], experts, shared=shared, prefill=prefill)
    return y, r


def merge(part_a, part_b):
    """Exact merge of two partial sums over disjoint expert subsets."""
    return np.asarray(part_a, dtype=np.float64) + np.asarray(part_b, dtype=np.float64)


def row_rel_error(got, ref):
    """max over rows of max|got - ref| / max|ref| (a row of zeros uses 1)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0

"""Algorithmic byte and FLOP counts of the routed MoE layer.

These are the bytes the method must move (weights of the distinct experts a
call touches, router weights, tokens in and outputs out) and the FLOPs of
the expert products; intermediates (h, sorted tokens, partial sums) and
padding are not counted.  They are the numerators of the roofline fractions
the benchmark reports.

Checked against the pages' own arithmetic: DeepSeek-V4-Flash's routed expert
set at FP4 is "roughly 140 GB" (ainewsfeed.tech article); GLM-5.2's 753B
parameters make a 433 GB NVFP4 checkpoint (explainx.ai guide, resource
table); moving a 64.4 GB expert pool at 52.7 GB/s takes the 1.19-1.22 s the
8,192-token prefill chunk took (explainx.ai guide, "Prefill: ...").
"""

MX_BLOCK = 32


def mxfp4_matrix_bytes(rows, K):
    """codes (K/2 bytes per row) + one e8m0 scale per 32 elements."""
    return rows * (K // 2) + rows * (K // MX_BLOCK)


def expert_bytes(hidden, inter, wtype):
    """Bytes of one SwiGLU expert (gate [I,H], up [I,H], down [H,I])."""
    if wtype == "bf16":
        return 3 * hidden * inter * 2
    if wtype == "f32":
        return 3 * hidden * inter * 4
    if wtype == "mxfp4":
        return 2 * mxfp4_matrix_bytes(inter, hidden) + mxfp4_matrix_bytes(hidden, inter)
    if wtype == "nvfp4":
        # e2m1 codes, an E4M3 byte per 16 elements, an fp32 scale per matrix
        return 3 * (hidden * inter // 2 + hidden * inter // 16 + 4)
    raise ValueError(wtype)


def router_bytes(hidden, n_experts, wtype):
    return hidden * n_experts * (4 if wtype == "f32" else 2)


def decode_call_bytes(hidden, inter, n_experts, wtype, T, n_distinct,
                      shared=False, route=True):
    """Algorithmic HBM bytes of one decode layer call.

    n_distinct: number of distinct routed experts the T tokens select.
    Counts expert weights once per distinct expert (+ shared), the router
    matrix once, x in (BF16), y out (fp32).
    """
    e = n_distinct + (1 if shared else 0)
    b = e * expert_bytes(hidden, inter, wtype)
    if route:
        b += router_bytes(hidden, n_experts, wtype)
    b += T * hidden * 2 + T * hidden * 4
    return b


def expected_distinct(n_experts, top_k, T):
    """E * (1 - (1 - k/E)^T): expected distinct experts of T uniform tokens."""
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** T)


def expert_flops(hidden, inter, pairs):
    """FLOPs of the three expert products over ``pairs`` (token, expert)."""
    return 2 * 3 * hidden * inter * pairs


def router_flops(hidden, n_experts, T):
    return 2 * T * n_experts * hidden

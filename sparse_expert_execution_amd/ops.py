"""PyTorch-facing wrappers over the C ABI (argument marshalling only).

Tensors supply device / pinned memory, torch streams supply hipStream_t.
Every step of the layer runs in libmoe.so's kernels; nothing here computes.
"""

import ctypes

import torch

from . import _lib
from ._lib import MoeDesc, MoePlan, check, lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(hidden, inter, n_experts, top_k, has_shared=False, renorm=False,
              wtype="mxfp4", router_wtype="bf16"):
    wt = {"bf16": _lib.WTYPE_BF16, "mxfp4": _lib.WTYPE_MXFP4, "nvfp4": _lib.WTYPE_NVFP4}[wtype]
    rt = {"f32": _lib.WTYPE_F32, "bf16": _lib.WTYPE_BF16}[router_wtype]
    return MoeDesc(hidden, inter, n_experts, top_k, int(has_shared), int(renorm), wt, rt)


def expert_layout(desc):
    off = (ctypes.c_size_t * 6)()
    nbytes = ctypes.c_size_t()
    check(lib().moe_expert_layout(ctypes.byref(desc), off, ctypes.byref(nbytes)),
          "moe_expert_layout")
    return list(off), nbytes.value


def workspace_bytes(desc, T, mode):
    return lib().moe_workspace_bytes(ctypes.byref(desc), T, mode)


def workspace(desc, T, mode, device="cuda"):
    """Zero-filled workspace (decode workspaces need a zero header once)."""
    n = max(workspace_bytes(desc, T, mode), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def route(desc, x, w_router, ids, w, ws, stream=None):
    T = x.shape[0]
    check(lib().moe_route(ctypes.byref(desc), _ptr(x), _ptr(w_router), T, _ptr(ids),
                          _ptr(w), _ptr(ws), ws.numel(), _stream(stream)), "moe_route")


def decode(desc, x, ids, w, pool, y, ws, slot_of=None, shared=None, stream=None):
    check(lib().moe_decode(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(ids), _ptr(w),
                           _ptr(slot_of), _ptr(pool), _ptr(shared), _ptr(y), _ptr(ws),
                           ws.numel(), _stream(stream)), "moe_decode")


def route_decode(desc, x, w_router, ids, w, pool, y, ws, slot_of=None, shared=None,
                 stream=None):
    check(lib().moe_route_decode(ctypes.byref(desc), _ptr(x), _ptr(w_router), x.shape[0],
                                 _ptr(ids), _ptr(w), _ptr(slot_of), _ptr(pool), _ptr(shared),
                                 _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
          "moe_route_decode")


def route_decode_noalloc(desc, x, w_router, ids, w, pool, y, wait_status=None, slot_of=None,
                         shared=None, stream=None):
    """moe_route_decode_noalloc: route_decode without a workspace (the
    library's static device scratch); wait_status: optional device int32[1]."""
    check(lib().moe_route_decode_noalloc(ctypes.byref(desc), _ptr(x), _ptr(w_router),
                                         x.shape[0], _ptr(ids), _ptr(w), _ptr(slot_of),
                                         _ptr(pool), _ptr(shared), _ptr(y), _ptr(wait_status),
                                         _stream(stream)), "moe_route_decode_noalloc")


def decode_launch_tokens(desc):
    """moe_decode_launch_tokens: tokens one decode launch takes for this shape."""
    n = lib().moe_decode_launch_tokens(ctypes.byref(desc))
    check(n if n < 0 else 0, "moe_decode_launch_tokens")
    return n


def decode_status(ws, clear=True, stream=None):
    """The decode workspace's wait-expired word (0: every wait inside the
    launches on ws since the last clear finished in time), read after
    synchronising the stream, then cleared when ``clear``."""
    out = torch.full((1,), -1, dtype=torch.int32, device=ws.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    check(lib().moe_decode_status(_ptr(ws), ws.numel(), _ptr(out), int(clear), _stream(s)),
          "moe_decode_status")
    s.synchronize()
    return int(out.item())


def prefill(desc, x, ids, w, pool, y, ws, slot_of=None, shared=None, stream=None):
    check(lib().moe_prefill(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(ids), _ptr(w),
                            _ptr(slot_of), _ptr(pool), _ptr(shared), _ptr(y), _ptr(ws),
                            ws.numel(), _stream(stream)), "moe_prefill")


def prefill_sort_view(desc, T, ws):
    """(seg_start, tiles, sorted_pair) int32 views into a prefill workspace
    (moe_debug_prefill_layout), read after a moe_prefill call on ws."""
    out = (ctypes.c_int64 * 5)()
    check(lib().moe_debug_prefill_layout(ctypes.byref(desc), T, out),
          "moe_debug_prefill_layout")
    seg, tiles, pairs, max_tiles, n_pairs = (int(v) for v in out)
    i32 = lambda off, n: ws[off:off + 4 * n].view(torch.int32)
    return i32(seg, desc.n_experts + 2), i32(tiles, 1 + 2 * max_tiles), i32(pairs, n_pairs)


def merge_partials(a, b, y, stream=None):
    check(lib().moe_merge_partials(_ptr(a), _ptr(b), _ptr(y), a.numel(), _stream(stream)),
          "moe_merge_partials")


def quantize_mxfp4(src, codes, scales, stream=None):
    """src [rows, K] float32 (device) -> codes [rows, K/2] u8, scales [rows, K/32] u8."""
    rows, K = src.shape
    check(lib().moe_quantize_mxfp4(_ptr(src), rows, K, src.stride(0), _ptr(codes),
                                   _ptr(scales), _stream(stream)), "moe_quantize_mxfp4")


def dequant_mxfp4(codes, scales, out, stream=None):
    check(lib().moe_debug_dequant_mxfp4(_ptr(codes), _ptr(scales), scales.numel(), _ptr(out),
                                        _stream(stream)), "moe_debug_dequant_mxfp4")


def dot_fp4(wtype, codes, scales, x, out, stream=None):
    """Decode gate/up block step (test hook): codes [n, 16] u8, scales [n]
    (MXFP4) or [n, 2] (NVFP4) u8, x [n_x, 32] bf16 -> out [n, n_x] float32."""
    wt = {"mxfp4": _lib.WTYPE_MXFP4, "nvfp4": _lib.WTYPE_NVFP4}[wtype]
    n, n_x = codes.shape[0], x.shape[0]
    if out.numel() != n * n_x or x.shape[1] != 32 or codes.shape[1] != 16:
        raise ValueError("dot_fp4: codes [n, 16], x [n_x, 32], out [n, n_x]")
    check(lib().moe_debug_dot_fp4(wt, _ptr(codes), _ptr(scales), _ptr(x), n, n_x, _ptr(out),
                                  _stream(stream)), "moe_debug_dot_fp4")


def mfma_fp4_tile(a_codes, a_scales, b_codes, b_scales, out, stream=None):
    check(lib().moe_debug_mfma_fp4_tile(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                                        _ptr(b_scales), _ptr(out), _stream(stream)),
          "moe_debug_mfma_fp4_tile")


def read_probe(buf, blocks, out, stream=None):
    check(lib().moe_debug_read_probe(_ptr(buf), buf.numel() * buf.element_size(), blocks,
                                     _ptr(out), _stream(stream)), "moe_debug_read_probe")


def wave_scan(inp, out, stream=None):
    """Inclusive scan of each group of 64 int32 values (device tensors)."""
    if inp.dtype != torch.int32 or out.dtype != torch.int32 or inp.numel() % 64 or \
            out.numel() != inp.numel() or not inp.is_contiguous() or not out.is_contiguous():
        raise ValueError("wave_scan takes contiguous int32 tensors of 64 n values")
    check(lib().moe_debug_wave_scan(_ptr(inp), _ptr(out), inp.numel() // 64, _stream(stream)),
          "moe_debug_wave_scan")


def qstar(m, b_pcie, b_host):
    return lib().moe_qstar(m, b_pcie, b_host)


def pack_expert(desc, block, gate, up, down, stream=None):
    """Write one expert into its byte block (a uint8 device tensor view) with
    moe_pack_expert.  gate/up/down: device fp32 or BF16 tensors, row-major."""
    dt = gate.dtype
    if dt not in (torch.float32, torch.bfloat16) or up.dtype != dt or down.dtype != dt:
        raise TypeError("expert matrices must all be float32 or all bfloat16")
    src = _lib.WTYPE_F32 if dt == torch.float32 else _lib.WTYPE_BF16
    g, u, d = (m.contiguous() for m in (gate, up, down))
    check(lib().moe_pack_expert(ctypes.byref(desc), _ptr(g), _ptr(u), _ptr(d), src, _ptr(block),
                                _stream(stream)), "moe_pack_expert")
    return expert_layout(desc)[1]


class Planner:
    """Host-only global LRU planner (moe_planner_*)."""

    def __init__(self, n_layers, n_experts, n_slots):
        self._h = ctypes.c_void_p()
        check(lib().moe_planner_create(ctypes.byref(self._h), n_layers, n_experts, n_slots),
              "moe_planner_create")
        self.n_experts = n_experts

    def __del__(self):
        if getattr(self, "_h", None):
            lib().moe_planner_destroy(self._h)
            self._h = None

    def set_bandwidths(self, b_pcie, b_host):
        check(lib().moe_planner_set_bandwidths(self._h, b_pcie, b_host), "set_bandwidths")

    def plan(self, layer, ids, w, q):
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
        p = MoePlan()
        check(lib().moe_planner_plan(self._h, layer, ids.ctypes.data_as(ctypes.c_void_p),
                                     w.ctypes.data_as(ctypes.c_void_p), ids.size, q,
                                     ctypes.byref(p)), "moe_planner_plan")
        return p

    def rollback(self):
        check(lib().moe_planner_rollback(self._h), "moe_planner_rollback")

    def slot_table(self, layer):
        import numpy as np
        out = np.empty(self.n_experts, dtype=np.int32)
        check(lib().moe_planner_slot_table(self._h, layer,
                                           out.ctypes.data_as(ctypes.c_void_p)),
              "moe_planner_slot_table")
        return out

    def resize(self, n_slots):
        """New slot budget; returns old_of_new (numpy int32 [n_slots])."""
        import numpy as np
        out = np.empty(n_slots, dtype=np.int32)
        check(lib().moe_planner_resize(self._h, n_slots, out.ctypes.data_as(ctypes.c_void_p)),
              "moe_planner_resize")
        return out

    @property
    def n_slots(self):
        return lib().moe_planner_n_slots(self._h)


def plan_dict(p):
    """A moe_plan as plain Python lists."""
    return {
        "layer": p.layer, "q": p.q,
        "selected": list(p.selected[:p.n_selected]),
        "hits": list(p.hits[:p.n_hits]), "hit_slot": list(p.hit_slot[:p.n_hits]),
        "misses": list(p.misses[:p.n_misses]),
        "fills": list(zip(p.fill_expert[:p.q], p.fill_slot[:p.q])),
        "victims": [(l, e) for l, e in zip(p.victim_layer[:p.q], p.victim_expert[:p.q])],
        "host": list(p.host_expert[:p.n_host]),
    }


class ExpertCache:
    """moe_cache_*: LRU slots in device memory filled from a pinned host pool.

    host_pool  pinned uint8 tensor [n_layers * n_experts * expert_bytes]
    dev_pool   device uint8 tensor [n_slots * expert_bytes]
    table      device int32 tensor [n_layers, n_experts] (kept by the cache)
    """

    def __init__(self, host_pool, n_layers, n_experts, expert_bytes, dev_pool, n_slots, table):
        self._h = ctypes.c_void_p()
        self._keep = (host_pool, dev_pool, table)
        check(lib().moe_cache_create(ctypes.byref(self._h), _ptr(host_pool), n_layers,
                                     n_experts, expert_bytes, _ptr(dev_pool), n_slots,
                                     _ptr(table)), "moe_cache_create")
        self.n_experts = n_experts

    def __del__(self):
        if getattr(self, "_h", None):
            lib().moe_cache_destroy(self._h)
            self._h = None

    def set_bandwidths(self, b_pcie, b_host):
        check(lib().moe_cache_set_bandwidths(self._h, b_pcie, b_host), "set_bandwidths")

    def plan(self, layer, ids, w, q):
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
        p = MoePlan()
        check(lib().moe_cache_plan(self._h, layer, ids.ctypes.data_as(ctypes.c_void_p),
                                   w.ctypes.data_as(ctypes.c_void_p), ids.size, q,
                                   ctypes.byref(p)), "moe_cache_plan")
        return p

    def fill(self, plan, side_stream, compute_stream=None):
        check(lib().cache_fill(self._h, ctypes.byref(plan), _stream(side_stream),
                               _stream(compute_stream)), "cache_fill")

    def release(self, plan, compute_stream=None):
        check(lib().moe_cache_release(self._h, ctypes.byref(plan), _stream(compute_stream)),
              "moe_cache_release")

    def resize(self, pool, n_slots, compute_stream=None):
        """Rebuild under n_slots slots held in `pool` (the current pool or a
        disjoint device buffer of n_slots * expert_bytes)."""
        check(lib().moe_cache_resize(self._h, _ptr(pool), n_slots, _stream(compute_stream)),
              "moe_cache_resize")

    def debug_fail_fills(self, n):
        check(lib().moe_cache_debug_fail_fills(self._h, n), "debug_fail_fills")

    def slot_table(self, layer):
        import numpy as np
        out = np.empty(self.n_experts, dtype=np.int32)
        check(lib().moe_planner_slot_table(lib().moe_cache_planner(self._h), layer,
                                           out.ctypes.data_as(ctypes.c_void_p)),
              "moe_planner_slot_table")
        return out


def host_experts(desc, x, ids, w, host_pool, y, include=None, host_index=None, threads=0):
    """moe_host_experts on host tensors: x [T][H] bf16, ids [T][k] int32, w [T][k]
    float32, include [T][k] uint8 or None, host_pool uint8 (pinned or not),
    host_index [E] int32 or None, y [T][H] float32 (overwritten)."""
    for t in (x, ids, w, host_pool, y) + tuple(v for v in (include, host_index) if v is not None):
        if t.is_cuda:
            raise ValueError("moe_host_experts takes host tensors")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    check(lib().moe_host_experts(ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(ids), _ptr(w),
                                 _ptr(include) if include is not None else None, _ptr(host_pool),
                                 _ptr(host_index) if host_index is not None else None, _ptr(y),
                                 threads), "moe_host_experts")


def host_expert_rate(desc, host_pool, n_experts=8, reps=3, threads=0):
    r = ctypes.c_double()
    check(lib().moe_host_expert_rate(ctypes.byref(desc), _ptr(host_pool), n_experts, reps,
                                     threads, ctypes.byref(r)), "moe_host_expert_rate")
    return r.value


def probe_bandwidths(pinned_host, dev, reps=3, threads=0, stream=None):
    bp, bh = ctypes.c_double(), ctypes.c_double()
    check(lib().moe_probe_bandwidths(_ptr(pinned_host), _ptr(dev), pinned_host.numel(), reps,
                                     threads, _stream(stream), ctypes.byref(bp),
                                     ctypes.byref(bh)), "moe_probe_bandwidths")
    return bp.value, bh.value


class LayerStream:
    """moe_layer_stream_*: full-layer streaming of expert blocks from a pinned
    host pool into one or two device buffers (double-buffered prefill).

    host_pool  pinned uint8 tensor of n_layers * layer_bytes
    bufs       one or two device uint8 tensors of layer_bytes each
    """

    def __init__(self, host_pool, n_layers, layer_bytes, bufs):
        self._h = ctypes.c_void_p()
        self._keep = (host_pool, tuple(bufs))
        b1 = _ptr(bufs[1]) if len(bufs) > 1 else None
        check(lib().moe_layer_stream_create(ctypes.byref(self._h), _ptr(host_pool), n_layers,
                                            layer_bytes, _ptr(bufs[0]), b1),
              "moe_layer_stream_create")
        self._bufs = list(bufs)

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().moe_layer_stream_destroy(self._h)
            self._h = ctypes.c_void_p()

    def acquire(self, layer, copy_stream, compute_stream=None):
        """Returns the device buffer (tensor) that holds `layer` for the work
        enqueued next on compute_stream."""
        out = ctypes.c_void_p()
        check(lib().moe_layer_stream_acquire(self._h, layer, _stream(copy_stream),
                                             _stream(compute_stream), ctypes.byref(out)),
              "moe_layer_stream_acquire")
        for b in self._bufs:
            if b.data_ptr() == out.value:
                return b
        raise RuntimeError("moe_layer_stream_acquire returned an unknown buffer")

    def release(self, layer, compute_stream=None):
        check(lib().moe_layer_stream_release(self._h, layer, _stream(compute_stream)),
              "moe_layer_stream_release")

#!/usr/bin/env python3
"""Benchmark of the routed MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

A step is one pass of the hot path over one batch: for each of the
workload's layers, moe_route then moe_decode (or moe_prefill), back to back on
one stream.  The headline workload is the Qwen3.6-35B-A3B-shaped BF16 decode
layer (hidden 2048, 128 routed experts, top-8, intermediate 768) at one token,
48 distinct layers per step; ``value`` is microseconds per token per MoE
layer.  Inputs are synthetic (seeded N(0, 0.02) weights, N(0, 1) tokens) and
resident in HBM before timing starts.  Other workloads (MXFP4 decode,
prefill, expert-cache decode) are reported under ``details``.

One JSON line is printed on stdout; progress goes to stderr.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import synth
from sparse_expert_execution_amd import bytemodel as bm

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK = 8.0e12            # bytes/s, MI355X published
FP4_PEAK = 10.1e15           # dense MXFP4 FLOP/s, MI355X published
BF16_PEAK = 2.5e15           # dense BF16 FLOP/s, MI355X published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def traffic_record(name):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None when the kernel sources changed since the counters were taken."""
    from sparse_expert_execution_amd import profiling
    path = os.path.join(ROOT, "profiles", f"{name}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != profiling.source_hash():
        return None
    return rec.get("bytes_per_launch")


class DecodeWaitExpired(RuntimeError):
    pass


def check_decode_status(ops, ws, what):
    """Every decode launch on ws since the last check finished its bounded
    waits in time; otherwise its output was wrong and the run is void."""
    if ops.decode_status(ws) != 0:
        raise DecodeWaitExpired(f"{what}: a wait inside the decode kernel expired "
                                "(the device was oversubscribed); the timed outputs are wrong")


# --------------------------------------------------------------------------
class Layers:
    """All layers of one workload resident in HBM."""

    def __init__(self, ops, name, n_layers, log_every=8, wtype=None):
        s = dict(synth.SHAPES[name])
        if wtype:
            s["wtype"] = wtype
        self.s = s
        self.name = name
        self.desc = ops.make_desc(s["hidden"], s["inter"], s["n_experts"], s["top_k"],
                                  has_shared=s["shared"], wtype=s["wtype"],
                                  router_wtype="bf16")
        _, eb = ops.expert_layout(self.desc)
        self.expert_bytes = eb
        E = s["n_experts"]
        self.pools, self.shared, self.routers = [], [], []
        t0 = time.time()
        for l in range(n_layers):
            pool = torch.empty(E * eb, dtype=torch.uint8, device="cuda")
            for e in range(E):
                g, u, d = synth.expert_weights(name, l, e, device="cuda")
                ops.pack_expert(self.desc, pool[e * eb:(e + 1) * eb], g, u, d)
            self.pools.append(pool)
            if s["shared"]:
                blk = torch.empty(eb, dtype=torch.uint8, device="cuda")
                g, u, d = synth.expert_weights(name, l, E, device="cuda")
                ops.pack_expert(self.desc, blk, g, u, d)
                self.shared.append(blk)
            else:
                self.shared.append(None)
            self.routers.append(synth.router_weights(name, l, device="cuda"))
            if (l + 1) % log_every == 0:
                torch.cuda.synchronize()
                log(f"{name}: {l + 1}/{n_layers} layers built ({time.time() - t0:.1f}s)")
        torch.cuda.synchronize()


def time_decode(ops, Lw, T, steps, warmup, mode="decode"):
    """Time `steps` passes over all layers; events around every expert call."""
    s = Lw.s
    n_layers = len(Lw.pools)
    H, k = s["hidden"], s["top_k"]
    xs = [synth.tokens(Lw.name, l, T, device="cuda") for l in range(n_layers)]
    ids = [torch.empty((T, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    ws_ = [torch.empty((T, k), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    ys = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    rws = ops.workspace(Lw.desc, T, 0)
    fmode = 1 if mode == "decode" else 2
    fws = ops.workspace(Lw.desc, T, fmode)
    fn = ops.decode if mode == "decode" else ops.prefill
    stream = torch.cuda.current_stream()

    def one_step(ev=None):
        for l in range(n_layers):
            if mode == "decode":
                # router + experts + combine in one call
                if ev is not None:
                    ev[l][0].record(stream)
                ops.route_decode(Lw.desc, xs[l], Lw.routers[l], ids[l], ws_[l], Lw.pools[l],
                                 ys[l], fws, shared=Lw.shared[l])
            else:
                ops.route(Lw.desc, xs[l], Lw.routers[l], ids[l], ws_[l], rws)
                if ev is not None:
                    ev[l][0].record(stream)
                fn(Lw.desc, xs[l], ids[l], ws_[l], Lw.pools[l], ys[l], fws,
                   shared=Lw.shared[l])
            if ev is not None:
                ev[l][1].record(stream)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    # distinct experts actually touched per layer (for the algorithmic bytes)
    distinct = [int(np.unique(i.cpu().numpy()).size) for i in ids]
    # the timed steps: calls back to back, events only around the whole run
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for st in range(steps):
        one_step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # a second pass with events around every expert call, on the stream the
    # kernels run on, for the per-launch duration of the dominant kernel
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(n_layers)] for _ in range(steps)]
    for st in range(steps):
        one_step(evs[st])
    torch.cuda.synchronize()
    call_ms = np.array([[e[0].elapsed_time(e[1]) for e in row] for row in evs])
    if mode == "decode":
        check_decode_status(ops, fws, f"{Lw.name} T={T}")
    return {"total_ms": total_ms, "step_ms": total_ms / steps, "call_ms": call_ms,
            "distinct": distinct, "ids": [i.cpu().numpy() for i in ids]}


def decode_record(ops, Lw, T, steps, warmup):
    s = Lw.s
    r = time_decode(ops, Lw, T, steps, warmup)
    n_layers = len(Lw.pools)
    H, I, E = s["hidden"], s["inter"], s["n_experts"]
    call_bytes = [bm.decode_call_bytes(H, I, E, s["wtype"], T, d, shared=s["shared"],
                                       route=True) for d in r["distinct"]]
    step_bytes = sum(call_bytes)
    step_s = r["step_ms"] * 1e-3
    mean_call_s = float(np.mean(r["call_ms"])) * 1e-3
    achieved = float(np.mean(call_bytes)) / mean_call_s
    return {
        "tokens": T, "layers": n_layers,
        "us_per_token_per_layer": step_s * 1e6 / (n_layers * T),
        "us_per_token_all_layers": step_s * 1e6 / T,
        "step_ms": r["step_ms"],
        "hbm_GBps_step": step_bytes / step_s / 1e9,
        "hbm_frac_step": step_bytes / step_s / HBM_PEAK,
        "decode_call_us": mean_call_s * 1e6,
        "decode_call_bytes": float(np.mean(call_bytes)),
        "decode_call_GBps": achieved / 1e9,
        "decode_call_frac": achieved / HBM_PEAK,
        "mean_distinct_experts": float(np.mean(r["distinct"])),
    }


def prefill_record(ops, Lw, T, steps, warmup):
    s = Lw.s
    r = time_decode(ops, Lw, T, steps, warmup, mode="prefill")
    H, I, E, k = s["hidden"], s["inter"], s["n_experts"], s["top_k"]
    pairs = T * (k + 1)
    flops = bm.expert_flops(H, I, pairs)
    distinct = r["distinct"][0] + (1 if s["shared"] else 0)
    wbytes = distinct * bm.expert_bytes(H, I, s["wtype"])
    io_bytes = T * H * 2 + T * H * 4
    call_s = float(np.mean(r["call_ms"])) * 1e-3
    step_s = r["step_ms"] * 1e-3
    alg_bytes = wbytes + io_bytes
    ai = flops / alg_bytes
    # MXFP4 runs FP4 x FP4 on the scaled matrix cores, NVFP4 BF16 x BF16
    peak = FP4_PEAK if s["wtype"] == "mxfp4" else BF16_PEAK
    bound = min(peak, ai * HBM_PEAK)
    return {
        "tokens": T, "weights": s["wtype"], "tokens_per_s": T / step_s, "step_ms": r["step_ms"],
        "prefill_call_us": call_s * 1e6,
        "expert_tflops": flops / call_s / 1e12,
        "mfma_peak_tflops": peak / 1e12,
        "mfma_frac_of_peak": flops / call_s / peak,
        "arithmetic_intensity": ai,
        "roofline_bound_tflops": bound / 1e12,
        "roofline_frac": (flops / call_s) / bound,
        "hbm_GBps_call": alg_bytes / call_s / 1e9,
    }


def prefill_stream_record(ops, Lp, host_pool, lb, T, n_layers, buffers):
    """Prefill over n_layers layers whose expert blocks stream from the pinned
    host pool through `buffers` (1 or 2) full-layer device buffers: per layer
    route, acquire (copy on a side stream), prefill, release.  The layers
    share one set of synthetic weights (copied into every host slot); each
    has its own synthetic tokens."""
    s = Lp.s
    H, k, E = s["hidden"], s["top_k"], s["n_experts"]
    eb = lb // (E + 1)
    bufs = [torch.empty(lb, dtype=torch.uint8, device="cuda") for _ in range(buffers)]
    ls = ops.LayerStream(host_pool, n_layers, lb, bufs)
    xs = [synth.tokens(Lp.name, l, T, device="cuda") for l in range(n_layers)]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    rws = ops.workspace(Lp.desc, T, 0)
    fws = ops.workspace(Lp.desc, T, 2)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()

    def one_pass():
        for l in range(n_layers):
            ops.route(Lp.desc, xs[l], Lp.routers[0], ids, w, rws)
            buf = ls.acquire(l, copy, comp)
            ops.prefill(Lp.desc, xs[l], ids, w, buf[:E * eb], y, fws, shared=buf[E * eb:])
            ls.release(l, comp)

    one_pass()                              # warm-up
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(comp)
    one_pass()
    e1.record(comp)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del ls, bufs
    return {"tokens": T, "layers": n_layers, "buffers": buffers,
            "ms_per_layer": ms / n_layers, "tokens_per_s": T * n_layers / (ms * 1e-3),
            "layer_bytes": lb, "stream_GBps": lb * n_layers / (ms * 1e-3) / 1e9}


def cache_record(ops, steps_limit=None, resize_at=None, q_sweep=None, sweep_steps=32):
    """Expert-cache decode: 64 LRU slots over a 256-expert pinned host pool,
    Zipf(1.1) trace drifting every 32 steps, q = q* from the measured PCIe
    rate and the measured host expert-kernel rate.  Per step: fills on a side
    stream, the GPU partial over resident + filled experts, the host partial
    over the other misses (moe_host_experts on the host cores, while the GPU
    works), then the exact merge on the GPU.  resize_at {step: n_slots}:
    elastic rebuilds of the cache before those steps (shrinking in place,
    growing into a pool allocated before the timed loop).  q_sweep [q, ...]:
    afterwards, the first sweep_steps steps again from a cold cache with each
    fixed q (clamped per step to the misses and free slots): µs per step, the
    fills, and the largest difference of y from the q = first-entry run (the
    split is exact, so y should not depend on q beyond rounding)."""
    name = "glm_cache_decode"
    s = synth.SHAPES[name]
    H, I, E, k, slots = s["hidden"], s["inter"], s["n_experts"], s["top_k"], s["slots"]
    steps = s["steps"] if steps_limit is None else steps_limit
    desc = ops.make_desc(H, I, E, k, wtype="mxfp4", router_wtype="bf16")
    _, eb = ops.expert_layout(desc)
    host_pool = torch.empty(E * eb, dtype=torch.uint8).pin_memory()
    stage = torch.empty(eb, dtype=torch.uint8, device="cuda")
    for e in range(E):
        g, u, d = synth.expert_weights(name, 0, e, device="cuda")
        ops.pack_expert(desc, stage, g, u, d)
        host_pool[e * eb:(e + 1) * eb].copy_(stage)
    dev_pool = torch.empty(slots * eb, dtype=torch.uint8, device="cuda")
    table = torch.empty((1, E), dtype=torch.int32, device="cuda")
    probe_dev = torch.empty(eb * 4, dtype=torch.uint8, device="cuda")
    bp, bh = ops.probe_bandwidths(host_pool[:eb * 4], probe_dev, reps=3)
    bx = ops.host_expert_rate(desc, host_pool, n_experts=8, reps=2)
    cache = ops.ExpertCache(host_pool, 1, E, eb, dev_pool, slots, table)
    cache.set_bandwidths(bp, bx)
    ids_tr, w_tr = synth.zipf_trace(E, k, steps, s["zipf"], s["drift"])
    xs = synth.tokens(name, 0, steps, device="cuda")
    xs_host = xs.cpu()
    d_ids = torch.from_numpy(ids_tr).cuda()
    d_w = torch.from_numpy(w_tr).cuda()
    h_ids = torch.from_numpy(ids_tr.astype(np.int32))
    h_w = torch.from_numpy(w_tr.astype(np.float32))
    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
    host_part = torch.zeros((steps, H), dtype=torch.float32).pin_memory()
    dev_part = torch.empty((1, H), dtype=torch.float32, device="cuda")
    host_experts = 0
    ws = ops.workspace(desc, 1, 1)
    side = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    hits = misses = fills = 0
    qs = []
    resize_at = resize_at or {}
    grow_pools, n_cur = {}, slots
    for st_r in sorted(resize_at):
        if resize_at[st_r] > n_cur:
            grow_pools[st_r] = torch.empty(resize_at[st_r] * eb, dtype=torch.uint8,
                                           device="cuda")
        n_cur = resize_at[st_r]
    phases = [[0, 0]]                      # [hits, misses] per budget phase
    rebuild_ev = []
    cur_pool = dev_pool
    # events around each step's decode (the GPU part of the split)
    dec_ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(steps)]
    gpu_experts = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.time()
    t_start.record(comp)
    for st in range(steps):
        if st in resize_at:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            cur_pool = grow_pools.get(st, cur_pool)
            e0.record(comp)
            cache.resize(cur_pool, resize_at[st], comp)
            e1.record(comp)
            rebuild_ev.append((st, resize_at[st], e0, e1))
            phases.append([0, 0])
        plan = cache.plan(0, ids_tr[st], w_tr[st], -1)
        hits += plan.n_hits
        misses += plan.n_misses
        phases[-1][0] += plan.n_hits
        phases[-1][1] += plan.n_misses
        fills += plan.q
        qs.append(plan.q)
        cache.fill(plan, side, comp)
        dec_ev[st][0].record(comp)
        ops.decode(desc, xs[st:st + 1], d_ids[st:st + 1], d_w[st:st + 1], cur_pool, y, ws,
                   slot_of=table[0])
        dec_ev[st][1].record(comp)
        gpu_experts.append(plan.n_hits + plan.q)
        cache.release(plan, comp)
        # the host side runs while the GPU works on the fills and the decode
        host = set(int(e) for e in ops.plan_dict(plan)["host"])
        if host:
            inc = torch.tensor([[int(e) in host for e in ids_tr[st]]], dtype=torch.uint8)
            ops.host_experts(desc, xs_host[st:st + 1], h_ids[st:st + 1], h_w[st:st + 1],
                             host_pool, host_part[st:st + 1], include=inc)
            host_experts += len(host)
        dev_part.copy_(host_part[st:st + 1], non_blocking=True)
        ops.merge_partials(y, dev_part, y)
    t_end.record(comp)
    torch.cuda.synchronize()
    wall = time.time() - wall0
    check_decode_status(ops, ws, "cache decode trace")
    dec_s = np.array([a.elapsed_time(b) for a, b in dec_ev]) * 1e-3
    gpu_bytes = np.array(gpu_experts, dtype=np.float64) * eb + H * 2 + H * 4
    gpu_part = {"gpu_part_us_per_step": float(dec_s.mean() * 1e6),
                "gpu_part_bytes_per_step": float(gpu_bytes.mean()),
                "gpu_part_GBps": float(gpu_bytes.sum() / dec_s.sum() / 1e9),
                "gpu_part_hbm_frac": float(gpu_bytes.sum() / dec_s.sum() / HBM_PEAK)}
    ms = t_start.elapsed_time(t_end)
    sweep = {}
    if q_sweep:
        ys_ref = None
        for qf in q_sweep:
            pool_q = torch.empty(slots * eb, dtype=torch.uint8, device="cuda")
            table_q = torch.empty((1, E), dtype=torch.int32, device="cuda")
            cq = ops.ExpertCache(host_pool, 1, E, eb, pool_q, slots, table_q)
            ys = torch.empty((sweep_steps, H), dtype=torch.float32, device="cuda")
            hp = torch.zeros((sweep_steps, H), dtype=torch.float32).pin_memory()
            n_fill = 0
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a0.record(comp)
            for st in range(sweep_steps):
                plan = cq.plan(0, ids_tr[st], w_tr[st], qf)
                n_fill += plan.q
                cq.fill(plan, side, comp)
                ops.decode(desc, xs[st:st + 1], d_ids[st:st + 1], d_w[st:st + 1], pool_q,
                           ys[st:st + 1], ws, slot_of=table_q[0])
                cq.release(plan, comp)
                host = set(int(e) for e in ops.plan_dict(plan)["host"])
                if host:
                    inc = torch.tensor([[int(e) in host for e in ids_tr[st]]],
                                       dtype=torch.uint8)
                    ops.host_experts(desc, xs_host[st:st + 1], h_ids[st:st + 1],
                                     h_w[st:st + 1], host_pool, hp[st:st + 1], include=inc)
                dev_part.copy_(hp[st:st + 1], non_blocking=True)
                ops.merge_partials(ys[st:st + 1], dev_part, ys[st:st + 1])
            a1.record(comp)
            torch.cuda.synchronize()
            check_decode_status(ops, ws, f"cache q sweep q={qf}")
            yc = ys.cpu().double()
            if ys_ref is None:
                ys_ref = yc
            diff = float(((yc - ys_ref).abs().amax(dim=1) /
                          ys_ref.abs().amax(dim=1).clamp_min(1e-30)).max())
            sweep[str(qf)] = {"us_per_step": a0.elapsed_time(a1) * 1e3 / sweep_steps,
                              "filled": n_fill, "max_rel_diff_y": diff}
            del cq
    return {
        "steps": steps, "slots": slots, "us_per_step": ms * 1e3 / steps,
        "wall_us_per_step": wall * 1e6 / steps,
        "hits": hits, "misses": misses, "filled": fills,
        "miss_rate": misses / max(1, hits + misses),
        "q_hist": np.bincount(np.array(qs), minlength=k + 1).tolist(),
        "b_pcie_GBps": bp / 1e9, "b_host_read_GBps": bh / 1e9,
        "b_host_expert_kernel_GBps": bx / 1e9, "host_experts_run": host_experts,
        "fill_GBps": fills * eb / (ms * 1e-3) / 1e9, **gpu_part,
        **({"budgets": [slots] + [n for _, n, _, _ in rebuild_ev],
            "rebuild_at_step": [st for st, _, _, _ in rebuild_ev],
            "rebuild_ms": [a.elapsed_time(b) for _, _, a, b in rebuild_ev],
            "miss_rate_per_budget": [m / max(1, h + m) for h, m in phases]}
           if rebuild_ev else {}),
        **({"q_sweep_cold_steps": sweep_steps, "q_sweep": sweep} if sweep else {}),
    }


# --------------------------------------------------------------------------
def cpu_baseline(name, T, n_layers_sample, min_seconds=10.0):
    """The fp64 oracle on the host cores: route + combine of the first
    ``n_layers_sample`` layers at T tokens, repeated until min_seconds."""
    import threadpoolctl
    from oracle import formats, layer as olayer
    s = synth.SHAPES[name]
    prepared = []
    for l in range(n_layers_sample):
        x = synth.tokens(name, l, T, device="cuda")
        bits = x.cpu().view(torch.int16).numpy().view(np.uint16)
        xf = formats.bf16_decode(bits)
        wr = synth.router_weights(name, l, device="cuda", as_dtype=torch.float32).cpu().numpy()
        wr = formats.bf16_decode(formats.bf16_round(wr))
        r = olayer.route(xf, wr, s["top_k"])
        experts = {}
        for e in np.unique(r["ids"]):
            mats = synth.expert_weights(name, l, int(e), device="cuda", as_dtype=torch.float32)
            conv = []
            for m in mats:
                a = m.cpu().numpy()
                conv.append(formats.bf16_decode(formats.bf16_round(a)) if s["wtype"] == "bf16"
                            else formats.mxfp4_decode(*formats.mxfp4_encode(a)))
            experts[int(e)] = tuple(conv)
        prepared.append((xf, wr, experts))
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    reps = 0
    t0 = time.time()
    while True:
        for xf, wr, experts in prepared:
            y, _ = olayer.moe_layer(xf, wr, experts, s["top_k"])
        reps += 1
        if time.time() - t0 >= min_seconds:
            break
    el = time.time() - t0
    per = el / (reps * n_layers_sample * T)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info
                   if i.get("user_api") == "blas"})
    return {"value": per * 1e6, "unit": "us/token/layer", "cores": threads,
            "kind": "oracle", "cpu": cpu, "blas": blas, "os_cpu_count": os.cpu_count(),
            "sample": f"{name} T={T}: route + combine of {n_layers_sample} layers "
                      f"(fp64 NumPy), repeated {reps}x over {el:.1f}s; weights decoded "
                      f"to fp64 before timing"}


def _oracle_expert_mats(name, layer, experts, wtype, threads=16):
    """fp64 (gate, up, down) of each expert id as the oracle decodes them,
    prepared in parallel host threads before any timing."""
    import concurrent.futures as cf
    from oracle import formats

    def one(e):
        mats = synth.expert_weights(name, layer, int(e), device="cuda", as_dtype=torch.float32)
        out = []
        for m in mats:
            a = m.cpu().numpy()
            if wtype == "bf16":
                out.append(formats.bf16_decode(formats.bf16_round(a)))
            elif wtype == "nvfp4":
                out.append(formats.nvfp4_decode(*formats.nvfp4_encode(a)))
            else:
                out.append(formats.mxfp4_decode(*formats.mxfp4_encode(a)))
        return tuple(out)

    experts = [int(e) for e in experts]
    with cf.ThreadPoolExecutor(min(threads, max(1, len(experts)))) as ex:
        return dict(zip(experts, ex.map(one, experts)))


def _time_reps(fn, min_seconds):
    reps, t0 = 0, time.time()
    while True:
        fn()
        reps += 1
        if time.time() - t0 >= min_seconds:
            return (time.time() - t0) / reps, reps


def _blas_threads():
    import threadpoolctl
    info = threadpoolctl.threadpool_info()
    return max([i.get("num_threads", 1) for i in info] or [1])


def oracle_layer_timing(name, T, n_sample, prefill=False, min_seconds=3.0):
    """The fp64 oracle on layer 0 of a workload at T tokens, on a bounded
    sample: the oracle routes all T tokens, then runs the expert FFNs and the
    combine of the first n_sample distinct routed experts (all their pairs;
    the shared expert too, when the layer has one, except in prefill) with
    weights decoded to fp64 beforehand, repeated for min_seconds.  The time is
    scaled to the whole layer by the experts run (decode: weight-read bound)
    or by the (token, expert) pairs (prefill: FLOP bound)."""
    from oracle import formats, layer as olayer
    s = synth.SHAPES[name]
    E, k, H, I = s["n_experts"], s["top_k"], s["hidden"], s["inter"]
    x = synth.tokens(name, 0, T, device="cuda")
    xf = formats.bf16_decode(x.cpu().view(torch.int16).numpy().view(np.uint16))
    wr = synth.router_weights(name, 0, device="cuda", as_dtype=torch.float32).cpu().numpy()
    wr = formats.bf16_decode(formats.bf16_round(wr))
    r = olayer.route(xf, wr, k)
    ids, w = r["ids"], r["w"]
    order = list(dict.fromkeys(int(e) for e in ids.ravel()))
    sample = order[:n_sample]
    use_shared = bool(s["shared"]) and not prefill
    want = sample + ([E] if use_shared else [])
    mats = _oracle_expert_mats(name, 0, want, s["wtype"])
    shared = mats.pop(E) if use_shared else None
    inc = np.isin(ids, sample)
    contract = "mxfp4" if prefill else False
    per_rep, reps = _time_reps(
        lambda: olayer.combine(xf, ids, w, mats, shared=shared, prefill=contract, include=inc),
        min_seconds)
    ebytes = bm.expert_bytes(H, I, s["wtype"])
    n_run = len(sample) + (1 if use_shared else 0)
    n_all = len(order) + (1 if s["shared"] else 0)
    if prefill:
        pairs_all = T * (k + (1 if s["shared"] else 0))
        layer_s = per_rep * pairs_all / int(inc.sum())
    else:
        layer_s = per_rep * n_all / n_run
    out = {"cores": _blas_threads(),
           "implied_weight_GBps": n_run * ebytes / per_rep / 1e9,
           "sample": f"{name} layer 0, T={T}: expert FFNs + combine of {len(sample)} of "
                     f"{len(order)} routed experts ({int(inc.sum())} pairs)"
                     f"{' and the shared expert' if use_shared else ''}, fp64 NumPy, "
                     f"{reps} reps; scaled by {'pairs' if prefill else 'experts'} to the layer"}
    if prefill:
        out.update(value=T / layer_s, unit="tokens/s")
    else:
        out.update(value=layer_s * 1e6 / T, unit="us/token/layer")
    return out


def oracle_cache_timing(min_seconds=3.0):
    """The oracle on the expert-cache workload: the full 512-step LRU
    simulation (q* from the pages' 51.5 GB/s PCIe and 178 GB/s host rates),
    and the FFN work of trace step 0 (8 experts, one token) scaled to a
    32-step window."""
    from oracle import cache as ocache, formats, layer as olayer
    name = "glm_cache_decode"
    s = synth.SHAPES[name]
    E, k, H, I = s["n_experts"], s["top_k"], s["hidden"], s["inter"]
    ids_tr, w_tr = synth.zipf_trace(E, k, s["steps"], s["zipf"], s["drift"])
    t0 = time.time()
    plans, _ = ocache.lru_sim(ids_tr, w_tr, s["slots"], E, b_pcie=51.5e9, b_host=178e9)
    lru_s = time.time() - t0
    misses = sum(len(p["misses"]) for p in plans)
    x = synth.tokens(name, 0, 1, device="cuda")
    xf = formats.bf16_decode(x.cpu().view(torch.int16).numpy().view(np.uint16))
    mats = _oracle_expert_mats(name, 0, ids_tr[0], s["wtype"])
    per_rep, reps = _time_reps(
        lambda: olayer.combine(xf, ids_tr[:1], w_tr[:1].astype(np.float64), mats), min_seconds)
    ebytes = bm.expert_bytes(H, I, s["wtype"])
    return {"value": per_rep * 1e6, "unit": "us/step (FFN work of one decode step)",
            "window_32_steps_s": 32 * per_rep, "lru_sim_512_steps_s": lru_s,
            "lru_sim_miss_rate": misses / (s["steps"] * k),
            "implied_weight_GBps": k * ebytes / per_rep / 1e9, "cores": _blas_threads(),
            "sample": f"{name}: the oracle's LRU over all {s['steps']} trace steps, and the "
                      f"expert FFNs + combine of step 0 ({k} experts, T=1), fp64 NumPy, "
                      f"{reps} reps, weights decoded to fp64 beforehand"}


def cpu_details():
    """Oracle timing of every workload (a bounded sample each)."""
    out = {}
    jobs = [("qwen_bf16_decode_T1", lambda: oracle_layer_timing("qwen_bf16_decode", 1, 8)),
            ("qwen_bf16_decode_T8", lambda: oracle_layer_timing("qwen_bf16_decode", 8, 16)),
            ("dsv4_mxfp4_decode_T1", lambda: oracle_layer_timing("dsv4_mxfp4_decode", 1, 6)),
            ("dsv4_mxfp4_decode_T4", lambda: oracle_layer_timing("dsv4_mxfp4_decode", 4, 6)),
            ("dsv4_mxfp4_decode_T16", lambda: oracle_layer_timing("dsv4_mxfp4_decode", 16, 6)),
            ("prefill_T4096", lambda: oracle_layer_timing("dsv4_mxfp4_prefill", 4096, 4,
                                                          prefill=True)),
            ("glm_cache_decode", oracle_cache_timing)]
    for key, fn in jobs:
        t0 = time.time()
        try:
            out[key] = fn()
        except Exception as ex:          # the GPU figures stand without it
            out[key] = {"error": repr(ex)}
        log(f"cpu oracle {key}: {json.dumps(out[key])} ({time.time() - t0:.1f}s)")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X, and "
              "sharding it across GPUs is not implemented (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    from sparse_expert_execution_amd import ops
    ops._lib.lib()
    torch.cuda.set_device(0)

    details = {}
    name = "qwen_bf16_decode"
    s = synth.SHAPES[name]
    log("building", name)
    Lq = Layers(ops, name, s["layers"], log_every=16)
    log("timing", name, "T=1")
    head = decode_record(ops, Lq, 1, args.steps, args.warmup)
    log(json.dumps(head))
    if not args.quick:
        details["qwen_bf16_decode_T8"] = decode_record(ops, Lq, 8, args.steps, args.warmup)
        log("T=8", json.dumps(details["qwen_bf16_decode_T8"]))
    del Lq
    torch.cuda.empty_cache()

    if not args.quick:
        try:
            name2 = "dsv4_mxfp4_decode"
            log("building", name2)
            Ld = Layers(ops, name2, synth.SHAPES[name2]["layers"], log_every=8)
            for T in (1, 4, 16):
                details[f"dsv4_mxfp4_decode_T{T}"] = decode_record(ops, Ld, T, args.steps,
                                                                   args.warmup)
                log(f"dsv4 T={T}", json.dumps(details[f"dsv4_mxfp4_decode_T{T}"]))
            del Ld
            torch.cuda.empty_cache()
        except DecodeWaitExpired:
            raise
        except Exception as ex:  # keep the headline line
            details["dsv4_mxfp4_decode_error"] = repr(ex)
        try:
            # the same layers with NVFP4 experts (E4M3 scale per 16 + fp32 per matrix)
            log("building", name2, "with NVFP4 experts")
            Ln = Layers(ops, name2, synth.SHAPES[name2]["layers"], log_every=8, wtype="nvfp4")
            for T in (1, 4):
                details[f"dsv4_nvfp4_decode_T{T}"] = decode_record(ops, Ln, T, args.steps,
                                                                   args.warmup)
                log(f"dsv4 nvfp4 T={T}", json.dumps(details[f"dsv4_nvfp4_decode_T{T}"]))
            del Ln
            torch.cuda.empty_cache()
        except DecodeWaitExpired:
            raise
        except Exception as ex:
            details["dsv4_nvfp4_decode_error"] = repr(ex)
        try:
            name3 = "dsv4_mxfp4_prefill"
            log("building", name3)
            Lp = Layers(ops, name3, 1)
            for T in (4096, 8192, 16384):
                details[f"prefill_T{T}"] = prefill_record(ops, Lp, T, max(3, args.steps // 4),
                                                          2)
                log(f"prefill T={T}", json.dumps(details[f"prefill_T{T}"]))
            # the same layer with NVFP4 experts (BF16 matrix cores)
            Lpn = Layers(ops, name3, 1, wtype="nvfp4")
            details["prefill_nvfp4_T4096"] = prefill_record(ops, Lpn, 4096,
                                                            max(3, args.steps // 4), 2)
            log("prefill nvfp4 T=4096", json.dumps(details["prefill_nvfp4_T4096"]))
            del Lpn
            torch.cuda.empty_cache()
            # full-layer streaming from a pinned host pool: two buffers vs one
            n_st = 4
            E3 = Lp.s["n_experts"]
            _, eb3 = ops.expert_layout(Lp.desc)
            lb = (E3 + 1) * eb3
            host_pool = torch.empty(n_st * lb, dtype=torch.uint8).pin_memory()
            host_pool[:E3 * eb3].copy_(Lp.pools[0])
            host_pool[E3 * eb3:lb].copy_(Lp.shared[0])
            for l in range(1, n_st):
                host_pool[l * lb:(l + 1) * lb].copy_(host_pool[:lb])
            for T in (4096, 8192, 16384):
                for nbuf in (2, 1):
                    key = f"prefill_stream_T{T}_{nbuf}buf"
                    details[key] = prefill_stream_record(ops, Lp, host_pool, lb, T, n_st, nbuf)
                    log(key, json.dumps(details[key]))
                d2 = details[f"prefill_stream_T{T}_2buf"]["tokens_per_s"]
                d1 = details[f"prefill_stream_T{T}_1buf"]["tokens_per_s"]
                details[f"prefill_stream_T{T}_single_buffer_loss"] = 1.0 - d1 / d2
            del host_pool
            del Lp
            torch.cuda.empty_cache()
        except DecodeWaitExpired:
            raise
        except Exception as ex:
            details["prefill_error"] = repr(ex)
        try:
            log("cache decode trace")
            details["glm_cache_decode"] = cache_record(ops, q_sweep=[0, 1, 2, 4, 8])
            log(json.dumps(details["glm_cache_decode"]))
        except DecodeWaitExpired:
            raise
        except Exception as ex:
            details["glm_cache_decode_error"] = repr(ex)
        try:
            log("cache decode trace, elastic budget 64 -> 32 -> 96 slots")
            details["glm_cache_decode_elastic"] = cache_record(ops, resize_at={170: 32, 340: 96})
            log(json.dumps(details["glm_cache_decode_elastic"]))
        except DecodeWaitExpired:
            raise
        except Exception as ex:
            details["glm_cache_decode_elastic_error"] = repr(ex)

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline("qwen_bf16_decode", 1, 4)
        log(json.dumps(cpu))
        if not args.quick:
            cpu["details"] = cpu_details()

    traffic = traffic_record("decode_qwen_bf16_T1")
    out = {
        "metric": "MoE layer decode us/token (HBM GB/s %peak); prefill tokens/s (MFMA %peak)",
        "value": head["us_per_token_per_layer"],
        "unit": "us/token/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["step_ms"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen3.6-35B-A3B-shaped BF16 MoE decode layer, 1 token, "
                               "48 distinct layers per step (route + expert FFNs + combine)",
                   "hidden": 2048, "inter": 768, "n_experts": 128, "top_k": 8,
                   "tokens": 1, "layers": 48},
        "roofline": {"bound": "hbm", "kernel": "moe_route_decode (one persistent kernel)",
                     "achieved": head["decode_call_GBps"], "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": head["decode_call_frac"],
                     "traffic": traffic},
        "hbm_GBps_whole_step": head["hbm_GBps_step"],
        "hbm_frac_whole_step": head["hbm_frac_step"],
        "cpu_baseline": cpu,
        "details": details,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    try:
        main()
    except DecodeWaitExpired as ex:
        print(f"bench.py: {ex}", file=sys.stderr, flush=True)
        sys.exit(3)

"""Reproducible inputs for rocprofv3 and the summaries kept under profiles/.

    python -m sparse_expert_execution_amd.profiling run <workload> [--tokens T]
        [--layers L] [--calls N]
        Builds L synthetic layers of a decode workload and makes N
        moe_route_decode calls over them, then one HBM read-probe launch of a
        known size and one plain device copy of a known size; run it under
        ``rocprofv3 --pmc FETCH_SIZE`` (then WRITE_SIZE) to calibrate the
        counters against kernels whose traffic is known.

    python -m sparse_expert_execution_amd.profiling run-prefill <workload>
        [--tokens T] [--calls N]
        Builds one synthetic layer (every expert resident) and makes N
        moe_route + moe_prefill calls over T tokens, then the same two
        calibration launches, for a kernel trace or the counters.

    python -m sparse_expert_execution_amd.profiling summarize --name NAME
        --stats run_kernel_stats.csv --fetch fetch.csv --write write.csv
        --alg-bytes B --cmd-stats "..." --cmd-fetch "..." --cmd-write "..."
        Writes profiles/NAME.md (per-kernel durations, bytes per launch) and
        profiles/NAME.traffic.json (HBM bytes per decode launch, scaled by the
        calibration, with a hash of the kernel sources it was taken on).

The traffic is per launch of the kernel named by --kernel (the decode kernel
by default); every kernel of the run gets a row of its own.  FETCH_SIZE and WRITE_SIZE are
KiB per dispatch summed over the L2 channels; each is multiplied by
known_bytes / (counter * 1024) of its calibration kernel.
"""

import argparse
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE_SOURCES = ["decode_impl.hpp", "decode_mfma.hpp", "decode_launch.hpp", "decode.hip",
                  "decode_bf16.hip", "decode_mxfp4.hip", "device.hpp", "kernels.hpp"]
PREFILL_SOURCES = ["prefill.hip", "device.hpp", "kernels.hpp"]
PROBE_BYTES = 256 << 20
SIMDS = 256 * 4                     # MI355X: 256 compute units x 4 SIMDs
XCDS = 8                            # GRBM_GUI_ACTIVE comes summed over the 8 XCDs
COPY_BYTES = 256 << 20


def source_hash(files=DECODE_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_expert_execution_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cmd_run(args):
    import torch
    sys.path.insert(0, ROOT)
    import synth
    from sparse_expert_execution_amd import ops
    s = synth.SHAPES[args.workload]
    desc = ops.make_desc(s["hidden"], s["inter"], s["n_experts"], s["top_k"],
                         has_shared=s["shared"], wtype=s["wtype"], router_wtype="bf16")
    _, eb = ops.expert_layout(desc)
    E, T = s["n_experts"], args.tokens
    layers = []
    for l in range(args.layers):
        pool = torch.empty(E * eb, dtype=torch.uint8, device="cuda")
        for e in range(E):
            ops.pack_expert(desc, pool[e * eb:(e + 1) * eb],
                            *synth.expert_weights(args.workload, l, e, device="cuda"))
        sh = None
        if s["shared"]:
            sh = torch.empty(eb, dtype=torch.uint8, device="cuda")
            ops.pack_expert(desc, sh, *synth.expert_weights(args.workload, l, E, device="cuda"))
        layers.append((pool, sh, synth.router_weights(args.workload, l, device="cuda"),
                       synth.tokens(args.workload, l, T, device="cuda")))
    ids = torch.empty((T, s["top_k"]), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s["top_k"]), dtype=torch.float32, device="cuda")
    y = torch.empty((T, s["hidden"]), dtype=torch.float32, device="cuda")
    ws = ops.workspace(desc, T, 1)
    torch.cuda.synchronize()
    for c in range(args.calls):
        pool, sh, wr, x = layers[c % len(layers)]
        ops.route_decode(desc, x, wr, ids, w, pool, y, ws, shared=sh)
    torch.cuda.synchronize()
    _calibrate(torch, ops)
    print(f"profiling run: {args.calls} decode calls of {args.workload} T={T}, probe "
          f"{PROBE_BYTES} B, copy {COPY_BYTES} B", flush=True)


def _calibrate(torch, ops):
    """A read of PROBE_BYTES and a copy writing COPY_BYTES, for the counters."""
    buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.read_probe(buf, 8192, out)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(2.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def cmd_run_prefill(args):
    import torch
    sys.path.insert(0, ROOT)
    import synth
    from sparse_expert_execution_amd import ops
    s = synth.SHAPES[args.workload]
    desc = ops.make_desc(s["hidden"], s["inter"], s["n_experts"], s["top_k"],
                         has_shared=s["shared"], wtype=s["wtype"], router_wtype="bf16")
    _, eb = ops.expert_layout(desc)
    E, T, k = s["n_experts"], args.tokens, s["top_k"]
    pool = torch.empty(E * eb, dtype=torch.uint8, device="cuda")
    for e in range(E):
        ops.pack_expert(desc, pool[e * eb:(e + 1) * eb],
                        *synth.expert_weights(args.workload, 0, e, device="cuda"))
    sh = None
    if s["shared"]:
        sh = torch.empty(eb, dtype=torch.uint8, device="cuda")
        ops.pack_expert(desc, sh, *synth.expert_weights(args.workload, 0, E, device="cuda"))
    wr = synth.router_weights(args.workload, 0, device="cuda")
    x = synth.tokens(args.workload, 0, T, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, s["hidden"]), dtype=torch.float32, device="cuda")
    rws = ops.workspace(desc, T, 0)
    ws = ops.workspace(desc, T, 2)
    torch.cuda.synchronize()
    for _ in range(args.calls):
        ops.route(desc, x, wr, ids, w, rws)
        ops.prefill(desc, x, ids, w, pool, y, ws, shared=sh)
    torch.cuda.synchronize()
    _calibrate(torch, ops)
    print(f"profiling run: {args.calls} route + prefill calls of {args.workload} T={T}",
          flush=True)


def _counter_rows(path, counter):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def _mean(xs):
    return sum(xs) / len(xs) if xs else None


def _stats_table(stats):
    lines = ["| kernel | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:12]:
        lines.append(f"| {r['Name'][:80]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    return lines


def cmd_summarize(args):
    stats = list(csv.DictReader(open(args.stats)))
    if not args.fetch:
        lines = [f"# {args.name}", "", "Kernel trace (rocprofv3 --kernel-trace --stats):", "",
                 f"    {args.cmd_stats}", ""] + _stats_table(stats)
        if args.note:
            lines += ["", args.note]
        os.makedirs(args.out_dir, exist_ok=True)
        with open(os.path.join(args.out_dir, f"{args.name}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    fetch = _counter_rows(args.fetch, "FETCH_SIZE")
    write = _counter_rows(args.write, "WRITE_SIZE")
    dec = lambda n: args.kernel in n
    probe = lambda n: "read_probe" in n
    copy = lambda n: "copy" in n.lower() or "elementwise" in n.lower()
    f_dec = _mean([v for n, v in fetch if dec(n)])
    f_probe = _mean([v for n, v in fetch if probe(n)])
    w_dec = _mean([v for n, v in write if dec(n)])
    # the calibration copy is the run's last copy kernel (earlier fills of
    # weights and workspaces also match the name test)
    w_copy = ([v for n, v in write if copy(n)] or [0.0])[-1] or None
    f_scale = PROBE_BYTES / (f_probe * 1024) if f_probe else None
    w_scale = COPY_BYTES / (w_copy * 1024) if w_copy else None
    fetch_b = f_dec * 1024 * f_scale if f_dec and f_scale else None
    write_b = w_dec * 1024 * w_scale if w_dec is not None and w_scale else None
    total = (fetch_b or 0) + (write_b or 0) if fetch_b is not None else None
    sources = DECODE_SOURCES if "decode" in args.kernel else PREFILL_SOURCES
    rec = {"name": args.name, "kernel": args.kernel, "source_hash": source_hash(sources),
           "bytes_per_launch": total, "fetch_bytes_per_launch": fetch_b,
           "write_bytes_per_launch": write_b, "alg_bytes_per_launch": args.alg_bytes,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_kib_raw": f_dec, "write_kib_raw": w_dec,
           "probe_fetch_kib": f_probe, "copy_write_kib": w_copy,
           "cmd_fetch": args.cmd_fetch, "cmd_write": args.cmd_write}
    os.makedirs(args.out_dir, exist_ok=True)
    with open(os.path.join(args.out_dir, f"{args.name}.traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# {args.name}", "", "Kernel trace (rocprofv3 --kernel-trace --stats):", "",
             f"    {args.cmd_stats}", ""] + _stats_table(stats)
    per = []
    for name in sorted({n for n, _ in fetch if not probe(n) and not copy(n)}):
        fk = _mean([v for n, v in fetch if n == name])
        wk = _mean([v for n, v in write if n == name])
        per.append(f"| {name[:72]} | {fk * 1024 * f_scale / 1e6:.1f} | "
                   f"{(wk or 0) * 1024 * (w_scale or 0) / 1e6:.1f} |")
    lines += ["", f"HBM traffic of `{args.kernel}` (rocprofv3 --pmc, one counter per run):", "",
              f"    {args.cmd_fetch}", f"    {args.cmd_write}", "",
              f"- FETCH_SIZE per launch: {f_dec} KiB raw; read-probe calibration "
              f"{f_probe} KiB for {PROBE_BYTES} B -> scale {f_scale}",
              f"- WRITE_SIZE per launch: {w_dec} KiB raw; copy calibration {w_copy} KiB for "
              f"{COPY_BYTES} B -> scale {w_scale}",
              f"- traffic per launch: {total} B (algorithmic {args.alg_bytes} B)",
              f"- kernel sources hash: {rec['source_hash']}", "",
              "Scaled HBM traffic per dispatch, every kernel of the run:", "",
              "| kernel | fetch MB | write MB |", "|---|---|---|"] + per
    if args.mfma:
        lines += ["", "Matrix-core counters per dispatch (rocprofv3 --pmc "
                  "SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE):", "",
                  f"    {args.cmd_mfma}", "",
                  "busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
                  f"{XCDS} XCDs x {SIMDS} SIMDs); FP4 TFLOP executed = MOPS_F6F4 x 512 / 1e12 "
                  "(padding rows of partly filled tiles included)", "",
                  "| kernel | FP4 TFLOP executed | MFMA busy |", "|---|---|---|"]
        mops = _counter_rows(args.mfma, "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
        busy = _counter_rows(args.mfma, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = _counter_rows(args.mfma, "GRBM_GUI_ACTIVE")
        for name in sorted({n for n, _ in mops if "gemm" in n}):
            mo = _mean([v for n, v in mops if n == name])
            bu = _mean([v for n, v in busy if n == name])
            gu = _mean([v for n, v in gui if n == name])
            frac = bu / (gu / XCDS * SIMDS) if bu is not None and gu else float("nan")
            lines.append(f"| {name[:72]} | {mo * 512 / 1e12:.3f} | {100 * frac:.1f}% |")
    if args.note:
        lines += ["", args.note]
    with open(os.path.join(args.out_dir, f"{args.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec))


def cmd_counters(args):
    """Mean of every counter per dispatch, for each kernel whose name holds
    --match, from one or more rocprofv3 --pmc counter csv files."""
    vals = {}
    for path in args.csv:
        with open(path) as f:
            for r in csv.DictReader(f):
                if args.match not in r.get("Kernel_Name", ""):
                    continue
                key = (r["Kernel_Name"][:90], r["Counter_Name"])
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    lines = ["| kernel | counter | mean per dispatch | dispatches |", "|---|---|---|---|"]
    for (k, c), v in sorted(vals.items()):
        lines.append(f"| {k} | {c} | {sum(v) / len(v):.6g} | {len(v)} |")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "a") as f:
            f.write(text)
    print(text)


def cmd_markers(args):
    """Per-range summary of the roctx ranges around the library's C-ABI calls
    from a rocprofv3 --marker-trace run (its marker_api_trace.csv)."""
    per = {}
    with open(args.csv) as f:
        for r in csv.DictReader(f):
            name = r.get("Function") or r.get("Message") or r.get("Name") or ""
            try:
                dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            except (KeyError, ValueError):
                continue
            per.setdefault(name, []).append(dt)
    lines = [f"# {args.name}", "", "roctx ranges around the C-ABI calls (host time of each call, "
             "rocprofv3 --marker-trace):", "", f"    {args.command}", "",
             "| range | calls | mean us | min us | max us |", "|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -len(kv[1])):
        lines.append(f"| {name} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    if args.note:
        lines += ["", args.note]
    text = "\n".join(lines) + "\n"
    os.makedirs(args.out_dir, exist_ok=True)
    with open(os.path.join(args.out_dir, f"{args.name}.md"), "w") as f:
        f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("workload")
    r.add_argument("--tokens", type=int, default=1)
    r.add_argument("--layers", type=int, default=8)
    r.add_argument("--calls", type=int, default=16)
    rp = sub.add_parser("run-prefill")
    rp.add_argument("workload")
    rp.add_argument("--tokens", type=int, default=4096)
    rp.add_argument("--calls", type=int, default=10)
    s = sub.add_parser("summarize")
    s.add_argument("--name", required=True)
    s.add_argument("--stats", required=True)
    s.add_argument("--fetch", default=None)
    s.add_argument("--write", default=None)
    s.add_argument("--note", default="")
    s.add_argument("--alg-bytes", type=float, default=None)
    s.add_argument("--kernel", default="decode_kernel",
                   help="name fragment of the kernel whose traffic is recorded")
    s.add_argument("--cmd-stats", default="")
    s.add_argument("--cmd-fetch", default="")
    s.add_argument("--cmd-write", default="")
    s.add_argument("--mfma", default=None, help="counter csv of the matrix-core pass")
    s.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    s.add_argument("--cmd-mfma", default="")
    c = sub.add_parser("counters")
    c.add_argument("--csv", nargs="+", required=True)
    c.add_argument("--match", default="")
    c.add_argument("--out", default=None)
    mk = sub.add_parser("markers")
    mk.add_argument("--csv", required=True)
    mk.add_argument("--name", required=True)
    mk.add_argument("--command", default="", help="the rocprofv3 command, for the record")
    mk.add_argument("--note", default="")
    mk.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        cmd_counters(a)
        return
    if a.cmd == "markers":
        cmd_markers(a)
        return
    if a.cmd == "run":
        cmd_run(a)
    elif a.cmd == "run-prefill":
        cmd_run_prefill(a)
    else:
        cmd_summarize(a)


if __name__ == "__main__":
    main()

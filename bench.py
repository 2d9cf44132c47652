#!/usr/bin/env python3
"""Throughput of the MoE token shuffle on one MI355X.

One step = the whole hot path on one batch: plan (count, scan, place),
dispatch send (x -> rank-major xr), dispatch fan-out (xr -> expert-major
xe), combine (identity expert: ye = xe -> out).  Inputs are seeded
synthetic data already resident in HBM when the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

Prints one JSON line.  `value` is algorithmic bytes per step / wall time per
step (GB/s, plan included); algorithmic bytes are what the method must
move: 2H(T+N) + 2H(N+Tk) + 2H(Tk+T) + 4(N+Tk) + 8Tk, with N the number of
deduplicated (token, rank) rows.

After the timed region, the same line carries: the per-kernel breakdown
(HIP events between the calls) and the `roofline` of the fan-out; the
flushed protocol (memory-side cache evicted before each rep, events around
plan / dispatch / combine); the measured copy ceiling (the library's
reference streaming copy of 4 GiB); the step replayed from HIP graphs;
parity of the last step against the CPU oracle; and the oracle's own
throughput on the host (`cpu_baseline`).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
METRIC = "dispatch+combine effective HBM GB/s (fraction of peak) and tokens/s, 1 GPU"
KERNEL_DIR = os.path.join(ROOT, "moe_expert_token_amd", "csrc")
KERNEL_SRCS = ("device_common.h", "plan.hip", "rows.hip", "reduce.hip", "combine_bwd.hip", "copy_ref.hip")
# The files that hold the row kernels (everything but the plan): the stored
# traffic records cover only kernels defined here, so a change to the plan
# leaves them valid.
DATA_KERNEL_SRCS = tuple(n for n in KERNEL_SRCS if n != "plan.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(T, H, k, N):
    row = 2 * H
    send = row * (T + N) + 4 * N
    fanout = row * (N + T * k) + 4 * T * k
    combine = row * (T * k + T) + 8 * T * k
    return {"send": send, "fanout": fanout, "combine": combine, "total": send + fanout + combine}


def bf16_order(u):
    """Monotone integer key of bf16 bit patterns (+0 and -0 equal)."""
    import numpy as np
    u = u.astype(np.int64)
    return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def source_digest(names=KERNEL_SRCS) -> str:
    """Hash of the kernel sources (the files that hold device code)."""
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode() + b"\0" + open(os.path.join(KERNEL_DIR, name), "rb").read())
    return h.hexdigest()[:16]


def data_source_digest() -> str:
    """Hash of the row kernels' sources (the plan's excluded)."""
    return source_digest(DATA_KERNEL_SRCS)


KERNEL_NAMES = {"plan": "plan_count/scan/place", "send": "dispatch_send_kernel",
                "fanout": "dispatch_fanout_kernel", "combine": "combine_rows_kernel"}


def load_traffic(workload: str, kernel: str):
    """HBM traffic from the committed rocprofv3 counter summary, only while the
    kernel source still matches the one that was profiled."""
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_NAMES[kernel]}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    if rec.get("data_kernel_src_sha256_16") != data_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def load_path_traffic(workload: str, path: str, calls):
    """HBM bytes of the given calls of a --path run (summed), from the
    committed counter summaries, only while the kernel source matches."""
    total = 0
    for call in calls:
        f = os.path.join(ROOT, "profiles", f"traffic_{path}_{call}_{workload}.json")
        try:
            rec = json.load(open(f))
        except (OSError, ValueError):
            return None
        if rec.get("data_kernel_src_sha256_16") != data_source_digest():
            return None
        total += rec["hbm_bytes_per_call"]
    return total


def copy_bytes_of(T, H, k):
    """Size of the reference copy: a buffer as large as xe, at most 2 GiB."""
    return min(T * k * H * 2, 2 << 30)


def runtime_copy_gbps(dev, T, H, k):
    """The runtime's device-to-device copy of copy_bytes_of(T, H, k) bytes
    (read + write GB/s).  It is also the kernel of known size that scales the
    FETCH_SIZE / WRITE_SIZE counters of a --pmc run."""
    import torch
    nbytes = copy_bytes_of(T, H, k)
    a = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        b.copy_(a)
    c1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9


CEILING_COPY_BYTES = 4 << 30  # size of the copy that measures the HBM ceiling


def stream_copy_ceiling(dev, nbytes=CEILING_COPY_BYTES, warmup=2, reps=10):
    """The measured HBM ceiling: the library's reference streaming copy
    (16-byte vectors, non-temporal) of nbytes, median over reps of its
    read + write GB/s, each rep between HIP events on the current stream."""
    import numpy as np
    import torch

    import moe_expert_token_amd as ms
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(warmup):
        ms.moe_shuffle_copy_reference(a, b)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        ms.moe_shuffle_copy_reference(a, b)
        e1.record()
    torch.cuda.synchronize()
    ms_med = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    del a, b
    return {"GBps": round(2 * nbytes / (ms_med * 1e-3) / 1e9, 1), "bytes": nbytes, "reps": reps,
            "kernel": "copy_reference_kernel (16-byte vectors, non-temporal)"}


def n_rank_rows(topk_idx, E, R):
    """Distinct (token, rank) pairs of a routing (bookkeeping for byte counts)."""
    import numpy as np
    T = topk_idx.shape[0]
    pairs = np.arange(T, dtype=np.int64)[:, None] * R + topk_idx // (E // R)
    return int(np.unique(pairs).size)


def pmc_summary(args):
    """Turns two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and one kernel
    trace of this bench into profiles/: a markdown table per workload and one
    traffic record per kernel.  FETCH_SIZE / WRITE_SIZE are KiB per dispatch;
    each is scaled by what it reads for the runtime's copy kernel of known
    size in the same run (the bench's copy-ceiling leg)."""
    import csv
    import collections

    import synth
    if not args.commands:
        raise SystemExit("--pmc-summary needs --commands (the rocprofv3 lines that wrote the CSVs, and this one)")
    cfg = synth.CONFIGS[args.config]
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    idx, _ = synth.make_routing(cfg, args.seed)
    N = n_rank_rows(idx, E, R)
    B = algorithmic_bytes(T, H, k, N)
    copy_bytes = copy_bytes_of(T, H, k)

    def per_kernel(path):
        vals = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    if not args.fetch_csv:  # kernel trace only (no counter runs)
        stats = {r["Name"]: r for r in csv.DictReader(open(args.trace_stats))}
        lines = [f"# Kernel time — {cfg.name}, path {args.path}", "",
                 f"T={T} H={H} E={E} k={k} R={R}, N={N}; kernel source sha256[:16] {args.src_sha or source_digest()}.",
                 "", "Command (run from the repository root on one MI355X):", ""]
        lines += [f"    {c}" for c in args.commands] + ["", "| kernel | calls | avg us | min us | max us |",
                                                          "|---|---|---|---|---|"]
        for n, r in stats.items():
            lines.append(f"| `{n.split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        with open(os.path.join(args.out_dir, f"kernels_{args.path}_{cfg.name}.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return
    fetch, write = per_kernel(args.fetch_csv), per_kernel(args.write_csv)
    copy_name = next(n for n in fetch if "copyBuffer" in n)
    f_factor = copy_bytes / (max(fetch[copy_name]) * 1024)
    w_factor = copy_bytes / (max(write[copy_name]) * 1024)
    stats = {r["Name"]: r for r in csv.DictReader(open(args.trace_stats))}
    if args.path != "forward":
        return pmc_path_summary(args, cfg, N, fetch, write, f_factor, w_factor, stats, copy_bytes)

    short = {"dispatch_send_kernel": "send", "dispatch_fanout_kernel": "fanout", "combine_rows_kernel": "combine"}
    digest = args.src_sha or source_digest()
    rows = []
    for name in sorted(set(fetch) & set(write)):
        if "copyBuffer" in name or "ms::" not in name:  # the library's kernels only
            continue
        base = name.split("(")[0].replace("void ", "").split("<")[0].replace("ms::", "")
        fb = sum(fetch[name]) / len(fetch[name]) * 1024 * f_factor
        wb = sum(write[name]) / len(write[name]) * 1024 * w_factor
        st = next((r for n, r in stats.items() if n.split("(")[0] == name.split("(")[0]), None)
        avg_us = float(st["AverageNs"]) / 1e3 if st else float("nan")
        if base == "copy_reference_kernel":  # the ceiling's copy: a check of the counter scale
            rows.append((base, name.split("(")[0], avg_us, fb, wb, 2 * CEILING_COPY_BYTES))
            continue
        alg = B.get(short.get(base, ""), None)
        rows.append((base, name.split("(")[0], avg_us, fb, wb, alg))
        if alg is not None:
            rec = {"kernel": base, "workload": cfg.name, "kernel_src_sha256_16": digest,
                   "data_kernel_src_sha256_16": args.data_src_sha or data_source_digest(),
                   "hbm_bytes_per_launch": round(fb + wb), "fetch_bytes_per_launch": round(fb),
                   "write_bytes_per_launch": round(wb), "alg_bytes_per_launch": alg,
                   "traffic_over_alg": round((fb + wb) / alg, 4),
                   "fetch_scale": round(f_factor, 4), "write_scale": round(w_factor, 4),
                   "copy_kernel_bytes": copy_bytes, "commands": args.commands}
            with open(os.path.join(args.out_dir, f"traffic_{base}_{cfg.name}.json"), "w") as f:
                json.dump(rec, f, indent=1)
    lines = [f"# Kernel time and HBM traffic — {cfg.name}", "",
             f"T={T} H={H} E={E} k={k} R={R}, N={N} deduplicated rank rows; kernel source sha256[:16] {digest}.", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in args.commands] + [""]
    lines += [f"Counter scale from the runtime copy kernel of {copy_bytes} bytes in the same runs: "
              f"FETCH_SIZE x {f_factor:.4f}, WRITE_SIZE x {w_factor:.4f}.", "",
              "| kernel | avg us (trace) | HBM read MB | HBM write MB | algorithmic MB | traffic / alg | GB/s alg |",
              "|---|---|---|---|---|---|---|"]
    for base, full, us, fb, wb, alg in sorted(rows, key=lambda r: -r[2] if r[2] == r[2] else 0):
        ratio = f"{(fb + wb) / alg:.3f}" if alg else "-"
        gbs = f"{alg / (us * 1e-6) / 1e9:.0f}" if alg and us == us else "-"
        lines.append(f"| `{full}` | {us:.1f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                     f"{(alg / 1e6 if alg else float('nan')):.1f} | {ratio} | {gbs} |")
    lines += ["", "Kernel trace summary (rocprofv3 --stats):", "", "| kernel | calls | avg us | min us | max us |",
              "|---|---|---|---|---|"]
    for n, r in stats.items():
        lines.append(f"| `{n.split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    with open(os.path.join(args.out_dir, f"kernels_{cfg.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_summary(args):
    """Turns rocprofv3 --pmc passes of one command (any counters among
    GRBM_GUI_ACTIVE, SQ_WAVES, SQ_WAVE_CYCLES, SQ_BUSY_CYCLES,
    SQ_WAIT_INST_ANY, TCC_EA0_RDREQ(_LEVEL), TCC_EA0_WRREQ(_LEVEL),
    TCP_TCC_READ_REQ(_LATENCY), TCP_PENDING_STALL_CYCLES, TA_TA_BUSY, ...)
    into a markdown table per kernel under profiles/: the raw per-dispatch
    means and the derived occupancy, stall and latency figures.  The
    GRBM_GUI_ACTIVE value of a dispatch is the sum over the XCDs, so one
    XCD's busy cycles are that divided by their count (from the agent info)."""
    import csv
    import collections
    if not args.title or not args.commands:
        raise SystemExit("--counter-summary needs --title and --commands (the rocprofv3 lines that wrote the CSVs)")
    digest = args.src_sha or source_digest()
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    seen = collections.defaultdict(set)
    agent = {}
    for path in args.counter_csv:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if args.kernel_filter and not any(f in name for f in args.kernel_filter):
                continue
            counter = r["Counter_Name"][:-4] if r["Counter_Name"].endswith("_sum") else r["Counter_Name"]
            vals[name][counter].append(float(r["Counter_Value"]))
            if (path, r["Dispatch_Id"]) not in seen[name]:  # one row per counter of a dispatch
                seen[name].add((path, r["Dispatch_Id"]))
                dur[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        info = os.path.join(os.path.dirname(path), "pmc_agent_info.csv")
        if os.path.exists(info):
            for row in csv.DictReader(open(info)):
                if row.get("Name", "").startswith("gfx"):
                    agent = row
    xcc, cus, wpc = int(agent.get("Num_Xcc", 8)), int(agent.get("Cu_Count", 256)), int(agent.get("Max_Waves_Per_Cu", 32))
    lines = [f"# Counters — {args.title} (kernel source sha256[:16] {digest})", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in args.commands] + [""]
    lines += [f"Device: {agent.get('Name', '?')}, {cus} CUs in {xcc} XCDs, at most {wpc} waves per CU.  "
              "Each figure is the mean over the kernel's dispatches in these runs.", "",
              "Derived figures (cycles of one XCD: G = GRBM_GUI_ACTIVE / XCDs):",
              "- occupancy = 4 * SQ_WAVE_CYCLES / (G * CUs * waves per CU) (SQ_WAVE_CYCLES counts 4-cycle units);",
              "- issue wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES;",
              "- L1 -> L2 read latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ (cycles), and reads in flight "
              "per CU = TCP_TCC_READ_REQ_LATENCY / (G * CUs);",
              "- TCP pending stall = TCP_PENDING_STALL_CYCLES / (G * CUs); TA busy = TA_TA_BUSY / (G * CUs);",
              "- L2 -> memory read latency = TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ (cycles), and reads in flight in "
              "the whole device = TCC_EA0_RDREQ_LEVEL / G (writes alike).", ""]
    hdr = ("| kernel | dispatches | mean us | occupancy | issue wait | L1->L2 read latency | reads in flight / CU | "
           "TCP pending stall | TA busy | L2->mem read latency | mem reads in flight | mem writes in flight |")
    lines += [hdr, "|" + "---|" * (hdr.count("|") - 1)]
    raw = ["", "Raw counters (means per dispatch):", ""]

    def fmt(x, f="{:.2f}"):
        return "-" if x is None else f.format(x)
    for name in sorted(vals, key=lambda n: -sum(dur[n]) / len(dur[n])):
        v = {c: sum(x) / len(x) for c, x in vals[name].items()}
        g = v.get("GRBM_GUI_ACTIVE")
        G = g / xcc if g else None

        def q(num, den):
            return v[num] / den if num in v and den else None
        occ = q("SQ_WAVE_CYCLES", G * cus * wpc / 4) if G else None
        wait = q("SQ_WAIT_INST_ANY", v.get("SQ_WAVE_CYCLES"))
        lat = q("TCP_TCC_READ_REQ_LATENCY", v.get("TCP_TCC_READ_REQ"))
        infl = q("TCP_TCC_READ_REQ_LATENCY", G * cus) if G else None
        pend = q("TCP_PENDING_STALL_CYCLES", G * cus) if G else None
        ta = q("TA_TA_BUSY", G * cus) if G else None
        elat = q("TCC_EA0_RDREQ_LEVEL", v.get("TCC_EA0_RDREQ"))
        erd = q("TCC_EA0_RDREQ_LEVEL", G) if G else None
        ewr = q("TCC_EA0_WRREQ_LEVEL", G) if G else None
        lines.append(f"| `{name}` | {len(dur[name])} | {sum(dur[name]) / len(dur[name]):.1f} | {fmt(occ)} | "
                     f"{fmt(wait)} | {fmt(lat, '{:.0f}')} | {fmt(infl, '{:.1f}')} | {fmt(pend)} | {fmt(ta)} | "
                     f"{fmt(elat, '{:.0f}')} | {fmt(erd, '{:.0f}')} | {fmt(ewr, '{:.0f}')} |")
        raw.append(f"- `{name}`: " + ", ".join(f"{c} {x:.4g}" for c, x in sorted(v.items())))
    with open(os.path.join(args.out_dir, args.out_name), "w") as f:
        f.write("\n".join(lines + raw) + "\n")
    print("\n".join(lines + raw))


# The kernels that make up each call of the other paths (by kernel name).
PATH_KERNELS = {
    "backward": {"combine_bwd": ("combine_bwd_grad_kernel", "combine_bwd_dot_kernel", "gate_grad_kernel"),
                 "sum_expert_rows": ("sum_expert_rows_kernel",), "sum_rank_rows": ("sum_rank_rows_kernel",)},
    "rank-partial": {"sum_expert_rows": ("gate_of_row_kernel", "sum_expert_rows_kernel"),
                     "sum_rank_rows": ("sum_rank_rows_kernel",)},
}
PATH_KERNELS["rank-partial-f32"] = PATH_KERNELS["rank-partial"]


def pmc_path_summary(args, cfg, N, fetch, write, f_factor, w_factor, stats, copy_bytes):
    """The counter summary of --path backward / rank-partial / rank-partial-f32:
    HBM bytes per launch of every kernel and, per call of the path, the sum
    over its kernels against the call's algorithmic bytes."""
    T, H, k = cfg.T, cfg.H, cfg.k
    B = path_bytes(args.path, T, H, k, N)
    digest = args.src_sha or source_digest()
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    per = {}
    for name in set(fetch) & set(write):
        if "copyBuffer" in name or "ms::" not in name:  # the library's kernels only
            continue
        base = name.split("(")[0].replace("void ", "").split("<")[0].replace("ms::", "")
        st = next((r for n, r in stats.items() if n.split("(")[0] == name.split("(")[0]), None)
        per[name.split("(")[0]] = (base, float(st["AverageNs"]) / 1e3 if st else float("nan"),
                                   mean(fetch[name]) * 1024 * f_factor, mean(write[name]) * 1024 * w_factor)
    lines = [f"# Kernel time and HBM traffic — {cfg.name}, path {args.path}", "",
             f"T={T} H={H} E={cfg.E} k={k} R={cfg.R}, N={N}; kernel source sha256[:16] {digest}.", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in args.commands] + [""]
    lines += [f"Counter scale from the runtime copy kernel of {copy_bytes} bytes in the same runs: "
              f"FETCH_SIZE x {f_factor:.4f}, WRITE_SIZE x {w_factor:.4f}.", "",
              "| call | kernels | avg us (trace, sum) | HBM read MB | HBM write MB | algorithmic MB | traffic / alg |",
              "|---|---|---|---|---|---|---|"]
    for call, kernels in PATH_KERNELS[args.path].items():
        mine = [v for v in per.values() if v[0] in kernels]
        us, fb, wb = sum(v[1] for v in mine), sum(v[2] for v in mine), sum(v[3] for v in mine)
        lines.append(f"| {call} | {', '.join(sorted(v[0] for v in mine))} | {us:.1f} | {fb / 1e6:.1f} | "
                     f"{wb / 1e6:.1f} | {B[call] / 1e6:.1f} | {(fb + wb) / B[call]:.3f} |")
        rec = {"path": args.path, "call": call, "kernels": sorted(v[0] for v in mine), "workload": cfg.name,
               "kernel_src_sha256_16": digest, "data_kernel_src_sha256_16": args.data_src_sha or data_source_digest(),
               "hbm_bytes_per_call": round(fb + wb),
               "fetch_bytes_per_call": round(fb), "write_bytes_per_call": round(wb),
               "alg_bytes_per_call": B[call], "traffic_over_alg": round((fb + wb) / B[call], 4),
               "fetch_scale": round(f_factor, 4), "write_scale": round(w_factor, 4),
               "copy_kernel_bytes": copy_bytes, "commands": args.commands}
        with open(os.path.join(args.out_dir, f"traffic_{args.path}_{call}_{cfg.name}.json"), "w") as f:
            json.dump(rec, f, indent=1)
    lines += ["", "| kernel | avg us (trace) | HBM read MB | HBM write MB |", "|---|---|---|---|"]
    for full, (base, us, fb, wb) in sorted(per.items(), key=lambda kv: -kv[1][1] if kv[1][1] == kv[1][1] else 0):
        lines.append(f"| `{full}` | {us:.1f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    lines += ["", "Kernel trace summary (rocprofv3 --stats):", "", "| kernel | calls | avg us | min us | max us |",
              "|---|---|---|---|---|"]
    for n, r in stats.items():
        lines.append(f"| `{n.split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    with open(os.path.join(args.out_dir, f"kernels_{args.path}_{cfg.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def path_bytes(path, T, H, k, N):
    """Algorithmic bytes per kernel of the other paths."""
    row = 2 * H
    if path == "backward":
        # combine backward: grad_out once, ye and grad_ye for every slot, rows+gates in, grad_w out
        cbwd = row * (T + 2 * T * k) + 12 * T * k
        # receiver: grad_xe rows in, one row per (token, rank) out; sender: those in, grad_x out
        recv = row * (T * k + N) + 4 * T * k
        send = row * (N + T) + 4 * N
        return {"combine_bwd": cbwd, "sum_expert_rows": recv, "sum_rank_rows": send, "total": cbwd + recv + send}
    # rank-partial combine: gate scatter, weighted receiver sum, sender sum
    prow = 2 * row if path == "rank-partial-f32" else row   # fp32 partial rows are twice as wide
    recv = row * T * k + prow * N + 16 * T * k
    send = prow * N + row * T + 4 * N
    return {"sum_expert_rows": recv, "sum_rank_rows": send, "total": recv + send}


def bench_path(args):
    """--path backward | rank-partial: the training direction (combine
    backward + dispatch backward, on the forward's plan) or the combine with
    one row per (token, rank) on the return path."""
    import numpy as np
    import torch

    import moe_expert_token_amd as ms
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    KR = min(k, R)
    log(f"[bench] {args.path} on {cfg.name}: generating inputs")
    idx_h, w_h = synth.make_routing(cfg, args.seed)
    ye_h = synth.make_expert_outputs(cfg, args.seed)
    rng = np.random.default_rng(args.seed + 7)
    g16 = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)  # noqa: E731
    idx, w, ye = torch.from_numpy(idx_h).to(dev), torch.from_numpy(w_h).to(dev), g16(ye_h)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device=dev)
    plan = ms.moe_shuffle_plan(dims, idx, ws)
    N = ms.moe_shuffle_plan_query(plan)["N"]
    rows = torch.empty((T * KR, H), dtype=torch.int16, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    if args.path == "backward":
        gxe_h = synth.wide_bf16(rng, (T * k, H), -8, 8)
        gout_h = synth.wide_bf16(rng, (T, H), -8, 8)
        gxe = g16(gxe_h)
        # rotate copies of the token-major input, as the forward path does with x
        nb = int(min(8, max(2, -(-(512 << 20) // max(T * H * 2, 1)))))
        gouts = [g16(gout_h)]
        gouts += [gouts[0].clone() for _ in range(nb - 1)]
        turn = [0]

        def next_gout():
            turn[0] += 1
            return gouts[turn[0] % nb]
        gye = torch.empty((T * k, H), dtype=torch.int16, device=dev)
        gw = torch.empty((T * k,), dtype=torch.float32, device=dev)
        names = ("combine_bwd", "sum_expert_rows", "sum_rank_rows")
        calls = (lambda: ms.moe_shuffle_combine_backward(plan, next_gout(), ye, w, gye, gw),
                 lambda: ms.moe_shuffle_sum_expert_rows(plan, gxe, None, rows),
                 lambda: ms.moe_shuffle_sum_rank_rows(plan, rows, out))
    elif args.path == "rank-partial":
        names = ("sum_expert_rows", "sum_rank_rows")
        calls = (lambda: ms.moe_shuffle_sum_expert_rows(plan, ye, w, rows),
                 lambda: ms.moe_shuffle_sum_rank_rows(plan, rows, out))
    else:  # rank-partial-f32: one call, both stages
        rows32 = torch.empty((T * KR, H), dtype=torch.float32, device=dev)
        names = ("combine_rank_partial_f32",)
        calls = (lambda: ms.moe_shuffle_combine_rank_partial_f32(plan, ye, w, rows32, out),)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):   # the timed region: nothing between the calls
        for c in calls:
            c()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):   # the per-call breakdown, with HIP events between the calls
        events[i][0].record()
        for j, c in enumerate(calls):
            c()
            events[i][j + 1].record()
    torch.cuda.synchronize()
    us = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]) * 1e3)
          for j, n in enumerate(names)}
    B = path_bytes(args.path, T, H, k, N)
    copy_gbps = runtime_copy_gbps(dev, T, H, k)
    parity = None
    if not args.no_parity:
        import oracle
        orc = oracle.get()
        rc, o = orc.plan(idx_h, H, E, R)
        if args.path == "backward":
            o_gxr, o_gx = orc.dispatch_backward(o, gxe_h, T, E, k, R)
            o_gye, _ = orc.combine_backward(o["comb_row"], gout_h, ye_h, w_h, E, R)
            parity = {"grad_xr_bitexact": bool(np.array_equal(rows[:N].cpu().numpy().view(np.uint16), o_gxr)),
                      "grad_x_bitexact": bool(np.array_equal(out.cpu().numpy().view(np.uint16), o_gx)),
                      "grad_ye_bitexact": bool(np.array_equal(gye.cpu().numpy().view(np.uint16), o_gye))}
        elif args.path == "rank-partial":
            o_part, o_out = orc.combine_rank_partial(o, ye_h, w_h, E, R)
            parity = {"partial_bitexact": bool(np.array_equal(rows[:N].cpu().numpy().view(np.uint16), o_part)),
                      "out_bitexact": bool(np.array_equal(out.cpu().numpy().view(np.uint16), o_out))}
        else:
            o_part, o_out = orc.combine_rank_partial_f32(o, ye_h, w_h, E, R)
            parity = {"partial_bitexact": bool(np.array_equal(rows32[:N].cpu().numpy().view(np.uint32),
                                                              o_part.view(np.uint32))),
                      "out_bitexact": bool(np.array_equal(out.cpu().numpy().view(np.uint16), o_out))}
        log(f"[bench] parity vs oracle: {parity}")
    if args.path == "rank-partial-f32":
        B = dict(B, combine_rank_partial_f32=B["total"])
    dom = max(names, key=lambda n: B[n])
    # the fp32-partial entry point is both calls of its path in one
    dom_calls = tuple(PATH_KERNELS[args.path]) if dom not in PATH_KERNELS[args.path] else (dom,)
    traffic = load_path_traffic(cfg.name, args.path, dom_calls)
    value = B["total"] / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": f"{args.path} shuffle effective HBM GB/s (fraction of peak), 1 GPU", "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "R": R, "N": N, "path": args.path},
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4), "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "kernel_us": {n: round(us[n], 2) for n in names}, "algorithmic_bytes": B, "accumulate": "fp32",
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(B[dom] / (us[dom] * 1e-6) / 1e9, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(B[dom] / (us[dom] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": B[dom], "avg_launch_us": round(us[dom], 2)},
        "runtime_copy_GBps": round(copy_gbps, 1),
        "cpu_baseline": None, "parity": parity, "kernel_src_sha256_16": source_digest(),
    }
    ms.moe_shuffle_plan_destroy(plan)
    return rec


def path_summary(rec):
    """The figures of a --path record, for the per_path object of the forward line."""
    return {"ms_per_step": rec["ms_per_step"], "GBps": rec["value"], "frac_of_peak": rec["frac_of_peak"],
            "tokens_per_s": rec["tokens_per_s"], "kernel_us": rec["kernel_us"],
            "algorithmic_bytes": rec["algorithmic_bytes"]["total"],
            "roofline": {"kernel": rec["roofline"]["kernel"], "frac": rec["roofline"]["frac"],
                         "traffic": rec["roofline"]["traffic"]},
            "parity": rec["parity"]}


def bench_pipelined(args):
    """--path pipelined: the forward step with dispatch and combine run per
    chunk of tokens, chunk i's combine on a second stream overlapping chunk
    i+1's dispatch.  Reports its time next to the sequential step's."""
    import numpy as np
    import torch

    import moe_expert_token_amd as ms
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    KR = min(k, R)
    inp = synth.make_inputs(cfg, args.seed)
    nb = int(min(8, max(2, -(-(512 << 20) // max(T * H * 2, 1)))))
    x0 = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    xs = [x0] + [x0.clone() for _ in range(nb - 1)]
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    w = torch.from_numpy(inp["topk_w"]).to(dev)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device=dev)
    xr = torch.empty((T * KR, H), dtype=torch.int16, device=dev)
    xe = torch.empty((T * k, H), dtype=torch.int16, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    tile = 256
    bounds = sorted({min(T, -(-(i * T // args.chunks) // tile) * tile) for i in range(args.chunks)} | {T})
    bounds = [0] + [b for b in bounds if b > 0]
    a = torch.cuda.current_stream()
    bstream = torch.cuda.Stream()
    cu_split, masked = None, []
    if args.cu_split > 0:
        # The dispatch stream on the first CUs of the mask, the combine stream
        # on the rest (HIP's CU-masked streams; each takes a hardware queue of
        # its own, so the run needs GPU_MAX_HW_QUEUES above the default 4).
        props = torch.cuda.get_device_properties(dev)
        ncu = props.multi_processor_count
        nd = max(1, min(ncu - 1, int(round(args.cu_split * ncu))))
        words = (ncu + 31) // 32

        def mask_of(lo, hi):
            m = [0] * words
            for c in range(lo, hi):
                m[c // 32] |= 1 << (c % 32)
            return (ctypes.c_uint32 * words)(*m)
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                     ctypes.POINTER(ctypes.c_uint32)]
        for lo, hi in ((0, nd), (nd, ncu)):
            h = ctypes.c_void_p()
            rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), words, mask_of(lo, hi))
            if rc != 0:
                raise SystemExit(f"hipExtStreamCreateWithCUMask failed with HIP error {rc}")
            masked.append(h)
        a = torch.cuda.ExternalStream(masked[0].value, device=dev)
        bstream = torch.cuda.ExternalStream(masked[1].value, device=dev)
        cu_split = {"dispatch_cus": nd, "combine_cus": ncu - nd}

    def step_seq(i):
        p = ms.moe_shuffle_plan(dims, idx, ws)
        ms.moe_shuffle_dispatch(p, xs[i % nb], xr, xe)
        ms.moe_shuffle_combine(p, xe, w, out)
        return p

    def step_pipe(i):
        if masked:  # the plan, too, on the dispatch stream, after the previous step's combine
            a.wait_stream(torch.cuda.current_stream())
        p = ms.moe_shuffle_plan(dims, idx, ws, stream=a)
        x = xs[i % nb]
        for t0, t1 in zip(bounds[:-1], bounds[1:]):
            ms.moe_shuffle_dispatch_range(p, x, xr, xe, t0, t1, stream=a)
            ev = torch.cuda.Event()
            ev.record(a)
            bstream.wait_event(ev)
            ms.moe_shuffle_combine_range(p, xe, w, out, t0, t1, stream=bstream)
        a.wait_stream(bstream)
        if masked:
            torch.cuda.current_stream().wait_stream(a)
        return p

    def timed(fn):
        for i in range(args.warmup):
            ms.moe_shuffle_plan_destroy(fn(i))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        plans = [fn(i) for i in range(args.steps)]
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) * 1e3 / args.steps
        for p in plans[:-1]:
            ms.moe_shuffle_plan_destroy(p)
        return dt, plans[-1]

    seq_ms, p = timed(step_seq)
    ms.moe_shuffle_plan_destroy(p)
    pipe_ms, p = timed(step_pipe)
    N = ms.moe_shuffle_plan_query(p)["N"]
    B = algorithmic_bytes(T, H, k, N)
    parity = None
    if not args.no_parity:
        import oracle
        orc = oracle.get()
        rc, o = orc.plan(inp["topk_idx"], H, E, R)
        oxr, oxe = orc.dispatch(o, inp["x"], E, k, R)
        oout = orc.combine(o["comb_row"], oxe, inp["topk_w"], E, R)
        parity = {"xr_bitexact": bool(np.array_equal(xr[:N].cpu().numpy().view(np.uint16), oxr)),
                  "xe_bitexact": bool(np.array_equal(xe.cpu().numpy().view(np.uint16), oxe)),
                  "out_bitexact": bool(np.array_equal(out.cpu().numpy().view(np.uint16), oout))}
    ms.moe_shuffle_plan_destroy(p)
    if masked:
        torch.cuda.synchronize()
        hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        for h in masked:
            hip.hipStreamDestroy(h)
    value = B["total"] / (pipe_ms * 1e-3) / 1e9
    rec = {"metric": "pipelined forward shuffle effective HBM GB/s (fraction of peak), 1 GPU",
           "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(pipe_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "R": R, "N": N, "path": "pipelined",
                      "token_chunks": bounds, "cu_split": cu_split},
           "frac_of_peak": round(value / PEAK_HBM_GBPS, 4), "sequential_ms_per_step": round(seq_ms, 4),
           "speedup_vs_sequential": round(seq_ms / pipe_ms, 4), "algorithmic_bytes": B, "parity": parity,
           "roofline": None, "cpu_baseline": None, "kernel_src_sha256_16": source_digest()}
    return rec


def forward_run(args, cfg_id, dev, full=True, ceiling=None):
    """The forward step (plan + send + fan-out + combine) on workload cfg_id:
    the timed region, the per-kernel event breakdown, the flushed protocol,
    the graph replay and the parity of the last step against the oracle.
    With full, also the runtime copy and (unless given) the measured copy
    ceiling, and the CPU baseline.  Returns the record of the JSON line."""
    import numpy as np
    import torch

    import moe_expert_token_amd as ms
    import synth

    cfg = synth.CONFIGS[cfg_id]
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    KR = min(k, R)
    log(f"[bench] workload {cfg.name}: generating inputs")
    inp = synth.make_inputs(cfg, args.seed)
    # Each step takes the next of NB resident copies of the batch, NB * |x| >=
    # 512 MiB (twice the 256 MiB memory-side cache), so no step finds the
    # previous step's activations still cached.
    x_bytes = T * H * 2
    nb = int(min(8, max(2, -(-(512 << 20) // max(x_bytes, 1)))))
    x0 = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    xs = [x0] + [x0.clone() for _ in range(nb - 1)]
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    w = torch.from_numpy(inp["topk_w"]).to(dev)
    dims = ms.dims_of(T, H, E, k, R)
    ws = torch.empty(ms.moe_shuffle_workspace_size(dims), dtype=torch.uint8, device=dev)
    xr = torch.empty((T * KR, H), dtype=torch.int16, device=dev)   # no host sync: sized by T*min(k,R)
    xe = torch.empty((T * k, H), dtype=torch.int16, device=dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()

    counter = [0]

    def step(ev=None):
        x = xs[counter[0] % nb]
        counter[0] += 1
        if ev is not None:
            ev[0].record()
        plan = ms.moe_shuffle_plan(dims, idx, ws)
        if ev is not None:
            ev[1].record()
        ms.moe_shuffle_dispatch_send(plan, x, xr)
        if ev is not None:
            ev[2].record()
        ms.moe_shuffle_dispatch_fanout(plan, xr, xe)
        if ev is not None:
            ev[3].record()
        ms.moe_shuffle_combine(plan, xe, w, out)      # identity expert: ye is xe
        if ev is not None:
            ev[4].record()
        return plan

    for _ in range(args.warmup):
        ms.moe_shuffle_plan_destroy(step())
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    # The timed region: K steps with nothing between the calls (an event
    # marker between two kernels costs a few microseconds of its own).
    plans = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        plans.append(step())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for p in plans:
        ms.moe_shuffle_plan_destroy(p)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # The per-kernel breakdown: K more steps with HIP events recorded between
    # the calls on the stream they run on.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    plans = []
    torch.cuda.synchronize()
    for i in range(args.steps):
        plans.append(step(events[i]))
    torch.cuda.synchronize()
    last_plan = plans[-1]
    for p in plans[:-1]:
        ms.moe_shuffle_plan_destroy(p)
    names = ("plan", "send", "fanout", "combine")
    us = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]) * 1e3)
          for j, n in enumerate(names)}
    step_ms = np.array([events[i][0].elapsed_time(events[i][4]) for i in range(args.steps)])
    info = ms.moe_shuffle_plan_query(last_plan)
    N = info["N"]
    B = algorithmic_bytes(T, H, k, N)
    log(f"[bench] {ms_per_step:.3f} ms/step; kernels (us): " + ", ".join(f"{n} {us[n]:.1f}" for n in names))

    copy_gbps = runtime_copy_gbps(dev, T, H, k) if full else None
    if ceiling is None:
        ceiling = stream_copy_ceiling(dev)

    # The flushed protocol: before each of K reps, an untimed read of 1 GiB
    # evicts the 256 MB memory-side cache (a read leaves no dirty lines to be
    # written back inside the timed region); HIP events then bracket the
    # plan, the dispatch (send + fan-out) and the combine of that rep.
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    flush.fill_(1)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    sink = []
    for i in range(args.steps):
        sink.append(flush.sum())
        e = fev[i]
        e[0].record()
        p = ms.moe_shuffle_plan(dims, idx, ws)
        e[1].record()
        ms.moe_shuffle_dispatch_send(p, x0, xr)
        ms.moe_shuffle_dispatch_fanout(p, xr, xe)
        e[2].record()
        ms.moe_shuffle_combine(p, xe, w, out)
        e[3].record()
        ms.moe_shuffle_plan_destroy(p)
    torch.cuda.synchronize()
    del flush, sink
    f_plan = np.array([e[0].elapsed_time(e[1]) for e in fev]) * 1e3
    f_disp = np.array([e[1].elapsed_time(e[2]) for e in fev]) * 1e3
    f_comb = np.array([e[2].elapsed_time(e[3]) for e in fev]) * 1e3
    f_dc = f_disp + f_comb
    f_gbps = B["total"] / (float(np.median(f_dc)) * 1e-6) / 1e9
    flushed = {"reps": args.steps, "flush": "1 GiB read before each rep, not timed",
               "t_plan_us": round(float(np.median(f_plan)), 2), "t_dispatch_us": round(float(np.median(f_disp)), 2),
               "t_combine_us": round(float(np.median(f_comb)), 2),
               "dc_us_p10_p50_p90": [round(float(np.percentile(f_dc, q)), 2) for q in (10, 50, 90)],
               "dispatch_combine_GBps": round(f_gbps, 1), "frac_of_peak": round(f_gbps / PEAK_HBM_GBPS, 4),
               "frac_of_copy_ceiling": round(f_gbps / ceiling["GBps"], 4),
               "tokens_per_s": round(T / (float(np.median(f_dc)) * 1e-6), 1)}
    log(f"[bench] flushed protocol: {flushed}")

    # The same step captured once per rotating batch in a HIP graph and
    # replayed: one launch call per step instead of four.  Replays run back
    # to back on the host clock like the timed region above.
    graphs, gplans = [], []
    for i in range(nb):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            p = ms.moe_shuffle_plan(dims, idx, ws)
            ms.moe_shuffle_dispatch_send(p, xs[i], xr)
            ms.moe_shuffle_dispatch_fanout(p, xr, xe)
            ms.moe_shuffle_combine(p, xe, w, out)
        graphs.append(g)
        gplans.append(p)
    for i in range(args.warmup):
        graphs[i % nb].replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % nb].replay()
    torch.cuda.synchronize()
    g_ms = (time.perf_counter() - g0) * 1e3 / args.steps
    for p in gplans:
        ms.moe_shuffle_plan_destroy(p)
    del graphs
    graph_replay = {"ms_per_step": round(g_ms, 4), "GBps": round(B["total"] / (g_ms * 1e-3) / 1e9, 1),
                    "tokens_per_s": round(T / (g_ms * 1e-3), 1), "graphs": nb}
    log(f"[bench] graph replay: {graph_replay}")

    parity, oracle_s = None, None
    if not args.no_parity:
        import oracle
        orc = oracle.get()
        o0 = time.perf_counter()
        rc, o = orc.plan(inp["topk_idx"], H, E, R)
        o1 = time.perf_counter()
        v = ms.plan_array_views(last_plan, N)
        plan_ok = rc == 0 and o["N"] == N and all(
            np.array_equal(v[key].cpu().numpy(), o[key])
            for key in ("send_token", "tok_rank_row", "fan_src", "fan_dst", "comb_row", "expert_offset",
                        "rank_offset", "rank_segs", "expert_segs"))
        o2 = time.perf_counter()
        oxr, oxe = orc.dispatch(o, inp["x"], E, k, R)
        o3 = time.perf_counter()
        xr_ok = np.array_equal(xr[:N].cpu().numpy().view(np.uint16), oxr)
        xe_ok = np.array_equal(xe.cpu().numpy().view(np.uint16), oxe)
        o4 = time.perf_counter()
        oout = orc.combine(o["comb_row"], oxe, inp["topk_w"], E, R)
        o5 = time.perf_counter()
        got = out.cpu().numpy().view(np.uint16)
        # the identity expert (ye = xe) with gates summing to 1 returns x, -0 as +0
        x_rt = np.where(inp["x"] == 0x8000, 0, inp["x"]).astype(np.uint16)
        parity = {"plan_bitexact": bool(plan_ok), "xr_bitexact": bool(xr_ok), "xe_bitexact": bool(xe_ok),
                  "out_max_ulp": int(np.abs(bf16_order(got) - bf16_order(oout)).max()),
                  "out_ndiff": int((got != oout).sum()), "out_bitexact": bool(np.array_equal(got, oout)),
                  "roundtrip_bitexact": bool(np.array_equal(got, x_rt))}
        # the oracle calls of this check, timed once (single-threaded C, not pinned)
        oracle_s = {"plan": round(o1 - o0, 4), "dispatch": round(o3 - o2, 4), "combine": round(o5 - o4, 4),
                    "cores": 1, "host_cpus": os.cpu_count()}
        log(f"[bench] parity vs oracle: {parity}; oracle seconds {oracle_s}")

    cpu = None
    if full and not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        allowed = sorted(os.sched_getaffinity(0))
        os.sched_setaffinity(0, {allowed[0]})  # the oracle is single-threaded: pin it to one core
        try:
            reps, tcpu = 0, 0.0
            parts = {"plan": [], "dispatch": [], "combine": []}
            while reps == 0 or (tcpu < args.cpu_budget_s and reps < 20):
                s0 = time.perf_counter()
                rc, o = orc.plan(inp["topk_idx"], H, E, R)
                s1 = time.perf_counter()
                oxr, oxe = orc.dispatch(o, inp["x"], E, k, R)
                s2 = time.perf_counter()
                orc.combine(o["comb_row"], oxe, inp["topk_w"], E, R)
                s3 = time.perf_counter()
                for key, dt in (("plan", s1 - s0), ("dispatch", s2 - s1), ("combine", s3 - s2)):
                    parts[key].append(dt)
                tcpu += s3 - s0
                reps += 1
        finally:
            os.sched_setaffinity(0, set(allowed))
        t_rep = tcpu / reps
        cpu = {"value": round(B["total"] / t_rep / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the full {cfg.name} workload, {reps} pass(es) of plan+dispatch+combine, "
                         f"single-threaded C oracle pinned to one core, {t_rep:.2f} s per pass",
               "tokens_per_s": round(T / t_rep, 1), "host_cpus": os.cpu_count(),
               "host_cpus_allowed": len(allowed), "cpu_model": cpu_model(),
               "median_s": {key: round(float(np.median(v)), 4) for key, v in parts.items()}}
        log(f"[bench] cpu oracle: {cpu}")

    # dominant kernel by algorithmic bytes: the receiver fan-out
    dom = max(("send", "fanout", "combine"), key=lambda n: B[n])
    achieved = B[dom] / (us[dom] * 1e-6) / 1e9
    traffic = load_traffic(cfg.name, dom)
    dc_us = us["send"] + us["fanout"] + us["combine"]
    value = B["total"] / (ms_per_step * 1e-3) / 1e9
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "R": R, "N": N,
                   "parallelism": f"ep{R}-logical-on-1gpu", "rotating_batches": nb},
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "dispatch_combine_GBps": round((B["send"] + B["fanout"] + B["combine"]) / (dc_us * 1e-6) / 1e9, 1),
        "dispatch_combine_frac_of_peak": round((B["total"]) / (dc_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "kernel_us": {n: round(us[n], 2) for n in names},
        "step_ms_event_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
        "algorithmic_bytes": B,
        "copy_ceiling": ceiling,
        "frac_of_copy_ceiling": round(value / ceiling["GBps"], 4),
        "runtime_copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        "flushed_protocol": flushed,
        "graph_replay": graph_replay,
        "accumulate": "fp32",
        "roofline": {"kernel": KERNEL_NAMES[dom], "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": B[dom], "avg_launch_us": round(us[dom], 2)},
        "cpu_baseline": cpu,
        "parity": parity,
        "oracle_s": oracle_s,
        "kernel_src_sha256_16": source_digest(),
    }
    ms.moe_shuffle_plan_destroy(last_plan)
    del xs, x0, idx, w, ws, xr, xe, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec




def config_summary(rec):
    """The per-workload figures of a forward record, for the per_config object."""
    f, g, c = rec["flushed_protocol"], rec["graph_replay"], rec["config"]
    return {
        "workload": c["workload"], "T": c["T"], "H": c["H"], "E": c["E"], "k": c["k"], "R": c["R"], "N": c["N"],
        "algorithmic_bytes": rec["algorithmic_bytes"]["total"],
        "ms_per_step": rec["ms_per_step"], "GBps": rec["value"], "frac_of_peak": rec["frac_of_peak"],
        "tokens_per_s": rec["tokens_per_s"],
        "kernel_us": rec["kernel_us"],
        "dispatch_combine_GBps": rec["dispatch_combine_GBps"],
        "dispatch_combine_frac_of_peak": rec["dispatch_combine_frac_of_peak"],
        "flushed": {"t_plan_us": f["t_plan_us"], "t_dispatch_us": f["t_dispatch_us"],
                    "t_combine_us": f["t_combine_us"], "dc_us_p10_p50_p90": f["dc_us_p10_p50_p90"],
                    "dispatch_combine_GBps": f["dispatch_combine_GBps"], "frac_of_peak": f["frac_of_peak"],
                    "frac_of_copy_ceiling": f["frac_of_copy_ceiling"], "tokens_per_s": f["tokens_per_s"]},
        "graph_replay": {"ms_per_step": g["ms_per_step"], "GBps": g["GBps"], "tokens_per_s": g["tokens_per_s"]},
        "roofline_frac": rec["roofline"]["frac"],
        "parity": rec["parity"],
        "oracle_s": rec["oracle_s"],
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (0..4); default: DeepSeek-V3-like")
    ap.add_argument("--per-config", default="0,1,2,3,4",
                    help="workloads whose figures go into the per_config object of the forward line "
                         "(comma-separated ids, or none)")
    ap.add_argument("--per-path", default="auto",
                    help="other paths whose figures on the same workload go into the per_path object of the "
                         "forward line (comma-separated, or none; auto: backward, rank-partial, "
                         "rank-partial-f32 and pipelined unless --per-config is none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget-s", type=float, default=12.0, help="CPU-oracle timing budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--chunks", type=int, default=4, help="token chunks for --path pipelined")
    ap.add_argument("--cu-split", type=float, default=0.0,
                    help="--path pipelined: run dispatch and combine on CU-masked streams, this fraction of the "
                         "CUs for dispatch (0: two ordinary streams)")
    ap.add_argument("--path", default="forward",
                    choices=("forward", "backward", "rank-partial", "rank-partial-f32", "pipelined"),
                    help="forward (default): plan + dispatch + combine; backward: combine and dispatch backward; "
                         "rank-partial: combine through one row per (token, rank); rank-partial-f32: the same "
                         "with fp32 partial rows")
    ap.add_argument("--pmc-summary", action="store_true", help="summarise rocprofv3 CSVs into profiles/ (no GPU)")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--trace-stats")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--src-sha", default=None, help="kernel source hash of the profiled run (default: current)")
    ap.add_argument("--data-src-sha", default=None,
                    help="row-kernel source hash of the profiled run (default: current)")
    ap.add_argument("--counter-summary", action="store_true",
                    help="summarise rocprofv3 --pmc CSVs of any counters into profiles/ (no GPU)")
    ap.add_argument("--counter-csv", nargs="*", default=[])
    ap.add_argument("--kernel-filter", nargs="*", default=[])
    ap.add_argument("--out-name", default="counters.md")
    ap.add_argument("--title", default="")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the shuffle runs its expert-parallel ranks as logical "
              f"partitions of one GPU's HBM (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_expert_token_amd as ms

    if not os.path.exists(ms.LIB_PATH):
        from moe_expert_token_amd import build as hip_build
        hip_build.build()
    ms.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    if args.path == "pipelined":
        print(json.dumps(bench_pipelined(args)), flush=True)
        return
    if args.path != "forward":
        print(json.dumps(bench_path(args)), flush=True)
        return

    head = forward_run(args, args.config, dev, full=True)
    ids = [int(c) for c in args.per_config.split(",") if c.strip()] if args.per_config != "none" else []
    if ids:
        per = {}
        for cid in ids:
            if cid == args.config:
                per[str(cid)] = config_summary(head)
            else:
                per[str(cid)] = config_summary(forward_run(args, cid, dev, full=False,
                                                           ceiling=head["copy_ceiling"]))
        head["per_config"] = per
    per_path = args.per_path
    if per_path == "auto":
        per_path = "none" if args.per_config == "none" else "backward,rank-partial,rank-partial-f32,pipelined"
    paths = [p.strip() for p in per_path.split(",") if p.strip()] if per_path != "none" else []
    if paths:
        head["per_path"] = {}
        for p in paths:
            torch.cuda.empty_cache()
            sub = argparse.Namespace(**vars(args))
            sub.path = p
            if p == "pipelined":
                rec = bench_pipelined(sub)
                head["per_path"][p] = {"ms_per_step": rec["ms_per_step"], "GBps": rec["value"],
                                       "frac_of_peak": rec["frac_of_peak"],
                                       "sequential_ms_per_step": rec["sequential_ms_per_step"],
                                       "speedup_vs_sequential": rec["speedup_vs_sequential"],
                                       "token_chunks": rec["config"]["token_chunks"], "parity": rec["parity"]}
            else:
                head["per_path"][p] = path_summary(bench_path(sub))
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()

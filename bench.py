"""Benchmark of the fused tied LM head + softcap cross-entropy -> bits-per-byte path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-train] [--no-cpu] [--cold]
    python bench.py --calibrate-copy              # plain 512 MiB copy, for HBM counter scaling
    python bench.py --summarize-counters DIR      # rocprofv3 counter CSVs -> profiles/ summaries

A step is one pass of the scoring path over one synthetic batch shaped like the challenge's main
evaluation (T = 32 x 2048 rows, D = 512, V = 8192 BPE entries, bf16, softcap 30, every row scored):
the fused forward (logits, softcap, log-sum-exp, target gather) and the bits-per-byte reduction.
Inputs are resident in HBM before the timed region. The training step on the same shape (forward +
backward: recompute, dZ, dH, dE) is timed as well and reported beside it.

Prints one JSON line. `roofline` is for the dominant kernel (the fused forward): algorithmic
2*T*D*V FLOP per launch over its average launch time, measured with HIP events on its stream,
against the bf16 dense MFMA peak. `cpu_baseline` is the float64 oracle timed on a bounded row
sample on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_mfma_T65536_D512_V8192_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "lm_head_cross_pg_amd", "csrc", f)
                  for f in ("pg_fwd.hip", "pg_common.h", "pg_tile.h")]
# the symmetric, fixed-shift forward on a bf16 head (no dZ, not the int8 head)
FWD_KERNEL = "fwd_mfma_kernel<512, true, 1, false, false, false"
COPY_BYTES = 1 << 29          # --calibrate-copy moves 512 MiB each way per launch


def kernel_source_hash() -> str:
    """Hash of the forward kernel's sources without comments and blank space, so that the counter
    runs stay attached to the code they measured across comment edits."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the fused forward from the committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def _counter_rows(d):
    """Rows of every rocprofv3 *_counter_collection.csv below directory d."""
    import csv
    rows = []
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(root, f)) as fh:
                    rows.extend(csv.DictReader(fh))
    return rows


def _long_dispatches(rows, match):
    """Dispatch ids of the rows that satisfy match whose duration is at least half the longest of
    them: the full-size launches of a kernel that also runs on masked batches of the same grid."""
    dur = {}
    for r in rows:
        if match(r):
            dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    top = max(dur.values(), default=0)
    return {k for k, v in dur.items() if 2 * v >= top}


def _per_dispatch(rows, name_part, counter, long_only=False):
    """Mean over dispatches of kernels whose name contains name_part of one counter (summed over
    the per-agent rows of a dispatch); long_only keeps the full-size launches (_long_dispatches)."""
    match = lambda r: name_part.lower() in r["Kernel_Name"].lower()
    keep = _long_dispatches(rows, match) if long_only else None
    per = {}
    for r in rows:
        if match(r) and r["Counter_Name"] == counter and (keep is None or r["Dispatch_Id"] in keep):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return (sum(per.values()) / len(per), len(per)) if per else (None, 0)


def summarize_counters(d):
    """Turn the counter runs under d (fetch/, write/, calib_fetch/, calib_write/, mfma/, each a
    rocprofv3 --pmc output directory) into the traffic file read by the roofline report and a
    short markdown summary next to it."""
    out = {"kernel": FWD_KERNEL + ">", "workload": "fwd_v8192 T=65536 D=512 V=8192",
           "kernel_source_sha256_16": kernel_source_hash()}
    cf, _ = _per_dispatch(_counter_rows(os.path.join(d, "calib_fetch")), "copy", "FETCH_SIZE")
    cw, _ = _per_dispatch(_counter_rows(os.path.join(d, "calib_write")), "copy", "WRITE_SIZE")
    ff, nf = _per_dispatch(_counter_rows(os.path.join(d, "fetch")), FWD_KERNEL, "FETCH_SIZE", long_only=True)
    fw, nw = _per_dispatch(_counter_rows(os.path.join(d, "write")), FWD_KERNEL, "WRITE_SIZE", long_only=True)
    lines = ["# HBM traffic of the fused forward (T=65536, D=512, V=8192)", ""]
    if None in (cf, cw, ff, fw):
        raise SystemExit("missing counter runs under " + d)
    kf, kw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    fetch_b, write_b = ff * 1024.0 * kf, fw * 1024.0 * kw
    out.update({"copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_scale": kf, "write_scale": kw,
                "fetch_kib_per_launch": ff, "write_kib_per_launch": fw, "launches": [nf, nw],
                "fetch_bytes": fetch_b, "write_bytes": write_b, "bytes_per_launch": fetch_b + write_b})
    lines += ["| quantity | value |", "|---|---|",
              f"| copy kernel, 512 MiB each way: FETCH_SIZE | {cf:.0f} KiB (scale {kf:.3f}) |",
              f"| copy kernel: WRITE_SIZE | {cw:.0f} KiB (scale {kw:.3f}) |",
              f"| forward FETCH_SIZE per launch ({nf} launches) | {ff:.0f} KiB -> {fetch_b / 2**20:.1f} MiB |",
              f"| forward WRITE_SIZE per launch ({nw} launches) | {fw:.0f} KiB -> {write_b / 2**20:.2f} MiB |",
              f"| compulsory (H 64 MiB + E 8 MiB + targets 256 KiB; nats + lse 512 KiB) | 72.25 MiB read, 0.5 MiB written |"]
    mrows = _counter_rows(os.path.join(d, "mfma"))
    if mrows:
        busy, _ = _per_dispatch(mrows, FWD_KERNEL, "SQ_VALU_MFMA_BUSY_CYCLES", True)
        gui, _ = _per_dispatch(mrows, FWD_KERNEL, "GRBM_GUI_ACTIVE", True)
        mops, _ = _per_dispatch(mrows, FWD_KERNEL, "SQ_INSTS_VALU_MFMA_MOPS_BF16", True)
        valu, _ = _per_dispatch(mrows, FWD_KERNEL, "SQ_INSTS_VALU", True)
        lds, _ = _per_dispatch(mrows, FWD_KERNEL, "SQ_INSTS_LDS", True)
        conf, _ = _per_dispatch(mrows, FWD_KERNEL, "SQ_LDS_BANK_CONFLICT", True)
        if busy and gui:
            # GRBM_GUI_ACTIVE comes back summed over the 8 XCDs; per XCD it is the kernel's cycles
            cyc = gui / 8.0
            keep = _long_dispatches(mrows, lambda r: FWD_KERNEL in r["Kernel_Name"])
            durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in mrows
                    if r["Dispatch_Id"] in keep and r["Counter_Name"] == "GRBM_GUI_ACTIVE"]
            dur_ns = sum(durs) / len(durs)
            out["mfma_busy_pct"] = 100.0 * busy / (cyc * 1024)
            out["clock_ghz"] = cyc / dur_ns
            lines.append(f"| MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) | "
                         f"{out['mfma_busy_pct']:.1f} % |")
            lines.append(f"| mean shader clock during the launch (GRBM_GUI_ACTIVE / 8 / duration) | "
                         f"{out['clock_ghz']:.2f} GHz over {dur_ns / 1e3:.1f} us |")
        if mops:
            out["mfma_flop"] = mops * 512
            lines.append(f"| bf16 MFMA FLOP (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) | {mops * 512:.4g} "
                         f"(algorithmic 2TDV = {2.0 * 65536 * 512 * 8192:.4g}) |")
        for nm, v in (("SQ_INSTS_VALU", valu), ("SQ_INSTS_LDS", lds), ("SQ_LDS_BANK_CONFLICT", conf)):
            if v is not None:
                out[nm] = v
                lines.append(f"| {nm} per launch | {v:.4g} |")
    trows = _counter_rows(os.path.join(d, "tcc"))
    if trows:
        hit, _ = _per_dispatch(trows, FWD_KERNEL, "TCC_HIT_sum", True)
        miss, _ = _per_dispatch(trows, FWD_KERNEL, "TCC_MISS_sum", True)
        if hit is not None and miss is not None and hit + miss > 0:
            out["l2_hit_pct"] = 100.0 * hit / (hit + miss)
            lines.append(f"| L2 hits / (hits + misses), TCC_HIT_sum and TCC_MISS_sum | {out['l2_hit_pct']:.1f} % "
                         f"({hit:.4g} hits, {miss:.4g} misses) |")
    # HBM traffic of every kernel of the training step (and the rest of the benchmark), same scales
    tf, tw = _counter_rows(os.path.join(d, "train_fetch")), _counter_rows(os.path.join(d, "train_write"))
    train_lines = []
    if tf and tw:
        names = sorted({r["Kernel_Name"] for r in tf if r["Kernel_Name"].startswith("void pg::") or
                        r["Kernel_Name"].startswith("pg::")})
        train_lines = ["", "HBM traffic per launch of each library kernel in the benchmark run with the training "
                           "step (without the sliding-window leg), at each kernel's largest grid (the T = 65536 "
                           "workloads; of those, the launches at least half as long as the longest, so that masked "
                           "batches of the same grid do not mix in): FETCH_SIZE x fetch scale, WRITE_SIZE x write "
                           "scale, MiB.", "",
                       "| kernel | grid (work-items) | launches | fetched | written |", "|---|---|---|---|---|"]

        def at_grid(rows, nm, counter, grid):
            keep = _long_dispatches(rows, lambda r: r["Kernel_Name"] == nm and int(r["Grid_Size"]) == grid)
            per = {}
            for r in rows:
                if r["Dispatch_Id"] in keep and r["Counter_Name"] == counter:
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
            return (sum(per.values()) / len(per), len(per)) if per else (None, 0)

        for nm in names:
            short = nm.split("(")[0].replace("void ", "")
            grid = max(int(r["Grid_Size"]) for r in tf if r["Kernel_Name"] == nm)
            fv, n = at_grid(tf, nm, "FETCH_SIZE", grid)
            wv, _ = at_grid(tw, nm, "WRITE_SIZE", grid)
            if fv is None or wv is None:
                continue
            train_lines.append(f"| `{short}` | {grid} | {n} | {fv * 1024.0 * kf / 2**20:.1f} | "
                               f"{wv * 1024.0 * kw / 2**20:.1f} |")
    lines += train_lines
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    md = TRAFFIC_FILE.replace("_traffic.json", "_counters.md")
    lines += ["", "Commands (from the repository root, cd /tmp first as rocprofv3 wants a writable cwd):", "",
              "```",
              "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -- python3 bench.py --steps 3 --warmup 1 --no-train --no-cpu",
              "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -- python3 bench.py --steps 3 --warmup 1 --no-train --no-cpu",
              "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/calib_fetch -- python3 bench.py --calibrate-copy",
              "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/calib_write -- python3 bench.py --calibrate-copy",
              "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU "
              "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT --output-format csv -d <dir>/mfma -- python3 bench.py --steps 3 --warmup 1 --no-train --no-cpu",
              "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d <dir>/tcc -- python3 bench.py --steps 3 --warmup 1 --no-train --no-cpu",
              "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/train_fetch -- python3 bench.py --steps 3 --warmup 1 --no-cpu --no-window",
              "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/train_write -- python3 bench.py --steps 3 --warmup 1 --no-cpu --no-window",
              "python3 bench.py --summarize-counters <dir>",
              "```", ""]
    with open(md, "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(out))


def _oracle_pass(inp, rows, train: bool, chunk: int = 1024, fn=None):
    """The float64 oracle over the given rows of a workload once, in row chunks run concurrently
    on all of the host's cores: each worker thread calls the unchanged oracle on its chunks with one
    BLAS thread (numpy releases the GIL in the matmul and the elementwise steps). train adds the
    oracle's backward (g = 1 / rows) after the forward of each chunk; fn(H, y), when given, replaces
    both (another oracle entry on the chunk). Returns (rows, seconds, worker threads)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as ora
    from lm_head_cross_pg_amd import synth
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    E = synth.as_f64(inp["embed"], inp["dtype"])
    c = inp["softcap"]
    rows = np.asarray(rows)
    g = 1.0 / max(len(rows), 1)

    def work(r0):
        r = rows[r0:r0 + chunk]
        H = synth.as_f64(inp["hidden"][r], inp["dtype"])
        y = inp["target"][r]
        if fn is not None:
            fn(H, y)
            return len(r)
        ora.forward(H, E, y, c)
        if train:
            ora.backward(H, E, y, c, g)
        return len(r)

    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        one_blas_thread = threadpool_limits(limits=1)
    except Exception:
        one_blas_thread = contextlib.nullcontext()
    with one_blas_thread:
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=cores) as ex:
            done = sum(ex.map(work, range(0, len(rows), chunk)))
        dt = time.perf_counter() - t0
    return done, dt, cores


def cpu_baseline(inp, train: bool = False, fn=None, what=None):
    """The oracle's forward (or forward + backward, or fn) over every row of the workload once."""
    rows, dt, cores = _oracle_pass(inp, np.arange(inp["T"]), train, fn=fn)
    what = what or ("forward + backward" if train else "forward")
    return {"value": rows / dt, "unit": "scored tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full {what}: all {rows} rows of the same workload once, 1024-row chunks on {cores} "
                      f"worker threads (one per host core, one BLAS thread each), float64 numpy "
                      f"(matmul, tanh, exp, log), {dt:.1f} s wall"}


def other_configs(abi, synth, args):
    """Forward + bits per byte on the smaller workloads, each as its own step: the tiny fp32 shape,
    the baseline vocabulary (T = 8192, V = 1024) and the stride-64 masked evaluation (2048 scored
    rows of 65536). Mean step time over --steps back-to-back steps after --warmup, and the mean of
    HIP-event-timed single steps."""
    import torch
    res = {}
    for name in ("tiny_f32", "fwd_v1024", "masked_stride64"):
        inp = synth.make_inputs(name, args.seed)
        T, D, V, c = inp["T"], inp["D"], inp["V"], inp["softcap"]
        d = abi.to_device(inp)
        nats = torch.empty(T, dtype=torch.float32, device="cuda")
        out = torch.empty(4, dtype=torch.float64, device="cuda")
        ws_f = torch.empty(abi.workspace_bytes(abi.PG_OP_FWD, T, D, V), dtype=torch.uint8, device="cuda")
        ws_b = torch.empty(abi.workspace_bytes(abi.PG_OP_BPB, T, D, V), dtype=torch.uint8, device="cuda")

        def step():
            abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], d["mask"], c, nats, None, ws_f)
            abi.pg_bpb_reduce(nats, d["target"], d["mask"], d["byte_len"], None, V, out, ws_b)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        ev_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        n_scored = int(out[2].item())
        flop = 2.0 * n_scored * D * V
        res[name] = {"T": T, "D": D, "V": V, "dtype": inp["dtype"], "scored_rows": n_scored,
                     "ms_per_step": wall * 1e3, "event_ms_per_step": ev_ms,
                     "scored_tokens_per_s": n_scored / wall,
                     "frac_bf16_peak": flop / wall / 1e12 / PEAK_BF16_TFLOPS, "bpb": float(out[3].item())}
        if not args.no_cpu:
            # the oracle beside it: its forward over the scored rows (the definition's loop), the
            # median of 5 passes
            rows = np.arange(T) if inp["mask"] is None else np.nonzero(inp["mask"])[0]
            passes = [_oracle_pass(inp, rows, False) for _ in range(5)]
            dt = float(np.median([p[1] for p in passes]))
            res[name]["cpu_baseline"] = {
                "value": len(rows) / dt, "unit": "scored tokens/s", "cores": passes[0][2], "kind": "oracle",
                "sample": f"the forward over the {len(rows)} scored rows, median of 5 passes on "
                          f"{passes[0][2]} worker threads, float64 numpy, {dt * 1e3:.1f} ms per pass"}
    print(json.dumps({"other_configs": res, "steps": args.steps, "warmup": args.warmup}), flush=True)


PMC_SET = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU SQ_INSTS_LDS "
           "SQ_LDS_BANK_CONFLICT")


def _pmc_kernel_table(d):
    """Markdown rows: per MFMA kernel of the counter run under d, the mean over its launches of the
    duration, MFMA busy, clock, bf16 MFMA FLOP, fraction of the dense bf16 peak, VALU and LDS
    instructions and LDS bank conflicts."""
    import collections
    rows = _counter_rows(d)
    # one group per kernel and launch size (bf16 MFMA operations per launch), so that the smaller
    # launches of other workloads do not mix into the main shape's figures
    byd = collections.defaultdict(dict)
    for r in rows:
        byd[r["Dispatch_Id"]][r["Counter_Name"]] = byd[r["Dispatch_Id"]].get(r["Counter_Name"], 0.0) + float(
            r["Counter_Value"])
        byd[r["Dispatch_Id"]]["_name"] = r["Kernel_Name"]
        byd[r["Dispatch_Id"]]["_dur"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for v in byd.values():
        k = (v["_name"], round(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) / 1e6))
        for c, x in v.items():
            if not c.startswith("_"):
                per[k][c].append(x)
        dur[k].append(v["_dur"])
    out = ["Per kernel, the mean over its launches. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 "
           "XCDs x 1024 SIMDs);",
           "clock = GRBM_GUI_ACTIVE / 8 / duration; MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; frac = MFMA FLOP "
           "/ duration / 2516.6 TFLOP/s.", "",
           "| kernel | launches | duration us | MFMA busy | clock GHz | MFMA FLOP | frac | VALU instr | LDS instr | "
           "LDS bank conflicts |",
           "|---|---|---|---|---|---|---|---|---|---|"]

    def mean(v):
        return sum(v) / len(v) if v else float("nan")
    for k in sorted(per, key=lambda k: -mean(dur[k])):
        mops = mean(per[k]["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
        if not mops > 0:
            continue
        dk, cyc = mean(dur[k]), mean(per[k]["GRBM_GUI_ACTIVE"]) / 8.0
        busy = mean(per[k]["SQ_VALU_MFMA_BUSY_CYCLES"])
        nm = k[0].split("(")[0].replace("void ", "").replace("pg::", "")[:90]
        frac = mops * 512 / (dk * 1e-9) / 1e12 / PEAK_BF16_TFLOPS
        out.append(f"| `{nm}` | {len(dur[k])} | {dk / 1e3:.0f} | {100 * busy / (cyc * 1024):.1f} % | {cyc / dk:.2f} | "
                   f"{mops * 512:.3g} | {frac:.3f} | {mean(per[k]['SQ_INSTS_VALU']):.3g} | "
                   f"{mean(per[k]['SQ_INSTS_LDS']):.3g} | {mean(per[k]['SQ_LDS_BANK_CONFLICT']):.0f} |")
    return out


def summarize_library(d):
    """profiles/library_gemm_counters.md from a counter run of `bench.py --library-gemm`: what the
    vendor GEMM reaches on this chip (a random bf16 8192^3 product and the head's shapes)."""
    lines = ["# The vendor GEMM under the same counters (random bf16 operands)", "",
             "`torch.mm` on hipBLASLt: a square 8192^3 product (bf16 out) and the head's three product shapes at",
             "T = 65536, D = 512, V = 8192. Context for the fused kernels: the square product shows the MFMA",
             "rate and clock this chip sustains on a large plain GEMM of random data.", "",
             "From `rocprofv3 --pmc " + PMC_SET + " --output-format csv -d <dir> -- python3 $R/bench.py "
             "--library-gemm --steps 5` (cd /tmp first; R = repository root), summarised by "
             "`python3 bench.py --summarize-library <dir>`.", ""] + _pmc_kernel_table(d)
    out = os.path.join(ROOT, "profiles", "library_gemm_counters.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def summarize_trace(d, steps, warmup):
    """profiles/kernels_fwd_bwd_T65536_D512_V8192.md from a profiling directory: per-kernel trace
    statistics (d/trace, from `rocprofv3 --kernel-trace --stats ... -- python3 bench.py --no-cpu`),
    the forward's launches in the sustained loop and the isolated ones, and per-kernel counters of
    the training step (d/cnt/train_mfma)."""
    import csv
    stats = list(csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))))
    main_kernel = "void pg::" + FWD_KERNEL + ">"
    lines = ["# Kernel time, bench step + training step (T=65536, D=512, V=8192, bf16, softcap 30)", "",
             "rocprofv3 `--kernel-trace --stats` of the benchmark: per kernel, the number of launches and the",
             f"average / min / max duration. The main forward (`{FWD_KERNEL}>`) runs in the",
             "bench steps, the event-timed launches, the quantised-head launches and the training steps; the",
             "asymmetric-cap forward (`<512, true, 1, true, false, false>`) is a kernel of its own, and so is the",
             "forward on the int8 head (`<512, true, 1, false, false, true>`, masked and small calls); the",
             "dZ-writing forwards (`..., false, true, false>`, and `..., true, true, false>` for asymmetric caps)",
             "and the backward kernels run once per training step. The kernels run back to back, so the clock",
             "falls under the sustained load: compare the min column with isolated launches.", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:72]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    # bench.py's order: untimed forwards while the clock settles, --steps isolated forwards back to
    # back, then the warmup and timed steps of the sustained loop (each forward followed by the two
    # bits-per-byte kernels). A main-forward launch followed by the reduction belongs to the loop;
    # the isolated leg is the --steps forwards just before the loop's first one.
    tr = sorted(csv.DictReader(open(os.path.join(d, "trace", "run_kernel_trace.csv"))),
                key=lambda r: int(r["Start_Timestamp"]))
    fwds = []                 # (duration us, followed by the reduction)
    for i, r in enumerate(tr):
        if not r["Kernel_Name"].startswith(main_kernel):
            continue
        nxt = tr[i + 1]["Kernel_Name"] if i + 1 < len(tr) else ""
        fwds.append(((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, "bpb_partial_kernel" in nxt))
    first = next((k for k, (_, in_loop) in enumerate(fwds) if in_loop), len(fwds))
    sustained = [dt for dt, in_loop in fwds if in_loop]
    isolated = [dt for dt, _ in fwds[max(0, first - steps):first]]
    timed = sustained[warmup:warmup + steps]
    flop = 2.0 * 65536 * 512 * 8192
    if isolated:
        m = sum(isolated) / len(isolated)
        lines += ["", f"The {len(isolated)} isolated forwards (back to back, events between them, after untimed ones "
                      "that let the clock settle): mean",
                  f"{m:.1f} us (min {min(isolated):.1f}, max {max(isolated):.1f}), frac "
                  f"{flop / (m * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.3f}."]
    if timed:
        m = sum(timed) / len(timed)
        lines += ["", f"The `roofline` figure of `bench.py` is the forward's own time inside its sustained loop: the "
                      f"{len(timed)} timed forwards", f"(after {warmup} warmup steps), each "
                      "followed by the bits-per-byte reduction, in this trace taken on the benchmark's command:",
                  f"mean {m:.1f} us (min {min(timed):.1f}, max {max(timed):.1f}): "
                  f"{flop / (m * 1e-6) / 1e12:.0f} TFLOP/s, frac {flop / (m * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.3f}."]
    lines += ["", "Commands (cd /tmp first; R = repository root; summarised by "
                  "`python3 bench.py --summarize-trace <dir>`):", "", "```",
              f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o run -- python3 $R/bench.py "
              f"--steps {steps} --warmup {warmup} --no-cpu",
              "```", ""]
    lines += ["## Counters per kernel (training step)", "",
              "From `rocprofv3 --pmc " + PMC_SET + " --output-format csv -d <dir>/cnt/train_mfma -- python3 "
              "$R/bench.py --steps 3 --warmup 1 --no-cpu`.", ""] + _pmc_kernel_table(os.path.join(d, "cnt", "train_mfma"))
    out = os.path.join(ROOT, "profiles", "kernels_fwd_bwd_T65536_D512_V8192.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def library_gemm(steps):
    """The vendor GEMM (torch.mm, hipBLASLt on this stack) on the products of the head at T = 65536,
    D = 512, V = 8192, bf16 in: the logits H E^T (written out, T x V bf16), dZ E (T x D) and
    dZ^T H (V x D), with float32 outputs where torch offers them. Context for the fused kernels,
    which never write the logits; the medians of HIP-event-timed calls."""
    import torch
    T, D, V = 65536, 512, 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    H = torch.randn(T, D, device="cuda", generator=g).bfloat16()
    E = (torch.randn(V, D, device="cuda", generator=g) * 0.02).bfloat16()
    dZ = (torch.randn(T, V, device="cuda", generator=g) * 1e-3).bfloat16()
    Et = E.t().contiguous()

    def med_ms(f):
        for _ in range(5):
            f()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record()
            f()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    flop = 2.0 * T * D * V
    # a large square product: what the vendor GEMM reaches on this chip with random bf16 operands
    S = 8192
    A = torch.randn(S, S, device="cuda", generator=g).bfloat16()
    B = torch.randn(S, S, device="cuda", generator=g).bfloat16()
    sq = {"square 8192^3 (bf16 out)": lambda: torch.mm(A, B)}
    cases = {"logits H E^T (bf16 out)": lambda: torch.mm(H, Et),
             "dH = dZ E (bf16 out)": lambda: torch.mm(dZ, E),
             "dE = dZ^T H (bf16 out)": lambda: torch.mm(dZ.t(), H)}
    try:
        torch.mm(dZ, E, out_dtype=torch.float32)
        cases["dH = dZ E (f32 out)"] = lambda: torch.mm(dZ, E, out_dtype=torch.float32)
        cases["dE = dZ^T H (f32 out)"] = lambda: torch.mm(dZ.t(), H, out_dtype=torch.float32)
    except (TypeError, RuntimeError):
        pass
    res = {}
    for k, f in sq.items():
        ms = med_ms(f)
        fl = 2.0 * S ** 3
        res[k] = {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    for k, f in cases.items():
        ms = med_ms(f)
        res[k] = {"ms": ms, "tflops": flop / (ms * 1e-3) / 1e12, "frac": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    print(json.dumps({"library_gemm": res, "T": T, "D": D, "V": V, "calls": steps}), flush=True)


def window_eval(abi, synth, args):
    """The sliding-window evaluation driver on a stream of 2048 + 95 x 64 + 1 tokens: 96 windows of
    2048 at stride 64 in 3 batches of 32 windows (65,536 rows each; 8128 predictions scored), D = 512,
    V = 8192, with and without one score-first SGD step per batch, and on the int8 head (evaluation
    only). The hidden states of the scored rows are drawn once and kept on the device; a pass is the
    driver's steps over the 3 batches."""
    import torch
    from lm_head_cross_pg_amd.window_eval import SlidingWindowEval
    n_tokens, L, s, B, D, V = 2048 + 95 * 64 + 1, 2048, 64, 32, 512, 8192
    st = synth.make_stream(args.seed, n_tokens, V, D=D)
    tokens = torch.from_numpy(st["tokens"]).cuda()
    blen = torch.from_numpy(st["byte_len"]).cuda()
    res = {}
    E0 = torch.from_numpy(st["embed"].view(np.int16)).cuda().view(torch.bfloat16)
    q8 = torch.empty((V, D), dtype=torch.int8, device="cuda")
    sc8 = torch.empty(V, dtype=torch.float32, device="cuda")
    abi.pg_quantize_q8(E0, q8, sc8)
    for lr, int8 in ((0.0, False), (2.0, False), (0.0, True)):
        E16 = E0.clone()
        master = E0.float() if lr else None
        drv = SlidingWindowEval(tokens, blen, V, D, L, s, B, 30.0, ttt_lr=lr, embed_master=master, int8_head=int8)
        hid = []
        for w0, nw in drv.batches():
            H = torch.zeros((nw * L, D), dtype=torch.bfloat16, device="cuda")
            for b in range(nw):
                w = w0 + b
                lo = 0 if w == 0 else L - s
                n = drv.scored(w, 1)
                H[b * L + lo: b * L + lo + n] = torch.from_numpy(
                    synth.window_hidden(args.seed, w, n, D).view(np.int16)).cuda().view(torch.bfloat16)
            hid.append(H)
        passes = 5
        times = []
        for it in range(passes + 1):
            drv.out.zero_()
            E16.copy_(E0)                            # every pass starts from the same embedding
            if master is not None:
                master.copy_(E0.float())
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if int8:
                n = sum(drv.step_int8(H, q8, sc8, w0, nw) for H, (w0, nw) in zip(hid, drv.batches()))
            else:
                n = sum(drv.step(H, E16, w0, nw) for H, (w0, nw) in zip(hid, drv.batches()))
            b.record()
            torch.cuda.synchronize()
            if it:                                   # the first pass is a warmup
                times.append(a.elapsed_time(b))
        ms = float(np.median(times))
        # per scored row: the forward, and with training the embedding's gradient dE (the driver takes
        # no gradient of the hidden states, so that product does not run and is not counted)
        flop = (4.0 if lr else 2.0) * n * D * V
        entry = {"ms_per_pass": ms, "predictions": n, "scored_tokens_per_s": n / (ms * 1e-3),
                 "frac_bf16_peak": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "frac_counted_as": "4 T_s D V (forward + dE)" if lr else "2 T_s D V (forward)",
                 "bpb": drv.result()[3]}
        if not args.no_cpu:
            # the oracle's own sliding-window loop on the same stream, hidden states and steps
            from oracle import oracle as ora
            try:
                cores = len(os.sched_getaffinity(0))
            except AttributeError:
                cores = os.cpu_count() or 1
            E_ref = synth.bf16_to_f64(st["embed"])
            if int8:   # the head the int8 form scores: the dequantised embedding
                E_ref = ora.dequantize_rows_q8(*ora.quantize_rows_q8(E_ref))
            t0 = time.perf_counter()
            ref = ora.sliding_window_eval(st["tokens"], st["byte_len"],
                                          lambda w, k: synth.bf16_to_f64(synth.window_hidden(args.seed, w, k, D)),
                                          E_ref, 30.0, L, s, B, lr=lr)
            dt = time.perf_counter() - t0
            entry["bpb_oracle"] = ref["bpb"]
            entry["cpu_baseline"] = {
                "value": ref["n_scored"] / dt, "unit": "scored tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"the oracle's sliding-window loop over the same {ref['n_scored']} predictions "
                          f"(3 batches{', each with its backward and SGD step' if lr else ''}), float64 numpy "
                          f"(BLAS on every core, the elementwise steps on one thread), {dt:.1f} s wall"}
        res["int8_head" if int8 else "ttt_lr_%g" % lr] = entry
    res["workload"] = "stream of %d tokens, windows of %d at stride %d, %d windows per batch, D=%d, V=%d" % (
        n_tokens, L, s, B, D, V)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-window", action="store_true",
                    help="leave out the sliding-window driver leg (for counter runs of the training step)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB scratch tensor between timed forward launches (cold L2/MALL)")
    ap.add_argument("--other-configs", action="store_true",
                    help="only time forward + bits per byte on the smaller workloads (their own JSON line)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor GEMM (torch.mm on hipBLASLt) on the head's three product shapes")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="summarise a rocprofv3 kernel trace (DIR/trace) and the training counter run "
                         "(DIR/cnt/train_mfma) into profiles/ and exit")
    ap.add_argument("--summarize-library", metavar="DIR",
                    help="summarise a rocprofv3 counter run of --library-gemm into profiles/ and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="summarise rocprofv3 counter runs under DIR into profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_library:
        summarize_library(args.summarize_library)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps, args.warmup)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the data-parallel head needs no exchange until the "
              "final three-scalar sum, and this benchmark measures a single MI355X (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 27, dtype=torch.float32, device="cuda")   # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": 5}))
        return
    if args.library_gemm:
        library_gemm(args.steps)
        return
    from lm_head_cross_pg_amd import abi, build, synth
    if not os.path.exists(abi.LIB_PATH):
        build.build()
    abi.load()
    if args.other_configs:
        other_configs(abi, synth, args)
        return

    inp = synth.make_inputs("fwd_v8192", args.seed)
    T, D, V, c = inp["T"], inp["D"], inp["V"], inp["softcap"]
    d = abi.to_device(inp)
    nats = torch.empty(T, dtype=torch.float32, device="cuda")
    lse = torch.empty(T, dtype=torch.float32, device="cuda")
    out = torch.empty(4, dtype=torch.float64, device="cuda")
    ws_fwd = torch.empty(abi.workspace_bytes(abi.PG_OP_FWD, T, D, V), dtype=torch.uint8, device="cuda")
    ws_bpb = torch.empty(abi.workspace_bytes(abi.PG_OP_BPB, T, D, V), dtype=torch.uint8, device="cuda")

    def step():
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, c, nats, lse, ws_fwd)
        abi.pg_bpb_reduce(nats, d["target"], None, d["byte_len"], None, V, out, ws_bpb)

    # the GPU's power management takes 10-20 ms of load to settle (launches run up to 20 % slower on
    # the way): untimed forwards first, so that both timed legs below see the settled clock
    for _ in range(max(30, args.warmup)):
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, c, nats, lse, ws_fwd)
    torch.cuda.synchronize()
    # the forward alone, launches back to back with events between them (the isolated figure)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if args.cold else None
    for a, b in ev:
        if scratch is not None:
            scratch.fill_(1.0)
        a.record()
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, c, nats, lse, ws_fwd)
        b.record()
    torch.cuda.synchronize()
    launch = np.array([a.elapsed_time(b) for a, b in ev])
    iso_ms = float(np.mean(launch))
    # the sustained loop: steps back to back; HIP events on the library's stream (torch's current
    # stream, which the binding passes) bracket each forward inside it, so the roofline figure is
    # the forward's own time within the timed region
    ev_s = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev_s:
        a.record()
        abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], None, c, nats, lse, ws_fwd)
        b.record()
        abi.pg_bpb_reduce(nats, d["target"], None, d["byte_len"], None, V, out, ws_bpb)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    bpb = out.cpu().numpy().tolist()
    sustained = np.array([a.elapsed_time(b) for a, b in ev_s])
    fwd_ms = float(np.mean(sustained))
    flop_fwd = 2.0 * T * D * V
    achieved = flop_fwd / (fwd_ms * 1e-3) / 1e12


    ms_per_step = wall / args.steps * 1e3
    result = {
        "metric": "scored tokens/s fused LM-head+softcap CE->BPB (D=512,V=8192); % bf16 MFMA peak",
        "value": T * args.steps / wall,
        "unit": "scored tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; unit-RMS hidden, N(0,0.02^2) tied embedding, Zipf(1.1) targets)",
        "config": {"workload": "fwd_v8192: T=65536 (32 x 2048), D=512, V=8192, bf16, softcap 30, all rows scored; "
                               "step = fused forward + bits-per-byte reduction",
                   "T": T, "D": D, "V": V, "softcap": c, "seed": args.seed},
        "pct_bf16_mfma_peak_step": 100.0 * flop_fwd / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "bpb": bpb[3],
        "roofline": {"bound": "mfma", "kernel": FWD_KERNEL + ">", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(),
                     "launch_ms": fwd_ms,
                     "launch_ms_p10_p50_p90": [float(np.percentile(sustained, q)) for q in (10, 50, 90)],
                     "timed_in": "the sustained forward + BPB loop (events around each forward)",
                     "isolated_launch_ms": iso_ms,
                     "isolated_frac": flop_fwd / (iso_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "isolated_launch_ms_p10_p50_p90": [float(np.percentile(launch, q)) for q in (10, 50, 90)],
                     "l2_mall": "cold (1 GiB written between isolated launches)" if args.cold else "warm",
                     "algorithmic": "2*T*D*V = %.4g FLOP per launch" % flop_fwd},
    }

    # the bits-per-byte reduction alone (reads nats, target and the byte length of each target)
    ev_b = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev_b:
        a.record()
        abi.pg_bpb_reduce(nats, d["target"], None, d["byte_len"], None, V, out, ws_bpb)
        b.record()
    torch.cuda.synchronize()
    bpb_launch = np.array([a.elapsed_time(b) for a, b in ev_b]) * 1e3
    result["bpb_reduce"] = {
        "launch_us": float(np.mean(bpb_launch)),
        "launch_us_p10_p50_p90": [float(np.percentile(bpb_launch, q)) for q in (10, 50, 90)],
        "bytes": T * 12,
        "note": "two launches (per-workgroup partials, fixed-order final); 12 B per row: nats, target, byte length"}

    # the asymmetric softcap (separate caps for z >= 0 and z < 0) on the same workload
    caps = (30.0, 20.0)
    for _ in range(3):
        abi.pg_lmhead_ce_fwd_asym(d["hidden"], d["embed"], d["target"], None, caps[0], caps[1], nats, lse, ws_fwd)
    ev_a = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev_a:
        a.record()
        abi.pg_lmhead_ce_fwd_asym(d["hidden"], d["embed"], d["target"], None, caps[0], caps[1], nats, lse, ws_fwd)
        b.record()
    torch.cuda.synchronize()
    asym_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_a]))
    abi.pg_bpb_reduce(nats, d["target"], None, d["byte_len"], None, V, out, ws_bpb)
    result["asym_softcap"] = {
        "caps": list(caps), "launch_ms": asym_ms, "tokens_per_s": T / (asym_ms * 1e-3),
        "achieved_tflops": flop_fwd / (asym_ms * 1e-3) / 1e12,
        "frac": flop_fwd / (asym_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "bpb": float(out[3].item()),
        "note": "fused forward with separate caps for z >= 0 and z < 0 (each side's tanh series below min(caps)/8, exact softcap above)"}
    if not args.no_cpu:
        from oracle import oracle as ora
        E64 = synth.as_f64(inp["embed"], inp["dtype"])
        result["asym_softcap"]["cpu_baseline"] = cpu_baseline(
            inp, fn=lambda H, y: ora.forward(H, E64, y, caps), what="forward with caps (30, 20)")

    # the same head on logits of a trained model's magnitude: hidden x 8 (exact in bf16) gives z with
    # standard deviation ~3.6, so almost every 32 x 32 block has some |z| > c/8 and the epilogue
    # takes the exact softcap (exp2, fma, rcp, exp2 per logit) instead of the series
    hid8 = d["hidden"] * 8
    for _ in range(3):
        abi.pg_lmhead_ce_fwd(hid8, d["embed"], d["target"], None, c, nats, lse, ws_fwd)
    ev_l = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev_l:
        a.record()
        abi.pg_lmhead_ce_fwd(hid8, d["embed"], d["target"], None, c, nats, lse, ws_fwd)
        b.record()
    torch.cuda.synchronize()
    big_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_l]))
    abi.pg_bpb_reduce(nats, d["target"], None, d["byte_len"], None, V, out, ws_bpb)
    result["large_logits"] = {
        "hidden_scale": 8, "launch_ms": big_ms, "tokens_per_s": T / (big_ms * 1e-3),
        "frac": flop_fwd / (big_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "bpb": float(out[3].item()),
        "note": "same forward, hidden x 8 (z std ~3.6): the epilogue takes the exact softcap in almost every block"}
    del hid8

    # the quantised tied head: per-row int8 embedding (quantised once), scored through the fused path
    q8 = torch.empty((V, D), dtype=torch.int8, device="cuda")
    sc8 = torch.empty(V, dtype=torch.float32, device="cuda")
    ws_q8 = torch.empty(abi.workspace_bytes(abi.PG_OP_FWD_Q8, T, D, V), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        abi.pg_quantize_q8(d["embed"], q8, sc8)
        abi.pg_lmhead_ce_fwd_q8(d["hidden"], q8, sc8, d["target"], None, c, nats, lse, ws_q8)
    ev_q = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ev_q:
        a.record()
        abi.pg_quantize_q8(d["embed"], q8, sc8)
        b.record()
    # int8 and bf16 launches alternate, so that both see the same clock
    def q8_ab(mask_t, n):
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
              for _ in range(2)]
        for i in range(n):
            ev[0][i][0].record()
            abi.pg_lmhead_ce_fwd_q8(d["hidden"], q8, sc8, d["target"], mask_t, c, nats, lse, ws_q8)
            ev[0][i][1].record()
            ev[1][i][0].record()
            abi.pg_lmhead_ce_fwd(d["hidden"], d["embed"], d["target"], mask_t, c, nats, lse, ws_fwd)
            ev[1][i][1].record()
        torch.cuda.synchronize()
        return [float(np.mean([a.elapsed_time(b) for a, b in e])) for e in ev]
    q8_ms, bf16_ms = q8_ab(None, args.steps)
    torch.cuda.synchronize()
    quant_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_q]))
    abi.pg_lmhead_ce_fwd_q8(d["hidden"], q8, sc8, d["target"], None, c, nats, lse, ws_q8)
    abi.pg_bpb_reduce(nats, d["target"], None, d["byte_len"], None, V, out, ws_bpb)
    bpb_q8 = float(out[3].item())
    # the stride-64 evaluation's mask (the last 64 rows of each 2048 scored): few row tiles, so the
    # head's bytes weigh more
    m64 = torch.zeros(T, dtype=torch.uint8, device="cuda")
    m64.view(-1, 2048)[:, -64:] = 1
    q8_m_ms, bf16_m_ms = q8_ab(m64, max(args.steps, 20))
    quant_bytes = V * D * 2 + V * D + V * 4          # read bf16 E, write int8 q and float32 scales
    result["q8_head"] = {
        "format": "per-row symmetric int8, float32 scales; head computes on bf16(q * scale)",
        "quantize_us": quant_ms * 1e3, "quantize_gbps": quant_bytes / (quant_ms * 1e-3) / 1e9,
        "launch_ms": q8_ms, "tokens_per_s": T / (q8_ms * 1e-3),
        "frac": flop_fwd / (q8_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "bpb": bpb_q8,
        "bf16_launch_ms": bf16_ms,
        "stride64_mask": {"scored": int(m64.sum().item()), "launch_ms": q8_m_ms, "bf16_launch_ms": bf16_m_ms},
        "note": "all rows (launch_ms): the bf16 head is written first (one pass), then the bf16 forward; "
                "with the stride-64 mask the forward reads the int8 rows and converts each tile on chip; "
                "bf16_launch_ms: the bf16 head's forward, launches alternating with the int8 ones"}
    if not args.no_cpu:
        from oracle import oracle as ora
        q_o, s_o = ora.quantize_rows_q8(synth.as_f64(inp["embed"], inp["dtype"]))
        result["q8_head"]["cpu_baseline"] = cpu_baseline(
            inp, fn=lambda H, y: ora.forward_q8(H, q_o, s_o, y, c), what="forward on the int8 head")

    if not args.no_train:
        tin = synth.make_inputs("train_v8192", args.seed)
        td = abi.to_device(tin)
        dH = torch.empty((T, D), dtype=torch.float32, device="cuda")
        dE = torch.empty((V, D), dtype=torch.float32, device="cuda")
        ws_bwd = torch.empty(abi.workspace_bytes(abi.PG_OP_BWD, T, D, V), dtype=torch.uint8, device="cuda")
        tl = torch.empty(T, dtype=torch.float32, device="cuda")

        ws_fb = torch.empty(abi.workspace_bytes(abi.PG_OP_FWD_BWD, T, D, V), dtype=torch.uint8, device="cuda")

        def train_step(hid):          # one call: the logits are computed once
            abi.pg_lmhead_ce_fwd_bwd(hid, td["embed"], td["target"], None, c, 1.0 / T, nats, tl, dH, dE, ws_fb)

        def train_step_two_calls(hid):   # forward, then the backward that recomputes the logits
            abi.pg_lmhead_ce_fwd(hid, td["embed"], td["target"], None, c, nats, tl, ws_fwd)
            abi.pg_lmhead_ce_bwd(hid, td["embed"], td["target"], None, tl, c, 1.0 / T, dH, dE, ws_bwd)

        caps = (30.0, 20.0)

        def train_step_asym(hid):     # asymmetric caps, one call
            abi.pg_lmhead_ce_fwd_bwd_asym(hid, td["embed"], td["target"], None, caps[0], caps[1], 1.0 / T, nats, tl,
                                          dH, dE, ws_fb)

        def time_train(step, hid, ksteps):
            """ksteps training steps back to back after a warmup, HIP events around each: the
            per-step times (ms) and the wall time per step."""
            for _ in range(max(5, args.warmup // 2)):
                step(hid)
            ev_t = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ksteps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for a, b in ev_t:
                a.record()
                step(hid)
                b.record()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / ksteps
            return np.array([a.elapsed_time(b) for a, b in ev_t]), wall

        hid8 = td["hidden"] * 8                     # logits of trained-model size, as for the forward
        ksteps = max(40, args.steps)
        per = {}
        for key, step, hid, k in (("one", train_step, td["hidden"], ksteps),
                                  ("two", train_step_two_calls, td["hidden"], 20),
                                  ("one8", train_step, hid8, 20), ("two8", train_step_two_calls, hid8, 20),
                                  ("asym", train_step_asym, td["hidden"], 20)):
            per[key] = time_train(step, hid, k)
        del hid8
        ms, wall = per["one"]
        med = float(np.median(ms))
        result["train_step"] = {
            "workload": "train_v8192: T=65536, D=512, V=8192, bf16 in, fp32 dH/dE, mean CE (g=1/T)",
            "entry": "pg_lmhead_ce_fwd_bwd",
            "ms_per_step": med, "ms_per_step_p10_p50_p90": [float(np.percentile(ms, q)) for q in (10, 50, 90)],
            "ms_per_step_wall_mean": wall * 1e3, "steps": ksteps,
            "tokens_per_s": T / (med * 1e-3),
            "pct_bf16_mfma_peak_counted": 100.0 * 6.0 * T * D * V / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "ms_per_step_large_logits": float(np.median(per["one8"][0])),
            "ms_per_step_two_calls": float(np.median(per["two"][0])),
            "ms_per_step_two_calls_large_logits": float(np.median(per["two8"][0])),
            "ms_per_step_asym_caps_30_20": float(np.median(per["asym"][0])),
            "note": "medians of HIP-event-timed steps run back to back (20 for the variants)",
        }

        if not args.no_cpu:
            result["train_step"]["cpu_baseline"] = cpu_baseline(tin, train=True)

    if not args.no_train and not args.no_window:
        result["window_eval"] = window_eval(abi, synth, args)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

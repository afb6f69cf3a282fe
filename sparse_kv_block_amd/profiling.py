"""Turns rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m sparse_kv_block_amd.profiling stats DIR --cmd "..." --out profiles/X.txt
    python -m sparse_kv_block_amd.profiling counters --fetch DIR1 --write DIR2 \
        --kernel layer_step_bf16 --copy-kernel elementwise --copy-bytes N \
        --cmd-fetch "..." --cmd-write "..." --out profiles/X.json
    python -m sparse_kv_block_amd.profiling per-kernel --fetch DIR1 --write DIR2 \
        --stats DIR3 --copy-kernel elementwise --copy-bytes N \
        --cmd-fetch "..." --cmd-write "..." --cmd-stats "..." --out profiles/X.md
    python -m sparse_kv_block_amd.profiling pipeline BENCH.json --cmd "..." --out profiles/X.md
    python -m sparse_kv_block_amd.profiling sq NAME=DIR ... --kernel layer_step --cmd "..." \
        --out profiles/X.md

`counters` scales the kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by
what the same counters read for a plain copy kernel of known size, and records
a hash of the HIP sources so that stale numbers can be recognised.
`per-kernel` does the same for every kernel of the library that the runs
launched and divides the bytes by the kernel's median duration from a
separate kernel-trace run (counter runs serialise dispatches, so their own
timestamps are not used), as a table of HBM GB/s per kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".h", ".hip")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[-1]


def _rows(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats(d: str, cmd: str, out: str, top: int = 12):
    rows = _rows(_find(d, "kernel_stats.csv"))
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}",
             f"# kernel sources: {kernel_source_hash()}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel"]
    for r in rows[:top]:
        name = r.get("Name") or r.get("KernelName") or "?"
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r.get('Percentage', 0)):8.2f}  {name[:110]}")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def _counter_per_dispatch(d: str, counter: str, substr: str):
    rows = _rows(_find(d, "counter_collection.csv"))
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter or substr not in r.get("Kernel_Name", ""):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for kernels matching {substr!r} in {d}")
    vals = list(per.values())
    return statistics.median(vals), len(vals)


def counters(fetch_dir, write_dir, kernel, copy_kernel, copy_bytes, cmd_fetch, cmd_write, out,
             algorithmic_bytes=None):
    f_k, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    f_c, _ = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", copy_kernel)
    w_k, nw = _counter_per_dispatch(write_dir, "WRITE_SIZE", kernel)
    w_c, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", copy_kernel)
    sf = copy_bytes / (f_c * 1024.0)
    sw = copy_bytes / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * sf
    write_b = w_k * 1024.0 * sw
    rec = {
        "kernel": kernel, "source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k, "dispatches": [nf, nw],
        "copy_kernel": copy_kernel, "copy_bytes": copy_bytes,
        "copy_fetch_kib": f_c, "copy_write_kib": w_c,
        "fetch_scale": sf, "write_scale": sw,
        "hbm_read_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "algorithmic_bytes_per_launch": algorithmic_bytes,
        "commands": [cmd_fetch, cmd_write],
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def _short(name: str) -> str:
    n = name.split("(")[0]
    return n[5:] if n.startswith("void ") else n


def per_kernel(fetch_dir, write_dir, stats_dir, copy_kernel, copy_bytes, cmds, out,
               match="oasis::", peak_gbs=8000.0):
    f_c, _ = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", copy_kernel)
    w_c, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", copy_kernel)
    sf = copy_bytes / (f_c * 1024.0)
    sw = copy_bytes / (w_c * 1024.0)
    names = sorted({r["Kernel_Name"] for r in _rows(_find(fetch_dir, "counter_collection.csv"))
                    if match in r["Kernel_Name"]})
    spans = {}
    for r in _rows(_find(stats_dir, "kernel_trace.csv")):
        spans.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# HBM traffic per kernel (rocprofv3 counters)", "",
             f"Kernel sources: {kernel_source_hash()}.",
             f"FETCH_SIZE x {sf:.4f} and WRITE_SIZE x {sw:.4f} give bytes: the factors make a "
             f"plain {copy_bytes} B copy kernel ({copy_kernel}) read and write {copy_bytes} B.",
             "Bytes: median over a kernel's dispatches in the counter runs. Durations: median "
             "over its dispatches in the kernel-trace run. GB/s = (read + write) / duration; "
             f"% of the {peak_gbs:.0f} GB/s HBM peak (the gather and append kernels move "
             "their bytes over the host link, not HBM).", "",
             "| kernel | dispatches | read MB | write MB | median us | GB/s | % peak |",
             "|---|---|---|---|---|---|---|"]
    for name in names:
        fk, nf = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", name)
        wk, _ = _counter_per_dispatch(write_dir, "WRITE_SIZE", name)
        rb, wb = fk * 1024.0 * sf, wk * 1024.0 * sw
        sp = spans.get(name)
        us = statistics.median(sp) if sp else float("nan")
        gbs = (rb + wb) / us / 1e3 if sp else float("nan")
        lines.append(f"| `{_short(name)}` | {nf} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {us:.1f} | "
                     f"{gbs:.0f} | {100 * gbs / peak_gbs:.0f} |")
    lines += ["", "Commands:", ""] + [f"    {c}" for c in cmds]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def pipeline(bench_json: str, cmd: str, out: str):
    """The 36-layer fetch-cap sweep and the host-link budget of one
    `bench.py --pipeline --capmodel` run, as a table."""
    with open(bench_json) as f:
        lines = [l for l in f if l.strip().startswith("{")]
    res = json.loads(lines[-1])
    pl, cmod, pcie = res["pipeline_36_layer"], res["cap_model"], res["pcie"]
    L = [f"# 36-layer decode step: fetch-cap sweep and host-link budget", "",
         f"Command (repository root, one MI355X): `{cmd}`", "",
         f"Kernel sources: {kernel_source_hash()}.  {pl['layers']} layers, batch {pl['batch']}, "
         f"context {pl['ctx']}, K = {pl['k_resident']}, {pl['host_pool']}; per layer the fused "
         "step on the main stream and the gather prefetch of its admissions on a side stream "
         "(layer-local events).  Bytes per step from the admission counts; the bound is "
         "layers x units x max_admit x record bytes.  Overlap fraction = (fused kernels alone + "
         "transfer alone - step) / the shorter of the two, the transfer alone being the bytes "
         "at the gather kernel's measured host-link rate.", "",
         "| cap | max_admit | bytes moved / step | bound | step ms | fused kernels alone ms | "
         "transfer alone ms | overlap fraction | host link GB/s |",
         "|---|---|---|---|---|---|---|---|---|"]
    for r in pl["caps"]:
        L.append(f"| {r['cap']} | {r['max_admit']} | {r['bytes_per_step'] / 1e9:.3f} GB | "
                 f"{r['bytes_bound'] / 1e9:.3f} GB | {r['step_ms']:.2f} | {r['compute_only_ms']:.2f} | "
                 f"{r.get('transfer_alone_ms', float('nan')):.2f} | "
                 f"{r.get('overlap_fraction', float('nan')):.2f} | {r['host_link_GBps']:.1f} |")
    lk = cmod["link_GBps"]
    L += ["", f"Host link: gather kernel {lk['gather_kernel']} GB/s "
              f"({pcie['gather']['bytes'] / 1e6:.1f} MB of one step's admissions), one contiguous "
              f"1 GiB SDMA copy from the pinned pool {lk['sdma_1GiB_copy']} GB/s.",
          "Fused step: " + ", ".join(f"K = {k}: {v} us" for k, v in cmod["fused_step_us"].items())
          + f" (window = {cmod['layers']} layers x fused step).", "",
          "| K | link | window ms | largest max_admit that hides | cap | bytes |",
          "|---|---|---|---|---|---|"]
    for h in cmod["largest_hidden"]:
        L.append(f"| {h['K']} | {h['link']} | {h['window_ms']:.2f} | {h['max_admit']} | "
                 f"{h['cap']} | {h['bytes'] / 1e9:.3f} GB |")
    L += ["", "| cap | max_admit | model, overlapped ms | model with the bytes moved ms | "
              "serial ms | measured ms |", "|---|---|---|---|---|---|"]
    for p in cmod["predicted_step_ms"]:
        L.append(f"| {p['cap']} | {p['max_admit']} | {p['overlapped_ms']} | "
                 f"{p['overlapped_ms_moved_bytes']} | {p['serial_ms']} | {p['measured_ms']} |")
    text = "\n".join(L) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_ANY",
               "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES",
               "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS"]


def sq(runs, substr: str, cmd: str, out: str, xcds: int = 8, simds: int = 1024):
    """Median per dispatch of each SQ/GRBM counter of the kernels matching
    `substr`, one column per run (NAME=DIR), and two shares of the SIMD
    cycles: VALU issue (SQ_INSTS_VALU x 4 cycles, one wave64 instruction on a
    16-lane SIMD) and MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES), each over the
    kernel's cycles (GRBM_GUI_ACTIVE, summed over the XCDs) x the SIMDs."""
    cols = []
    for spec in runs:
        name, d = spec.split("=", 1)
        rows = _rows(_find(d, "counter_collection.csv"))
        per = {}
        for r in rows:
            if substr not in r.get("Kernel_Name", ""):
                continue
            c = r["Counter_Name"]
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            per.setdefault(c, {})
            per[c][key] = per[c].get(key, 0.0) + float(r["Counter_Value"])
        if not per:
            raise ValueError(f"no rows for kernels matching {substr!r} in {d}")
        cols.append((name, {c: statistics.median(v.values()) for c, v in per.items()},
                     len(next(iter(per.values())))))
    lines = ["# SQ counters of the fused layer step", "",
             f"Kernel sources: {kernel_source_hash()}.  Median per dispatch of kernels matching "
             f"`{substr}`; one rocprofv3 pass per workload (command below, NAME = the workload).", "",
             "| counter | " + " | ".join(n for n, _, _ in cols) + " |",
             "|---|" + "---|" * len(cols)]
    for c in SQ_COUNTERS:
        if all(c in m for _, m, _ in cols):
            lines.append(f"| {c} | " + " | ".join(f"{m[c]:.4g}" for _, m, _ in cols) + " |")
    lines.append("| dispatches | " + " | ".join(str(k) for _, _, k in cols) + " |")
    cyc = [m["GRBM_GUI_ACTIVE"] / xcds * simds for _, m, _ in cols]
    lines.append("| VALU issue share | " + " | ".join(
        f"{m['SQ_INSTS_VALU'] * 4 / y:.1%}" for (_, m, _), y in zip(cols, cyc)) + " |")
    lines.append("| MFMA busy share | " + " | ".join(
        f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / y:.1%}" for (_, m, _), y in zip(cols, cyc)) + " |")
    lines += ["", f"Shares: over GRBM_GUI_ACTIVE / {xcds} XCDs x {simds} SIMDs; VALU = "
              "SQ_INSTS_VALU x 4 cycles.", "", "Command:", "", "    " + cmd, ""]
    text = "\n".join(lines)
    with open(out, "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=12)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--copy-kernel", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--cmd-fetch", required=True)
    c.add_argument("--cmd-write", required=True)
    c.add_argument("--algorithmic-bytes", type=int, default=None)
    c.add_argument("--out", required=True)
    k = sub.add_parser("per-kernel")
    k.add_argument("--fetch", required=True)
    k.add_argument("--write", required=True)
    k.add_argument("--stats", required=True)
    k.add_argument("--copy-kernel", required=True)
    k.add_argument("--copy-bytes", type=int, required=True)
    k.add_argument("--cmd-fetch", required=True)
    k.add_argument("--cmd-write", required=True)
    k.add_argument("--cmd-stats", required=True)
    k.add_argument("--out", required=True)
    pp = sub.add_parser("pipeline")
    pp.add_argument("bench_json")
    pp.add_argument("--cmd", required=True)
    pp.add_argument("--out", required=True)
    q = sub.add_parser("sq")
    q.add_argument("runs", nargs="+")
    q.add_argument("--kernel", required=True)
    q.add_argument("--cmd", required=True)
    q.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "sq":
        print(sq(a.runs, a.kernel, a.cmd, a.out))
        return
    if a.what == "pipeline":
        print(pipeline(a.bench_json, a.cmd, a.out))
        return
    if a.what == "per-kernel":
        print(per_kernel(a.fetch, a.write, a.stats, a.copy_kernel, a.copy_bytes,
                         [a.cmd_stats, a.cmd_fetch, a.cmd_write], a.out))
        return
    if a.what == "stats":
        print(stats(a.dir, a.cmd, a.out, a.top))
    else:
        print(json.dumps(counters(a.fetch, a.write, a.kernel, a.copy_kernel, a.copy_bytes,
                                  a.cmd_fetch, a.cmd_write, a.out, a.algorithmic_bytes), indent=1))


if __name__ == "__main__":
    main()

"""Summaries of rocprofv3 output for the kernels of this library.

    python -m load_balanced_split_amd.profiling stats <rocprof-dir> <title> <command>
    python -m load_balanced_split_amd.profiling pmc <fetch-dir> <write-dir> <title> <command>
    python -m load_balanced_split_amd.profiling counters <title> <command> <pmc-dir>...
    python -m load_balanced_split_amd.profiling balance <title> <command> <trace-json>...
    python -m load_balanced_split_amd.profiling budget <title> <command> <trace-json> <bench-json> <workload>

`stats` reads a `--kernel-trace --stats` run (CSV or rocpd database) and prints
per-kernel call counts and durations. `pmc` reads two `--pmc` runs (FETCH_SIZE,
then WRITE_SIZE, KiB per dispatch), calibrates FETCH_SIZE on the reduction and
WRITE_SIZE on the fill that `bench.py --pmc-run` launches over a buffer of known
size (each touches the buffer once in one direction), and prints the HBM bytes
per launch of each kernel, plus a JSON block that bench.py reads back (tagged
with a hash of the kernel sources, so a stale reading is never reported for
changed kernels). `counters` reads any number of `--pmc` runs and prints, per kernel,
the mean over dispatches of every counter they hold, with the ratios derived from
them (L2 hit rate, instructions per wave by kind). `balance` tabulates the
per-CU busy time of `bench.py --trace` runs (instrumented build: per-wave
realtime stamps and hardware CU ids of one attention launch per schedule).
`budget` splits one workload's fused step into phases: start-up, stream and tail
from a `bench.py --trace` run, kernel and step times from a `bench.py` run (HIP
events on the product build).
"""

import csv
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CALIBRATION_BYTES = 1 << 30          # bench.py --pmc-run copies this many bytes


# sources of kernels that no attention-path launch runs (the router GEMM, the MoE
# pipeline, the read probe, the page packer, the allocation-free wrapper): a change
# there leaves the attention path's counter readings valid
_NOT_ATTENTION = ("router", "moe", "probe", "pack", "noalloc")


def source_hash() -> str:
    """Hash of the sources the attention path's kernels and launches are built from."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        if not os.path.basename(f).startswith(_NOT_ATTENTION):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """Library kernels as name<template args> without spaces (attn_fused_kernel<false,true>
    is the E4M3-less fused kernel with the in-kernel merge); calibration kernels tagged."""
    name = re.sub(r"\((?:hpa::)?(?:\(anonymous namespace\)::)?(\w+)\)", r"(\1)", name)   # enum casts
    m = re.search(r"(attn_\w+_kernel|merge_kernel|plan_kernel|prologue_kernel|router_\w+_kernel|moe_\w+_kernel|"
                  r"stream_read_kernel)"
                  r"(<[^>]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "").replace(" ", "")
    if "reduce_kernel" in name:
        return "calib_read:reduce_kernel"
    if "FillFunctor" in name:
        return "calib_write:fill"
    return name[:70]


def _kernel_rows(d):
    """(name, duration_ns) of every dispatch in a rocprofv3 output directory."""
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    if rows:
        return rows
    for f in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        db = sqlite3.connect(f)
        rows += [(n, e - s) for n, s, e in db.execute("select name, start, end from kernels")]
    return rows


def stats(d, title, command):
    agg = {}
    for name, dur in _kernel_rows(d):
        agg.setdefault(short_name(name), []).append(dur / 1000.0)
    lines = [f"# {title}", "", f"command: {command}", "",
             f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s}"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k:44s} {len(v):6d} {sum(v) / len(v):9.2f} {min(v):9.2f} {max(v):9.2f} {sum(v):10.1f}")
    return "\n".join(lines)


def _pmc_rows(d, counter):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if counter is None or r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"]), r.get("Counter_Name")))
    if rows:
        return rows
    for f in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        db = sqlite3.connect(f)
        try:
            q = ("select k.name, sum(p.value) from pmc_events p join kernels k on p.event_id = k.id "
                 "where p.counter_name = ? group by p.event_id")
            rows += [(n, v, counter) for n, v in db.execute(q, (counter,))]
        except sqlite3.Error:
            pass
    return rows


def pmc(fetch_dir, write_dir, title, command):
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for name, kib, _ in _pmc_rows(d, counter):
            per.setdefault(short_name(name), {}).setdefault(counter, []).append(kib)
    rd, wr = per.get("calib_read:reduce_kernel"), per.get("calib_write:fill")
    if not rd or not wr or "FETCH_SIZE" not in rd or "WRITE_SIZE" not in wr:
        raise SystemExit("calibration kernels missing from the PMC runs")
    known_kib = CALIBRATION_BYTES / 1024.0
    # the 1 GiB dispatches are the largest of their kind (workspace fills are small)
    f_fetch = known_kib / max(rd["FETCH_SIZE"])
    f_write = known_kib / max(wr["WRITE_SIZE"])
    lines = [f"# {title}", "", f"command: {command}", "",
             f"calibration: a reduction reading {CALIBRATION_BYTES} bytes -> FETCH_SIZE x {f_fetch:.4f}; "
             f"a fill writing {CALIBRATION_BYTES} bytes -> WRITE_SIZE x {f_write:.4f}",
             "", f"{'kernel':44s} {'fetch_KiB':>12s} {'write_KiB':>12s} {'hbm_bytes_per_launch':>22s}"]
    out = {"source_hash": source_hash(), "fetch_factor": f_fetch, "write_factor": f_write, "kernels": {}}
    for k, v in sorted(per.items()):
        if k.startswith("calib_"):
            continue
        fe = sum(v.get("FETCH_SIZE", [0])) / max(1, len(v.get("FETCH_SIZE", [])))
        wr = sum(v.get("WRITE_SIZE", [0])) / max(1, len(v.get("WRITE_SIZE", [])))
        hbm = (fe * f_fetch + wr * f_write) * 1024.0
        out["kernels"][k] = {"fetch_kib": fe, "write_kib": wr, "hbm_bytes": hbm}
        lines.append(f"{k:44s} {fe:12.1f} {wr:12.1f} {hbm:22.0f}")
    lines += ["", "json: " + json.dumps(out)]
    return "\n".join(lines)


def counters(title, command, dirs):
    """Per-kernel means of every counter in the given `--pmc` runs. Counters are summed
    over their dimensions within a dispatch (SE, XCC, instance), then averaged over the
    dispatches of each kernel."""
    per = {}
    for d in dirs:
        disp = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), short_name(r["Kernel_Name"]),
                       r["Counter_Name"])
                disp[key] = disp.get(key, 0.0) + float(r["Counter_Value"])
        for (_, k, c), v in disp.items():
            per.setdefault(k, {}).setdefault(c, []).append(v)
    names = sorted({c for v in per.values() for c in v})
    lines = [f"# {title}", "", f"command: {command}", "",
             "mean per dispatch; derived: l2_hit = TCC_HIT / (TCC_HIT + TCC_MISS), "
             "per-wave counts = SQ_INSTS_* / SQ_WAVES", ""]
    for k, v in sorted(per.items()):
        if k.startswith("calib_") or k.startswith("__amd"):
            continue
        m = {c: sum(x) / len(x) for c, x in v.items()}
        lines.append(f"{k}  (dispatches: {max(len(x) for x in v.values())})")
        for c in names:
            if c in m:
                lines.append(f"    {c:28s} {m[c]:16.4g}")
        hit, miss = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            lines.append(f"    {'l2_hit':28s} {hit / (hit + miss):16.3f}")
        waves = m.get("SQ_WAVES")
        if waves:
            for c in names:
                if c.startswith("SQ_INSTS_") and c in m:
                    lines.append(f"    {c.lower()[3:] + '_per_wave':28s} {m[c] / waves:16.1f}")
        lines.append("")
    return "\n".join(lines)


def balance(title, command, files):
    cols = [("makespan_us", "makespan"), ("cu_busy_mean_us", "busy_mean"), ("cu_busy_max_us", "busy_max"),
            ("cu_busy_min_us", "busy_min"), ("cu_busy_max_over_mean", "max/mean"), ("utilisation", "util"),
            ("worker_end_p50_us", "end_p50"), ("worker_end_p99_us", "end_p99"), ("workgroups", "wgs"),
            ("cus", "cus")]
    lines = [f"# {title}", "", f"command: {command}", "",
             "one attention launch per schedule (the shortest of 5), times in us on the 100 MHz realtime "
             "counter; busy = union of a CU's wave intervals; util = mean busy / makespan", ""]
    for f in files:
        data = None
        for line in open(f):
            if line.startswith("{"):
                data = json.loads(line)
        if data is None:
            raise SystemExit(f"{f}: no JSON line")
        lines.append(f"## {data['workload']} (W = {data['num_workers']})")
        lines.append(f"{'schedule':24s}" + "".join(f"{h:>11s}" for _, h in cols))
        for sched, r in data.items():
            if isinstance(r, dict) and "makespan_us" in r:
                lines.append(f"{sched:24s}" + "".join(f"{r.get(k, float('nan')):>11}" for k, _ in cols))
        xcd = data.get("fused", {}).get("worker_end_mean_by_xcd_us")
        if xcd:
            lines.append("fused: mean worker end by XCD (us): " + ", ".join(f"{k}: {v}" for k, v in xcd.items()))
        lines.append("")
    return "\n".join(lines)


def _last_json(path):
    data = None
    for line in open(path):
        if line.startswith("{"):
            data = json.loads(line)
    if data is None:
        raise SystemExit(f"{path}: no JSON line")
    return data


def budget(title, command, trace_file, bench_file, workload):
    """Per-phase budget of a workload's fused step. The instrumented build's start-up
    stamps wait for all of a wave's loads so far, so its phases before the first
    K/V issue run longer than in the product build; its launch is timed on its own."""
    t = _last_json(trace_file)
    f = t["fused"]
    it = f["items"]
    e = _last_json(bench_file)["per_config"][workload]
    fs = e["balanced_fused"]
    step, attn, merge = fs["us_per_step"], fs["kernel_us"]["attn"], fs["kernel_us"]["merge"]
    su = it["startup_us (range, item, length, q+page ids)"]
    issue, end50, span = it["first_issue_after_start_us"], f["worker_end_p50_us"], f["makespan_us"]
    stream = end50 - issue      # us
    xcd = f.get("worker_end_mean_by_xcd_us", {})
    rows = [
        ("dispatch -> worker start (p50 / max)", f"{f['worker_start_p50_us']} / {f['worker_start_max_us']}",
         "hardware dispatch of the workgroups"),
        ("work range known", su[0], "one HBM round trip (the lengths), then the closed-form partition"),
        ("first item's q and page ids in registers", su[3], "a second dependent round trip (page-table entries, q)"),
        ("first K/V loads issued", issue, "the third round trip (K/V) starts here"),
        ("K/V stream to the median worker end", round(stream, 2),
         f"all {e['kv_bytes'] / 1e6:.1f} MB from the first issue to the last worker end: "
         f"{e['kv_bytes'] / (span - issue) / 1e3:.0f} GB/s"),
        ("tail: median -> last worker end", round(span - end50, 2),
         "mean worker end by XCD " + ", ".join(f"{k}: {v}" for k, v in xcd.items())),
        ("instrumented launch (makespan)", span, "start-up stamps wait for each wave's loads"),
        ("attention kernel (events)", attn, "product build"),
        ("merge kernel (events)", merge, "launch, a round trip for split counts and slot bases, "
                                         "one for the partials, the reduction, the stores"),
        ("gaps between the two launches", round(step - attn - merge, 2), "graph replay of attention then merge"),
        ("step (events)", step, f"{e['kv_bytes'] / step / 1e3:.0f} GB/s of K/V, "
                                f"{e['kv_bytes'] / step / 1e3 / 8000:.3f} of 8 TB/s; attention + merge "
                                f"{e['attn_plus_merge_kv_frac']}"),
    ]
    lines = [f"# {title}", "", f"command: {command}", "",
             f"workload {t['workload']} (W = {t['num_workers']}); times in us from the kernel's first wave",
             "", f"{'phase':44s}{'us':>14s}  bound / note"]
    lines += [f"{name:44s}{str(v):>14s}  {note}" for name, v, note in rows]
    return "\n".join(lines) + "\n"


def read_traffic(summary_path, kernel):
    """HBM bytes per launch of `kernel` from a pmc summary, or None when the summary is
    missing or was taken on different kernel sources."""
    if not os.path.exists(summary_path):
        return None
    for line in open(summary_path):
        if line.startswith("json: "):
            data = json.loads(line[6:])
            if data.get("source_hash") != source_hash():
                return None
            k = data["kernels"].get(kernel)
            return None if k is None else k["hbm_bytes"]
    return None


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        print(stats(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif mode == "pmc":
        print(pmc(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5]))
    elif mode == "counters":
        print(counters(sys.argv[2], sys.argv[3], sys.argv[4:]))
    elif mode == "balance":
        print(balance(sys.argv[2], sys.argv[3], sys.argv[4:]))
    elif mode == "budget":
        print(budget(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6]), end="")
    else:
        raise SystemExit(__doc__)

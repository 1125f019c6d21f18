"""Benchmark: load-balanced split-KV decode attention on one MI355X.

A step is the whole hot path over one batch resident in HBM: plan -> attention
-> merge (plus the fused prologue for the E4M3 workload). The headline schedule
(--schedule, default fused) evaluates the planner's closed forms inside the
persistent attention kernel; the other balanced schedule (a separate planner
launch, same work list, same output bits) is reported beside it. The default
workload is the skewed batch (1 x 131072 + 31 x 4096 tokens, 8:1 GQA, head dim
128, 64-token pages, bf16 KV), where the pages report their kernel-level gain.

Timing:
* headline: K steps (rounded down to a multiple of R) replayed from one HIP
  graph holding R steps, back to back, bracketed by a device synchronise; the
  batch is held in R copies used round-robin so that
  R - 1 other copies (more than twice the 256 MB Infinity Cache) are read
  between two uses of the same bytes -- each step reads its KV from HBM.
* per kernel: for each launch kind (planner, attention, merge) a loop of
  back-to-back launches of that kind alone over the same rotating copies,
  bracketed by HIP events on the launch stream; average = span / launches.
* comparison: the same two passes for the static split-KV schedules.
* CPU baseline: the fp64 oracle timed on the host on the same batch.

Prints ONE JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn μs/step + achieved KV-read HBM GB/s (% of peak), mixed-length batch"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20
REALTIME_MHZ = 100.0      # the shader's constant "realtime" counter (s_memrealtime)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", type=int, default=2, help="0..4 (2 = skewed 1x128K + 31x4K)")
    p.add_argument("--num-workers", type=int, default=0)
    p.add_argument("--schedule", choices=["fused", "balanced"], default="fused",
                   help="headline balanced schedule: planner inside the persistent kernel (fused) "
                        "or a separate planner launch (balanced)")
    p.add_argument("--event-steps", type=int, default=60)
    p.add_argument("--no-static", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probe", action="store_true", help="skip the plain streaming-read probe")
    p.add_argument("--no-router", action="store_true", help="skip the split-precision router GEMM")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--trace", action="store_true",
                   help="use the instrumented build and report per-CU busy time (tail balance) instead")
    p.add_argument("--products", choices=["mfma", "valu"], default="mfma",
                   help="library build: MFMA products (the library) or the comparison build whose "
                        "attention kernels compute Q.K^T and P.V with VALU dot products")
    p.add_argument("--pmc-run", action="store_true",
                   help="short run for rocprofv3 counter passes: 1 GiB calibration read and write "
                        "kernels, a few steps of each schedule over rotating copies, then the router "
                        "GEMM at its three shapes")
    return p.parse_args()


def pmc_main(args):
    os.environ["HPA_PRODUCTS"] = args.products
    import torch
    from load_balanced_split_amd import _lib, inputs
    from load_balanced_split_amd.profiling import CALIBRATION_BYTES
    from load_balanced_split_amd.runner import DeviceStep
    _lib.lib()
    w = inputs.config_workload(args.workload)
    R = max(2, math.ceil(2 * MALL_BYTES / (w.k_cache.nbytes + w.v_cache.nbytes)) + 1)
    copies = [DeviceStep(w, num_workers=args.num_workers) for _ in range(min(R, 16))]
    # calibration kernels: a reduction that reads CALIBRATION_BYTES and writes one value,
    # and a fill that writes CALIBRATION_BYTES and reads nothing
    buf = torch.empty(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        buf.fill_(1.0)
        _ = buf.sum()
    torch.cuda.synchronize()
    del buf
    for sched in ("balanced", "fused", "single", "static_splits", "static_chunk"):
        for rep in range(2):
            for d in copies:
                d.step(sched)
        torch.cuda.synchronize()
    del copies
    # the router GEMM at its three shapes (kernels named by their tile shape)
    from load_balanced_split_amd.runner import RouterStep
    for T, E, H in ROUTER_SHAPES:
        r = RouterStep(inputs.router_workload(T, E, H, seed=T), top_k=ROUTER_TOP_K)
        for passes in (2, 2, 1):
            r.run(passes)
        torch.cuda.synchronize()
        del r
    print(json.dumps({"pmc_run": True, "workload": args.workload}), flush=True)


def balance_report(rec, items_per_worker=None):
    """Tail balance of one attention launch from per-wave records [blocks, waves, 4]:
    makespan, per-CU busy time (union of its waves' intervals), worker end times
    (overall, per XCD, and by the number of items a worker had)."""
    t0, t1, hw = rec[..., 0].astype(np.int64), rec[..., 1].astype(np.int64), rec[..., 2]
    live = t0 > 0
    start, end = t0[live].min(), t1[live].max()
    tick_us = 1.0 / REALTIME_MHZ
    hwid = (hw & 0xFFFFFFFF).astype(np.int64)
    key = ((hw >> 32).astype(np.int64) << 8) | (((hwid >> 13) & 7) << 5) | (((hwid >> 12) & 1) << 4) | ((hwid >> 8) & 15)
    busy = {}
    for k in np.unique(key[live]):
        sel = live & (key == k)
        iv = sorted(zip(t0[sel].tolist(), t1[sel].tolist()))
        tot, cs, ce = 0, iv[0][0], iv[0][1]
        for a, b in iv[1:]:
            if a > ce:
                tot += ce - cs
                cs, ce = a, b
            else:
                ce = max(ce, b)
        busy[int(k)] = tot + ce - cs
    bv = np.array(list(busy.values()), np.float64) * tick_us
    xcc_of_worker = ((hw[:, 0] >> 32).astype(np.int64))
    wl = live.any(axis=1)
    wend = (np.where(live, t1, 0).max(axis=1) - start)[wl] * tick_us
    wstart = (np.where(live, t0, np.iinfo(np.int64).max).min(axis=1) - start)[wl] * tick_us
    makespan = (end - start) * tick_us
    extra = {}
    wend_all = (np.where(live, t1, 0).max(axis=1) - start) * tick_us
    extra["worker_end_mean_by_xcd_us"] = {int(x): round(float(wend_all[wl & (xcc_of_worker == x)].mean()), 2)
                                          for x in np.unique(xcc_of_worker[wl])}
    if items_per_worker is not None:
        ipw = np.asarray(items_per_worker)
        n = min(len(ipw), len(wend_all))
        extra["worker_end_mean_by_items_us"] = {
            int(k): [round(float(wend_all[:n][wl[:n] & (ipw[:n] == k)].mean()), 2), int((wl[:n] & (ipw[:n] == k)).sum())]
            for k in np.unique(ipw[:n][wl[:n]])}
    return {**extra, "makespan_us": round(makespan, 2), "cus": len(bv), "cu_busy_mean_us": round(bv.mean(), 2),
            "cu_busy_max_us": round(bv.max(), 2), "cu_busy_min_us": round(bv.min(), 2),
            "cu_busy_max_over_mean": round(bv.max() / bv.mean(), 3),
            "utilisation": round(bv.mean() / makespan, 3),
            "worker_end_p50_us": round(float(np.percentile(wend, 50)), 2),
            "worker_end_p99_us": round(float(np.percentile(wend, 99)), 2),
            "worker_start_p50_us": round(float(np.percentile(wstart, 50)), 2),
            "worker_start_max_us": round(float(wstart.max()), 2),
            "worker_busy_p50_us": round(float(np.percentile(wend - wstart, 50)), 2),
            "worker_busy_p99_us": round(float(np.percentile(wend - wstart, 99)), 2),
            "workgroups": int(live.any(axis=1).sum())}


def item_phase_report(rec, item_tiles=None):
    """Per-item phases from the instrumented build (wave 0 of each workgroup): time
    from the kernel's first wave to its first item, stream time of the first and of
    later items (per tile when the plan's item sizes are given), the combine, and
    the gap between one item's combine and the next item's first issue."""
    from load_balanced_split_amd import _lib
    t0w = rec[..., 0].astype(np.int64)
    live = t0w > 0
    start = t0w[live].min()
    tick_us = 1.0 / REALTIME_MHZ
    o = 4 + _lib.TRACE_START
    ph = rec[:, 0, o:o + 3 * _lib.TRACE_ITEMS].astype(np.int64).reshape(len(rec), _lib.TRACE_ITEMS, 3)
    su = rec[:, 0, 4:o].astype(np.int64)
    ok = (su > 0).all(axis=1)
    startup = [round(float(((su[ok, k] - start) * tick_us).mean()), 3) for k in range(_lib.TRACE_START)] if ok.any() else None
    first, later, comb, gap, lead = [], [], [], [], []
    for b in range(len(rec)):
        for k in range(_lib.TRACE_ITEMS):
            t_issue, t_end, t_comb = ph[b, k]
            if t_issue == 0 or t_end == 0 or t_comb == 0:
                break
            dur = (t_end - t_issue) * tick_us
            if item_tiles is not None and b < len(item_tiles) and k < len(item_tiles[b]):
                dur /= max(1, item_tiles[b][k])
            (first if k == 0 else later).append(dur)
            comb.append((t_comb - t_end) * tick_us)
            if k == 0:
                lead.append((t_issue - start) * tick_us)
            elif ph[b, k - 1, 2] > 0:
                gap.append((t_issue - ph[b, k - 1, 2]) * tick_us)
    m = lambda x: round(float(np.mean(x)), 3) if x else None
    unit = "us_per_tile" if item_tiles is not None else "us"
    return {f"stream_first_item_{unit}": m(first), f"stream_later_items_{unit}": m(later),
            "later_items": len(later), "combine_us": m(comb), "issue_gap_us": m(gap),
            "first_issue_after_start_us": m(lead),
            "startup_us (range, item, length, q+page ids)": startup}


def trace_main(args):
    """Per-CU busy time of the attention kernel, balanced vs static split-KV."""
    os.environ["HPA_TRACE"] = "1"
    import torch
    from load_balanced_split_amd import _lib, inputs
    from load_balanced_split_amd.runner import DeviceStep
    _lib.lib()
    w = inputs.config_workload(args.workload)
    d = DeviceStep(w, num_workers=args.num_workers)
    W = d.num_workers
    out = {"metric": "attention tail balance (instrumented build)", "workload": inputs.CONFIG_NAMES[args.workload],
           "num_workers": W, "realtime_clock_mhz": REALTIME_MHZ}
    for sched in ("balanced", "fused", "single", "static_splits", "static_chunk"):
        reps = []
        for r in range(5):
            d.step(sched)                     # planner (if any) and a full step first
            torch.cuda.synchronize()
            d.partial_ws.zero_()              # partials and the record area of the traced launch
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            d.attend(sched, flags=_lib.ATTN_NO_MERGE)
            e1.record()
            torch.cuda.synchronize()
            ipw, tiles = None, None
            pa = d.plan_arrays() if sched == "balanced" else None
            if pa is not None and pa["D"] == 0:       # with a dynamic tail, items meet workers at run time
                off = np.array(pa["worker_off"])
                ipw = np.diff(off)
                sz = np.array(pa["item_t1"]) - np.array(pa["item_t0"])
                tiles = [sz[off[i]:off[i + 1]] for i in range(len(off) - 1)]
            recs = d.trace_records()
            rep = balance_report(recs, ipw)
            rep["items"] = item_phase_report(recs, tiles)
            rep["launch_event_us"] = round(e0.elapsed_time(e1) * 1e3, 2)
            reps.append(rep)
        out[sched] = min(reps, key=lambda x: x["makespan_us"])
    print(json.dumps(out), flush=True)


def algorithmic_bytes(w):
    """Bytes the method must move per step (valid tokens only): KV + q + out +
    page ids + lengths (+ scales); the prologue's reads and writes on top."""
    from load_balanced_split_amd.inputs import HEAD_DIM
    kv = w.kv_bytes()
    lens = w.attended_lens().astype(np.int64)
    pages = int(((lens + 63) // 64).sum())
    other = 2 * w.batch * w.hq * HEAD_DIM * 2 + pages * 4 + w.batch * 4
    if w.kv_dtype == "fp8":
        other += 8 * w.hkv
    pro = 0
    if w.has_prologue:
        pro = w.batch * (w.hq + 2 * w.hkv) * HEAD_DIM * 2 + w.batch * 2 * w.hkv * HEAD_DIM + 2 * HEAD_DIM * 4
    return kv, kv + other, pro


def main():
    args = parse()
    if args.trace:
        return trace_main(args)
    if args.pmc_run:
        return pmc_main(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is measured on one "
              "GPU's share of the work; across GPUs each would plan and attend only its own requests' tiles",
              file=sys.stderr)
        sys.exit(2)
    os.environ["HPA_PRODUCTS"] = args.products
    import torch
    from load_balanced_split_amd import _lib, inputs
    from load_balanced_split_amd.runner import DeviceStep

    assert torch.cuda.is_available(), "no GPU"
    _lib.lib()                               # fails loudly if libhpa.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.config_workload(args.workload)
    kv_bytes, alg_bytes, pro_bytes = algorithmic_bytes(w)
    pool_bytes = w.k_cache.nbytes + w.v_cache.nbytes
    R = max(2, math.ceil(2 * MALL_BYTES / max(pool_bytes, 1)) + 1)
    R = min(R, 16)
    # num_workers 0: each schedule takes the library's default for it
    copies = [DeviceStep(w, num_workers=args.num_workers, device="cuda:0") for _ in range(R)]
    W = copies[0].num_workers
    print(f"[bench] workload {args.workload} ({w.name}): KV {kv_bytes / 1e6:.1f} MB, {R} copies, W={W}",
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def run_step(d, sched):
        d.step(sched)

    # eager reference outputs (also the warm-up of every code path)
    scheds = ["balanced", "fused", "single"] + ([] if args.no_static else ["static_splits", "static_chunk"])
    eager = {}
    for s in scheds:
        for d in copies:
            run_step(d, s)
        torch.cuda.synchronize()
        eager[s] = copies[0].out.clone()
        assert copies[0].device_error() == 0

    spread = {}

    def graph_time(sched):
        """Seconds per step: one HIP graph holds one step per copy (R steps), replayed
        back to back, so host launch cost is paid once per R steps. Also keeps the
        10th/50th/90th percentile of the per-step time over the replays (HIP events
        around each replay on the launch stream)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in copies:
                run_step(d, sched)
        torch.cuda.synchronize()
        for i in range(max(1, args.warmup // R)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // R)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(reps):
            g.replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        per_step = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / R for i in range(reps))
        q = lambda f: per_step[min(len(per_step) - 1, int(f * len(per_step)))]
        spread[sched] = [round(q(0.1), 2), round(q(0.5), 2), round(q(0.9), 2)]
        # every copy's graph output equals the eager output, bit for bit
        for d in copies:
            assert torch.equal(d.out, eager[sched]), f"graph replay of {sched} differs from eager"
        del g
        return (t1 - t0) / (reps * R)

    def kernel_times(sched):
        """Average duration (ms) of each launch kind: HIP events on the launch stream
        around the replay of a graph of event_steps back-to-back launches of that kind
        alone (rotating copies), so that short kernels are not bound by host submission."""
        if w.has_prologue and sched == "balanced":
            kinds = ["prologue+plan"]                                   # one launch (runner.step)
        else:
            kinds = (["prologue"] if w.has_prologue else []) + (["plan"] if sched == "balanced" else [])
        kinds += ["attn"] if sched == "single" else ["attn", "merge"]    # single: one launch merges too
        launch = {
            "prologue+plan": lambda d: d.prologue_plan(),
            "prologue": lambda d: d.prologue(),
            "plan": lambda d: d.plan(),
            "attn": lambda d: d.attend(sched, flags=_lib.ATTN_NO_MERGE),
            "merge": lambda d: d.attend(sched, flags=_lib.ATTN_MERGE_ONLY),
        }
        res = {}
        for kind in kinds:
            for i in range(R):
                launch[kind](copies[i])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(args.event_steps):
                    launch[kind](copies[i % R])
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            res[kind] = e0.elapsed_time(e1) / args.event_steps
            del g
        for d in copies:
            assert torch.equal(d.out, eager[sched])
        return res

    # the balanced method -- headline schedule, the other balanced schedule beside it
    head = args.schedule
    other = "balanced" if head == "fused" else "fused"
    step_s = graph_time(head)
    ev = kernel_times(head)
    us = step_s * 1e6
    kv_gbps = kv_bytes / step_s / 1e9
    attn_s = ev["attn"] * 1e-3
    achieved = alg_bytes / attn_s / 1e9
    result = {
        "metric": METRIC,
        "value": round(kv_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": max(1, args.steps // R) * R,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8-e4m3 KV, bf16 q/out",
        "data": "synthetic (seeded; shapes and length mix of the pages' kernel benchmark)",
        "config": {"workload": inputs.CONFIG_NAMES[args.workload], "schedule": SCHED_NAMES[head],
                   "num_workers": W, "static_num_workers": copies[0].static_workers,
                   "products": args.products, "rotating_copies": R, "kv_bytes": kv_bytes,
                   "algorithmic_bytes": alg_bytes},
        "us_per_step": round(us, 2),
        "us_per_step_p10_p50_p90": spread[head],
        "kv_frac_of_peak": round(kv_gbps / PEAK_HBM_GBPS, 4),
        "kernel_us": {k: round(v * 1e3, 2) for k, v in ev.items()},
        "attn_plus_merge_kv_gbps": round(kv_bytes / ((ev["attn"] + ev.get("merge", 0.0)) * 1e-3) / 1e9, 1),
        "attn_plus_merge_kv_frac": round(kv_bytes / ((ev["attn"] + ev.get("merge", 0.0)) * 1e-3) / 1e9
                                         / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": attn_kernel_name(head, w.kv_dtype),
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_per_launch(head, w.kv_dtype, args.workload, args.products)},
    }
    if pro_bytes:
        result["config"]["prologue_bytes"] = pro_bytes
    # the other balanced schedule: same work list and bits, planner inside / outside the kernel
    tf = graph_time(other)
    ef = kernel_times(other)
    result[SCHED_NAMES[other]] = {"us_per_step": round(tf * 1e6, 2), "kv_gbps": round(kv_bytes / tf / 1e9, 1),
                                  "kernel_us": {k: round(v * 1e3, 2) for k, v in ef.items()},
                                  "kv_frac_of_peak": round(kv_bytes / tf / 1e9 / PEAK_HBM_GBPS, 4)}
    # single launch: planner, attention and merge in one persistent kernel
    t1 = graph_time("single")
    e1 = kernel_times("single")
    result["balanced_single_launch"] = {"us_per_step": round(t1 * 1e6, 2), "kv_gbps": round(kv_bytes / t1 / 1e9, 1),
                                        "kernel_us": {k: round(v * 1e3, 2) for k, v in e1.items()}}
    if not args.no_static:
        st = {}
        for s in scheds[3:]:
            t = graph_time(s)
            e = kernel_times(s)
            st[s] = {"us_per_step": round(t * 1e6, 2), "attn_us": round(e["attn"] * 1e3, 2),
                     "merge_us": round(e["merge"] * 1e3, 2),
                     "balanced_speedup": round(t / step_s, 3),
                     "balanced_attn_speedup": round(e["attn"] / ev["attn"], 3)}
        result["static_split_kv"] = st
    if not args.no_router:
        result["router_gemm"] = router_bench(args, stream)
    if not args.no_probe:
        probe = stream_read_probe(stream)
        probe["attn_frac_of_probe"] = round(achieved / probe["gbps"], 4)
        result["stream_read_probe"] = probe
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, kv_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


PEAK_BF16_TFLOPS = 2500.0
ROUTER_SHAPES = [(1, 256, 7168), (64, 256, 7168), (4096, 256, 7168)]
ROUTER_TOP_K = 8


def router_bytes_flops(T, E, H, passes, k=ROUTER_TOP_K):
    """Algorithmic HBM bytes (the weight halves read, x read, logits and top-k written)
    and MFMA flops of one router call."""
    nbytes = E * H * 2 * passes + T * H * 2 + T * E * 4 + T * k * 8
    return nbytes, 2 * passes * T * E * H


def router_bench(args, stream):
    """The split-precision router GEMM (pack once, then GEMM + top-k per call) on
    synthetic bf16 activations and an fp32 weight: per shape the time of one call,
    both kernels, replayed from a HIP graph over rotating copies (weights and
    activations read from HBM), its roofline, and PyTorch's fp32 GEMM + top-k on the
    same data for context."""
    import torch
    from load_balanced_split_amd import inputs
    from load_balanced_split_amd.runner import RouterStep
    out = {}
    for T, E, H in ROUTER_SHAPES:
        rw = inputs.router_workload(T, E, H, seed=T)
        foot = E * H * 4 + T * H * 2 + T * E * 4
        R = min(64, max(2, math.ceil(2 * MALL_BYTES / foot) + 1))
        steps = [RouterStep(rw, top_k=ROUTER_TOP_K) for _ in range(R)]
        res = {"tokens": T, "experts": E, "hidden": H, "top_k": ROUTER_TOP_K, "rotating_copies": R}
        for passes in (2, 1):
            for s in steps:
                s.run(passes)
            torch.cuda.synchronize()
            ref = steps[0].logits.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in steps:
                    s.run(passes)
            g.replay()
            torch.cuda.synchronize()
            reps = max(2, math.ceil(40 / R))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * R)
            assert torch.equal(steps[0].logits, ref), "router graph replay differs from eager"
            nbytes, flops = router_bytes_flops(T, E, H, passes)
            t_hbm, t_mfma = nbytes / (PEAK_HBM_GBPS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12)
            if t_hbm >= t_mfma:
                roof = {"bound": "hbm", "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s"}
            else:
                roof = {"bound": "mfma", "achieved": round(flops / (us * 1e-6) / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s"}
            roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
            res[f"passes{passes}"] = {"us_per_call": round(us, 2), "roofline": roof}
            del g
        # context: PyTorch's fp32 GEMM on the fp32 weight, then torch.topk
        xf = steps[0].x.float()
        wt = steps[0].w
        for _ in range(3):
            torch.topk(xf @ wt.t(), ROUTER_TOP_K, dim=1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            torch.topk(xf @ wt.t(), ROUTER_TOP_K, dim=1)
        e1.record(stream)
        torch.cuda.synchronize()
        res["torch_fp32_gemm_topk_us"] = round(e0.elapsed_time(e1) * 1e3 / 20, 2)
        out[f"T{T}"] = res
        del steps
    return out


def stream_read_probe(stream, gib=4, launches=10):
    """Plain streaming-read bandwidth of this GPU (the library's read probe: 16-byte
    non-temporal loads, one contiguous slice per workgroup) over a buffer far larger
    than the caches; the best of a few workgroup counts, timed with HIP events
    around a graph of back-to-back launches."""
    import torch
    from load_balanced_split_amd import _lib
    buf = torch.zeros(gib << 28, dtype=torch.int32, device="cuda")
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    best = None
    for wgs in (512, 1024, 2048, 4096):
        _lib.hpa_probe_stream_read(buf, wgs, sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(launches):
                _lib.hpa_probe_stream_read(buf, wgs, sink)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = buf.numel() * 4 * launches / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"gbps": round(gbps, 1), "workgroups": wgs, "bytes": buf.numel() * 4}
        del g
    del buf
    return best


SCHED_NAMES = {"fused": "balanced_fused", "balanced": "balanced_planned"}
WORKLOAD_KEYS = {0: "tiny", 1: "uniform", 2: "skewed", 3: "mix", 4: "fp8_prologue"}


def attn_kernel_name(sched, kv_dtype):
    base = "attn_fused_kernel" if sched == "fused" else "attn_balanced_kernel"
    return f"{base}<{'bf16' if kv_dtype == 'bf16' else 'fp8'}>"


def traffic_per_launch(sched, kv_dtype, workload, products="mfma"):
    """HBM bytes per launch of the headline attention kernel from the committed
    rocprofv3 counter summary of this workload; None when there is none, when it
    was taken on other kernel sources, or for the VALU-product build (the summary
    covers the library's MFMA kernels)."""
    from load_balanced_split_amd.profiling import read_traffic
    if products != "mfma":
        return None
    fp8 = "false" if kv_dtype == "bf16" else "true"
    key = f"attn_fused_kernel<{fp8},false>" if sched == "fused" else f"attn_balanced_kernel<{fp8}>"
    path = os.path.join(ROOT, "profiles", f"attn_hbm_traffic_{WORKLOAD_KEYS[workload]}.txt")
    t = read_traffic(path, key)
    return None if t is None else int(round(t))


def cpu_baseline(w, kv_bytes, budget_s):
    """The fp64 oracle, as it stands, on the host cores over the same batch."""
    import threadpoolctl
    from oracle import attention as oa
    from oracle import prologue as opro

    def once():
        if w.has_prologue:
            pr = opro.prologue(w)
            oa.decode_attention(pr["q_rot"], pr["k_cache"], pr["v_cache"], pr["seq_lens"], w.page_table, w.hkv,
                                w.sm_scale, w.kv_dtype, w.k_scale, w.v_scale)
        else:
            oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, w.hkv, w.sm_scale,
                                w.kv_dtype, w.k_scale, w.v_scale)

    def timed(budget):
        times = []
        t_end = time.perf_counter() + budget
        while True:
            t0 = time.perf_counter()
            once()
            times.append(time.perf_counter() - t0)
            if time.perf_counter() > t_end or len(times) >= 50:
                break
        return float(np.median(times)), len(times)

    t, n = timed(budget_s)
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    with threadpoolctl.threadpool_limits(1):
        t1, n1 = timed(budget_s / 3)
    return {"value": round(kv_bytes / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_step": round(t * 1e6, 1),
            "sample": f"the whole batch, {n} runs (median), numpy fp64 gather-then-softmax",
            "single_thread": {"value": round(kv_bytes / t1 / 1e9, 3), "us_per_step": round(t1 * 1e6, 1),
                              "runs": n1}}


if __name__ == "__main__":
    main()

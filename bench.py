"""Benchmark: load-balanced split-KV decode attention on one MI355X.

A step is the whole hot path over one batch resident in HBM: plan -> attention
-> merge (plus the fused prologue for the E4M3 workload). The headline schedule
(--schedule, default fused) evaluates the planner's closed forms inside the
persistent attention kernel; the other balanced schedule (a separate planner
launch, same work list, same output bits) is reported beside it. The default
workload is the skewed batch (1 x 131072 + 31 x 4096 tokens, 8:1 GQA, head dim
128, 64-token pages, bf16 KV), where the pages report their kernel-level gain.

Timing (every workload 0-4 by default; the headline is --workload, default 2):
* whole steps: HIP graphs holding at least 10 consecutive steps (whole
  rotations over R copies of the batch, used round-robin so that R - 1 other
  copies -- more than twice the 256 MB Infinity Cache -- are read between two
  uses of the same bytes: each step reads its KV from HBM). The replays are
  queued behind a bounded spin kernel, with HIP events between them, so each
  event span is GPU time only. The headline value is the mean over exactly
  --steps steps; every per_config entry times at least 100 steps, and
  p10/p50/p90 are over replays (a replay's span over its steps).
* per kernel: for each launch kind (prologue, planner, attention, merge) a graph
  of back-to-back launches of that kind alone over the same rotating copies,
  bracketed by HIP events on the launch stream; average = span / launches.
* comparison: the same for the static split-KV schedules.
* CPU baseline: the fp64 oracle timed on the host on the same batch (a bounded
  number of whole-batch runs; one thread as well for workloads 0-2).

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
    p.add_argument("--workload", type=int, default=2, help="headline workload 0..4 (2 = skewed 1x128K + 31x4K)")
    p.add_argument("--workloads", type=int, nargs="*", default=[0, 1, 2, 3, 4],
                   help="workloads measured for the per_config block (the headline one always)")
    p.add_argument("--only-headline", action="store_true", help="measure the headline workload only")
    p.add_argument("--num-workers", type=int, default=0)
    p.add_argument("--schedule", choices=["fused", "balanced"], default="fused",
                   help="headline balanced schedule: planner inside the persistent kernel (fused) "
                        "or a separate planner launch (balanced)")
    p.add_argument("--event-steps", type=int, default=60)
    p.add_argument("--no-static", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probe", action="store_true", help="skip the plain streaming-read probe")
    p.add_argument("--no-router", action="store_true", help="skip the split-precision router GEMM")
    p.add_argument("--no-moe", action="store_true", help="skip the fused FP8 MoE layer")
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
    # the fused FP8 MoE layer at its decode batch sizes (weights packed once)
    from load_balanced_split_amd.runner import MoeStep
    for T in MOE_TOKENS:
        m = MoeStep(inputs.moe_workload(T, seed=T, **MOE_SHAPE))
        for _ in range(3):
            m.run()
        torch.cuda.synchronize()
        del m
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
    """Per-CU busy time of the attention kernel: the balanced schedules (planned in
    every item order, with the merge kernel or merged in-kernel; fused; single
    launch) against static split-KV. The traced launch reads a copy of the batch
    that R - 1 other copies have been read after, so its KV comes from HBM."""
    os.environ["HPA_TRACE"] = "1"
    import torch
    from load_balanced_split_amd import _lib, inputs
    from load_balanced_split_amd.runner import DeviceStep
    _lib.lib()
    w = inputs.config_workload(args.workload)
    pool_bytes = w.k_cache.nbytes + w.v_cache.nbytes
    R = min(16, max(2, math.ceil(2 * MALL_BYTES / max(pool_bytes, 1)) + 1))
    copies = [DeviceStep(w, num_workers=args.num_workers) for _ in range(R)]
    W = copies[0].num_workers
    out = {"metric": "attention tail balance (instrumented build)", "workload": inputs.CONFIG_NAMES[args.workload],
           "num_workers": W, "realtime_clock_mhz": REALTIME_MHZ, "rotating_copies": R}
    runs = [("balanced", 0), ("balanced", 1), ("balanced", 2), ("balanced_inmerge", 0), ("balanced_inmerge", 2),
            ("fused", 0), ("single", 0), ("static_splits", 0), ("static_chunk", 0)]
    for sched, order in runs:
        one_launch = sched in ("single", "balanced_inmerge")
        reps = []
        for r in range(5):
            for c in copies:                          # copy 0 (plan included), then every other copy
                c.step(sched, item_order=order)
            torch.cuda.synchronize()
            d = copies[0]
            d.partial_ws.zero_()                      # the per-wave record area after the partials
            if one_launch:                            # partials NaN-filled for the in-kernel merges
                S, G = w.batch * w.hkv, w.hq // w.hkv
                d.partial_ws[: (5 * W + S) * G * (128 + 2) * 4].fill_(0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            d.attend(sched, flags=0 if one_launch else _lib.ATTN_NO_MERGE)
            e1.record()
            torch.cuda.synchronize()
            ipw, tiles = None, None
            pa = d.plan_arrays() if sched.startswith("balanced") else None
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
        out[sched + (f"_order{order}" if order else "")] = min(reps, key=lambda x: x["makespan_us"])
        print(f"[trace] {sched} order {order}: makespan {out[sched + (f'_order{order}' if order else '')]['makespan_us']}",
              file=sys.stderr, flush=True)
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


class Timer:
    """GPU time of back-to-back steps.

    Steps are captured in HIP graphs of several consecutive steps each (rotating
    over the copies). The replays are enqueued behind a spin kernel that holds
    the GPU for a few milliseconds (torch.cuda._sleep, bounded), so the host has
    queued every replay and event before the GPU reaches them: the span between
    two consecutive events is the GPU time of one replay's steps, with no host
    submission gap in it. A sample is one replay: its span over its step count.
    """

    BATCH = 40

    def __init__(self, stream):
        import torch
        self.torch, self.stream = torch, stream
        # calibrate the spin kernel: cycles per microsecond
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(2_000_000)
        e1.record(stream)
        torch.cuda.synchronize()
        per_us = 2_000_000 / max(1.0, e0.elapsed_time(e1) * 1e3)
        self.sleep_cycles = int(per_us * 4000)          # ~4 ms of spinning per batch

    def run(self, plan):
        """plan: [(graph, steps it holds)] replayed in order; returns [(span_us, steps)]."""
        torch = self.torch
        out = []
        for b0 in range(0, len(plan), self.BATCH):
            part = plan[b0:b0 + self.BATCH]
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(part) + 1)]
            torch.cuda.synchronize()
            torch.cuda._sleep(self.sleep_cycles)
            ev[0].record(self.stream)
            for i, (g, _) in enumerate(part):
                g.replay()
                ev[i + 1].record(self.stream)
            torch.cuda.synchronize()
            out += [(ev[i].elapsed_time(ev[i + 1]) * 1e3, n) for i, (_, n) in enumerate(part)]
        return out


GRAPH_STEPS = 10      # at least this many consecutive steps per captured graph


def pct(xs, f):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]


def measure_workload(idx, args, stream, timer, steps, headline):
    """Every schedule on one workload: per-step times of whole steps (HIP events),
    per-kernel averages, the attention kernel's roofline, static split-KV beside it
    and the oracle on the host cores."""
    import torch
    from load_balanced_split_amd import _lib, inputs
    from load_balanced_split_amd.runner import DeviceStep
    t_build = time.perf_counter()
    w = inputs.config_workload(idx)
    kv_bytes, alg_bytes, pro_bytes = algorithmic_bytes(w)
    pool_bytes = w.k_cache.nbytes + w.v_cache.nbytes
    R = min(16, max(2, math.ceil(2 * MALL_BYTES / max(pool_bytes, 1)) + 1))
    copies = [DeviceStep(w, num_workers=args.num_workers, device="cuda:0") for _ in range(R)]
    W = copies[0].num_workers
    print(f"[bench] workload {idx} ({w.name}): KV {kv_bytes / 1e6:.1f} MB, {R} copies, W={W}, "
          f"built in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)
    head = args.schedule
    scheds = ["fused", "balanced", "single"] + ([] if args.no_static else ["static_splits", "static_chunk"])
    eager = {}
    for s in scheds:
        for d in copies:
            d.step(s)
        torch.cuda.synchronize()
        eager[s] = copies[0].out.clone()
        assert copies[0].device_error() == 0, (idx, s)

    # steps per graph: whole rotations over the copies, at least GRAPH_STEPS
    per_graph = R * math.ceil(GRAPH_STEPS / R)

    def capture(sched, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                copies[i % R].step(sched)
        return g

    def step_times(sched, n):
        """n steps exactly: full graphs of per_graph steps, then one graph of the rest;
        returns the samples [(span_us, steps)]."""
        full = capture(sched, per_graph)
        rest = n % per_graph
        plan = [(full, per_graph)] * (n // per_graph)
        if rest:
            plan.append((capture(sched, rest), rest))
        torch.cuda.synchronize()
        timer.run([(full, per_graph)] * max(1, math.ceil(args.warmup / per_graph)))   # warm-up
        samples = timer.run(plan)
        for d in copies:                                  # every replay equals the eager output
            assert torch.equal(d.out, eager[sched]), f"graph replay of {sched} differs from eager"
        del plan, full
        return samples

    def kernel_times(sched):
        """Average duration (us) of each launch kind: HIP events on the launch stream
        around the replay of a graph of event_steps back-to-back launches of that kind
        alone (rotating copies)."""
        if w.has_prologue and sched == "balanced":
            kinds = ["prologue+plan"]
        else:
            kinds = (["prologue"] if w.has_prologue else []) + (["plan"] if sched == "balanced" else [])
        kinds += ["attn"] if sched == "single" else ["attn", "merge"]
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
            res[kind] = round(e0.elapsed_time(e1) * 1e3 / args.event_steps, 2)
            del g
        for d in copies:
            assert torch.equal(d.out, eager[sched])
        return res

    def summary(samples):
        steps = sum(n for _, n in samples)
        mean = sum(t for t, _ in samples) / steps
        per = [t / n for t, n in samples]
        return {"steps": steps, "samples": len(samples), "steps_per_sample": per_graph,
                "us_per_step": round(mean, 2),
                "us_p10_p50_p90": [round(pct(per, f), 2) for f in (0.1, 0.5, 0.9)],
                "kv_gbps": round(kv_bytes / (mean * 1e-6) / 1e9, 1),
                "kv_frac_of_peak": round(kv_bytes / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                "alg_gbps": round((alg_bytes + pro_bytes) / (mean * 1e-6) / 1e9, 1)}

    # context only: the products' flops (q.K and p.V, 2 flops per multiply-add) over the attended tokens
    alg_gflop = round(float(w.attended_lens().astype(np.int64).sum()) * w.hq * 4 * 128 / 1e9, 3)
    ent = {"workload": inputs.CONFIG_NAMES[idx], "num_workers": W, "static_num_workers": copies[0].static_workers,
           "rotating_copies": R, "kv_bytes": kv_bytes, "algorithmic_bytes": alg_bytes, "alg_gflop": alg_gflop}
    if pro_bytes:
        ent["prologue_bytes"] = pro_bytes
    ent[SCHED_NAMES[head]] = summary(step_times(head, max(100, steps)))
    # exactly the requested number of steps (the headline value)
    exact = summary(step_times(head, steps)) if headline else None
    kt = kernel_times(head)
    ent[SCHED_NAMES[head]]["kernel_us"] = kt
    attn_us = kt["attn"]
    am = attn_us + kt.get("merge", 0.0)
    ent["attn_kv_frac"] = round(kv_bytes / (attn_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
    ent["attn_plus_merge_kv_frac"] = round(kv_bytes / (am * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
    ent["roofline"] = {"bound": "hbm", "kernel": attn_kernel_name(head, w.kv_dtype),
                       "achieved": round(alg_bytes / (attn_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                       "unit": "GB/s", "frac": round(alg_bytes / (attn_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                       "traffic": traffic_per_launch(head, w.kv_dtype, idx, args.products)}
    if ent["roofline"]["traffic"]:
        # bytes the attention launch moves beyond the algorithmic ones (partial slots,
        # metadata, re-reads)
        ent["attn_overhead_bytes"] = ent["roofline"]["traffic"] - alg_bytes
    for other in ("balanced", "single", "fused"):
        if other == head:
            continue
        e = summary(step_times(other, max(100, steps)))
        e["kernel_us"] = kernel_times(other)
        ent[SCHED_NAMES[other]] = e
    if not args.no_static:
        st = {}
        for s in ("static_splits", "static_chunk"):
            e = summary(step_times(s, max(100, steps)))
            k = kernel_times(s)
            e.update({"attn_us": k["attn"], "merge_us": k["merge"],
                      "balanced_speedup": round(e["us_per_step"] / ent[SCHED_NAMES[head]]["us_per_step"], 3),
                      "balanced_attn_speedup": round(k["attn"] / attn_us, 3)})
            st[s] = e
        ent["static_split_kv"] = st
    del copies
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        ent["cpu_baseline"] = cpu_baseline(w, kv_bytes, CPU_BUDGET_S[idx], single_thread=idx <= 2)
    return ent, exact, w


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

    assert torch.cuda.is_available(), "no GPU"
    _lib.lib()                               # fails loudly if libhpa.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    timer = Timer(stream)
    workloads = [args.workload] if args.only_headline else sorted(set(args.workloads) | {args.workload})
    per_config = {}
    head_w = exact = None
    for idx in workloads:
        ent, exact_k, w = measure_workload(idx, args, stream, timer, args.steps, idx == args.workload)
        per_config[WORKLOAD_KEYS[idx]] = ent
        if idx == args.workload:
            head_w, exact = w, exact_k
    head = per_config[WORKLOAD_KEYS[args.workload]]
    hs = head[SCHED_NAMES[args.schedule]]
    mean_us = exact["us_per_step"]
    result = {
        "metric": METRIC,
        "value": round(head["kv_bytes"] / (mean_us * 1e-6) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": exact["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(mean_us * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head_w.kv_dtype == "bf16" else "fp8-e4m3 KV, bf16 q/out",
        "data": "synthetic (seeded; shapes and length mix of the pages' kernel benchmark)",
        "config": {"workload": head["workload"], "schedule": SCHED_NAMES[args.schedule],
                   "num_workers": head["num_workers"], "products": args.products,
                   "rotating_copies": head["rotating_copies"], "kv_bytes": head["kv_bytes"],
                   "algorithmic_bytes": head["algorithmic_bytes"]},
        "us_per_step": round(mean_us, 2),
        "us_per_step_p10_p50_p90": exact["us_p10_p50_p90"],
        "timing": f"HIP events around graph replays of {exact['steps_per_sample']} consecutive steps, queued "
                  "behind a spin kernel; value and ms_per_step: mean over exactly `steps` steps; "
                  "percentiles over replays (per_config: at least 100 steps)",
        "kv_frac_of_peak": round(head["kv_bytes"] / (mean_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "alg_gbps": round((head["algorithmic_bytes"] + head.get("prologue_bytes", 0)) / (mean_us * 1e-6) / 1e9, 1),
        "kernel_us": hs["kernel_us"],
        "attn_plus_merge_kv_frac": head["attn_plus_merge_kv_frac"],
        "roofline": head["roofline"],
    }
    if "attn_overhead_bytes" in head:
        result["attn_overhead_bytes"] = head["attn_overhead_bytes"]
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    result["per_config"] = per_config
    if not args.no_router:
        result["router_gemm"] = router_bench(args, stream)
    if not args.no_moe:
        result["fused_moe"] = moe_bench(args, stream)
    if not args.no_probe:
        probe = stream_read_probe(stream)
        probe["attn_frac_of_probe"] = round(head["roofline"]["achieved"] / probe["gbps"], 4)
        result["stream_read_probe"] = probe
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


MOE_SHAPE = dict(experts=128, top_k=8, hidden=2048, inter=768)
MOE_TOKENS = (1, 32, 128)


def moe_bytes(mw):
    """Algorithmic HBM bytes of one MoE call: the E4M3 weights and per-channel scales of
    the experts some token is routed to, the hidden states, the routing and the output."""
    used = np.unique(mw.ids[(mw.ids >= 0) & (mw.ids < mw.experts)])
    n_used = len(used)
    w = n_used * (3 * mw.inter * mw.hidden + (2 * mw.inter + mw.hidden) * 4)
    return w + 2 * mw.tokens * mw.hidden * 2 + mw.tokens * mw.top_k * 8, n_used


def moe_bench(args, stream):
    """The fused FP8 MoE layer at decode batch sizes (128 experts, top 8, hidden 2048,
    inter 768; synthetic weights and routing): one call = the layer's launches (two at
    one token, five at 32 and 128), replayed from a HIP graph over copies of the weights in separate buffers
    (more than twice the Infinity Cache between two uses of the same bytes), so the
    weights come from HBM; roofline against the HBM peak."""
    import torch
    from load_balanced_split_amd import inputs
    from load_balanced_split_amd.runner import MoeStep
    out = {}
    base = None
    for T in MOE_TOKENS:
        mw = inputs.moe_workload(T, seed=T, **MOE_SHAPE)
        if base is None:
            base = mw                                      # the weights, drawn once
        else:
            mw.w1, mw.s1, mw.w2, mw.s2 = base.w1, base.s1, base.w2, base.s2
        nbytes, n_used = moe_bytes(mw)
        touched = n_used * 3 * mw.inter * mw.hidden
        R = min(16, max(2, math.ceil(2 * MALL_BYTES / touched) + 1))
        steps = [MoeStep(mw) for _ in range(R)]
        for st in steps:
            st.run()
        torch.cuda.synchronize()
        ref = steps[0].out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for st in steps:
                st.run()
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
        assert torch.equal(steps[0].out, ref), "MoE graph replay differs from eager"
        assert int(steps[0].err.item()) == 0
        gbps = nbytes / (us * 1e-6) / 1e9
        out[f"T{T}"] = {"tokens": T, **MOE_SHAPE, "experts_used": n_used, "rotating_copies": R,
                        "us_per_call": round(us, 2), "algorithmic_bytes": nbytes,
                        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}}
        del g, steps
        torch.cuda.empty_cache()
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


SCHED_NAMES = {"fused": "balanced_fused", "balanced": "balanced_planned", "single": "balanced_single_launch"}
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
    key = f"attn_fused_kernel<{fp8},false>" if sched == "fused" else f"attn_balanced_kernel<{fp8},false>"
    path = os.path.join(ROOT, "profiles", f"attn_hbm_traffic_{WORKLOAD_KEYS[workload]}.txt")
    t = read_traffic(path, key)
    return None if t is None else int(round(t))


# seconds of oracle time per workload (each a bounded sample: whole batches, repeated)
CPU_BUDGET_S = {0: 2.0, 1: 3.0, 2: 6.0, 3: 8.0, 4: 8.0}


def cpu_baseline(w, kv_bytes, budget_s, single_thread=False):
    """The fp64 oracle, as it stands, on the host: the whole batch, repeated within a
    time budget (median). It runs with a BLAS pool of one thread per CPU this process
    may use; cores = that count, avg_busy_threads = process CPU time / wall time."""
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

    def timed(budget, threads):
        times = []
        with threadpoolctl.threadpool_limits(threads):
            c0, t_end = time.process_time(), time.perf_counter() + budget
            w0 = time.perf_counter()
            while True:
                t0 = time.perf_counter()
                once()
                times.append(time.perf_counter() - t0)
                if time.perf_counter() > t_end or len(times) >= 50:
                    break
            busy = (time.process_time() - c0) / max(1e-9, time.perf_counter() - w0)
        return float(np.median(times)), len(times), busy

    cpus = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    t, n, busy = timed(budget_s, cpus)
    out = {"value": round(kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": cpus, "kind": "oracle",
           "us_per_step": round(t * 1e6, 1), "os_cpu_count": os.cpu_count(),
           "avg_busy_threads": round(busy, 2),
           "sample": f"the whole batch, {n} runs (median), numpy fp64 gather-then-softmax"}
    if single_thread:
        t1, n1, _ = timed(budget_s / 2, 1)
        out["single_thread"] = {"value": round(kv_bytes / t1 / 1e9, 4), "us_per_step": round(t1 * 1e6, 1),
                                "runs": n1, "cores": 1}
    return out


if __name__ == "__main__":
    main()

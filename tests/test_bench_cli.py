"""Host-side checks of the benchmark and profiling tooling (no GPU): the one-GPU
rule of bench.py, and the rocprofv3 summary parsers on small synthetic outputs."""

import csv
import json
import os
import subprocess
import sys

from load_balanced_split_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_profiling_summaries_on_synthetic_outputs(tmp_path):
    kt = tmp_path / "trace"
    kt.mkdir()
    _write(kt / "x_kernel_trace.csv", [
        {"Kernel_Name": "void hpa::(anonymous namespace)::attn_fused_kernel<false, false>(hpa::AttnArgs)",
         "Start_Timestamp": 1000, "End_Timestamp": 26000},
        {"Kernel_Name": "void hpa::(anonymous namespace)::attn_fused_kernel<false, false>(hpa::AttnArgs)",
         "Start_Timestamp": 30000, "End_Timestamp": 57000},
        {"Kernel_Name": "void hpa::(anonymous namespace)::merge_kernel<(hpa::(anonymous namespace)::MergeMode)2>"
                        "(hpa::(anonymous namespace)::MergeArgs)", "Start_Timestamp": 0, "End_Timestamp": 5000}])
    text = profiling.stats(str(kt), "t", "c")
    assert "attn_fused_kernel<false,false>" in text and "merge_kernel<(MergeMode)2>" in text
    line = [l for l in text.splitlines() if l.startswith("attn_fused_kernel")][0].split()
    assert line[1] == "2" and float(line[2]) == 26.0            # calls, average microseconds

    reduce_name = "void at::native::reduce_kernel<512, 1>(...)"
    fill_name = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>(...)"
    kib = profiling.CALIBRATION_BYTES / 1024
    for counter, sub, cal_name, cal_val, kval in (("FETCH_SIZE", "f", reduce_name, kib / 2, 65000.0),
                                                   ("WRITE_SIZE", "w", fill_name, kib, 1100.0)):
        d = tmp_path / sub
        d.mkdir()
        _write(d / "x_counter_collection.csv", [
            {"Dispatch_Id": 1, "Kernel_Name": cal_name, "Counter_Name": counter, "Counter_Value": cal_val},
            {"Dispatch_Id": 2, "Kernel_Name": "hpa::attn_fused_kernel<false, false>(hpa::AttnArgs)",
             "Counter_Name": counter, "Counter_Value": kval}])
    out = profiling.pmc(str(tmp_path / "f"), str(tmp_path / "w"), "t", "c")
    data = json.loads([l for l in out.splitlines() if l.startswith("json: ")][0][6:])
    assert abs(data["fetch_factor"] - 2.0) < 1e-12 and abs(data["write_factor"] - 1.0) < 1e-12
    k = data["kernels"]["attn_fused_kernel<false,false>"]
    assert abs(k["hbm_bytes"] - (65000.0 * 2 + 1100.0) * 1024) < 1e-6
    assert data["source_hash"] == profiling.source_hash()
    summary = tmp_path / "traffic.txt"
    summary.write_text(out + "\n")
    assert profiling.read_traffic(str(summary), "attn_fused_kernel<false,false>") == k["hbm_bytes"]
    summary.write_text(out.replace(data["source_hash"], "0" * 16) + "\n")
    assert profiling.read_traffic(str(summary), "attn_fused_kernel<false,false>") is None   # stale sources

    c = tmp_path / "c"
    c.mkdir()
    _write(c / "x_counter_collection.csv", [
        {"Dispatch_Id": 1, "Kernel_Name": "hpa::router_topk_kernel<1>(hpa::RouterArgs)", "Counter_Name": n,
         "Counter_Value": v} for n, v in (("TCC_HIT_sum", 30.0), ("TCC_MISS_sum", 10.0), ("SQ_WAVES", 4.0),
                                          ("SQ_INSTS_VALU", 400.0))])
    text = profiling.counters("t", "c", [str(c)])
    assert "l2_hit" in text and "0.750" in text and "insts_valu_per_wave" in text


def test_phase_budget_on_synthetic_runs(tmp_path):
    """The per-phase budget: start-up stamps and worker ends from a trace run, kernel
    and step times from a bench run; the derived spans are differences of the two."""
    trace = {"workload": "w", "num_workers": 4, "fused": {
        "worker_start_p50_us": 0.5, "worker_start_max_us": 0.9, "worker_end_p50_us": 20.0, "makespan_us": 23.0,
        "worker_end_mean_by_xcd_us": {"0": 20.0, "1": 21.0},
        "items": {"first_issue_after_start_us": 5.0, "startup_us (range, item, length, q+page ids)": [1.5, 2.0, 2.5, 4.0]}}}
    bench = {"per_config": {"w": {"kv_bytes": 18_000_000, "attn_plus_merge_kv_frac": 0.5,
                                  "balanced_fused": {"us_per_step": 30.0, "kernel_us": {"attn": 24.0, "merge": 4.0}}}}}
    tf, bf = tmp_path / "t.json", tmp_path / "b.json"
    tf.write_text("[bench] noise\n" + json.dumps(trace) + "\n")
    bf.write_text(json.dumps(bench) + "\n")
    text = profiling.budget("title", "cmd", str(tf), str(bf), "w")
    rows = {l[:44].strip(): l[44:58].strip() for l in text.splitlines() if l[:1].isalpha() and "  " in l}
    assert rows["K/V stream to the median worker end"] == "15.0"          # 20 - 5
    assert rows["tail: median -> last worker end"] == "3.0"               # 23 - 20
    assert rows["gaps between the two launches"] == "2.0"                 # 30 - 24 - 4
    assert "1000 GB/s" in text                                            # 18 MB over 23 - 5 us


def test_committed_traffic_summaries_match_the_kernel_sources():
    """bench.py reports an attention launch's measured HBM bytes only from a counter
    summary taken on the current kernel sources; every committed summary must be one."""
    import glob
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "attn_hbm_traffic_*.txt")))
    assert files
    for f in files:
        line = next(l for l in open(f) if l.startswith("json: "))
        assert json.loads(line[6:])["source_hash"] == profiling.source_hash(), os.path.basename(f)

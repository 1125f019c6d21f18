"""Parity of the comparison build whose attention kernels compute Q.K^T and P.V
with VALU dot products (libhpa_valu.so) against the fp64 oracle, to the same
tolerances as the library. Run as a child process with HPA_PRODUCTS=valu (one
build of the library per process): tests/test_gpu_valu_products.py does that.
Prints each case before it runs; exits non-zero on the first failure."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from load_balanced_split_amd import _lib, inputs  # noqa: E402
from load_balanced_split_amd.runner import DeviceStep  # noqa: E402
from oracle import attention as oa  # noqa: E402
from oracle import prologue as opro  # noqa: E402
from tests.helpers import assert_within  # noqa: E402

EDGE_LENS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 700, 1000]


def oracle_out(w):
    if w.has_prologue:
        pr = opro.prologue(w)
        return oa.decode_attention(pr["q_rot"], pr["k_cache"], pr["v_cache"], pr["seq_lens"], w.page_table,
                                   w.hkv, w.sm_scale, w.kv_dtype, w.k_scale, w.v_scale)
    return oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, w.hkv, w.sm_scale,
                               w.kv_dtype, w.k_scale, w.v_scale)


def check(w, runs, ref=None):
    ref = oracle_out(w) if ref is None else ref
    outs = {}
    for sched, W in runs:
        print(f"valu {w.name} {w.kv_dtype} {w.hq}:{w.hkv} sched={sched} W={W}", flush=True)
        d = DeviceStep(w, num_workers=W)
        d.step(sched)
        torch.cuda.synchronize()
        assert d.device_error() == 0, (w.name, sched, W)
        got = d.output_f64()
        r = assert_within(got, ref, w.kv_dtype, f"valu {w.name} {sched} W={W}")
        print(f"  max err/tol {r['max_ratio']:.3f}", flush=True)
        outs[(sched, W)] = got
    return outs


def main():
    assert _lib.LIB_PATH.endswith("libhpa_valu.so"), _lib.LIB_PATH
    torch.cuda.set_device(0)
    _lib.lib()
    sched_runs = [("balanced", 0), ("balanced", 3), ("fused", 0), ("fused", 37), ("single", 0),
                  ("static_splits", 0), ("static_chunk", 0)]
    for kv in ("bf16", "fp8"):
        for hq, hkv in ((8, 1), (4, 1), (2, 2), (32, 4)):
            w = inputs.build_workload("edge", EDGE_LENS, hq, hkv, kv, seed=5, pool_pages=60, poison=True)
            outs = check(w, sched_runs)
            for W in (0,):
                # the same work list and merge order: the balanced schedules agree bit for bit
                assert np.array_equal(outs[("balanced", W)], outs[("fused", W)])
                assert np.array_equal(outs[("balanced", W)], outs[("single", W)])
    rng = np.random.default_rng(78)
    for trial in range(3):
        lens = rng.integers(0, 3000, size=int(rng.integers(1, 24)))
        w = inputs.build_workload("rand", lens, 8, 1, "bf16", seed=int(rng.integers(1 << 30)), poison=True)
        check(w, [("balanced", int(rng.integers(1, 50))), ("fused", 0)])
    check(inputs.config_workload(0), [("balanced", 0), ("static_splits", 0)])
    check(inputs.config_workload(2), [("fused", 0), ("balanced", 0), ("static_splits", 0)])
    check(inputs.config_workload(4), [("balanced", 0), ("fused", 0)])
    print("valu parity ok", flush=True)


if __name__ == "__main__":
    main()

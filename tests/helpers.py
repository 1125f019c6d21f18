"""Shared test helpers: tolerance checks and a cached library build."""

import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "load_balanced_split_amd", "libhpa.so")

# spec tolerances: |gpu - ref| <= atol + rtol * |ref| per element
TOL = {"bf16": (1e-2, 1e-2), "fp8": (3e-2, 3e-2)}


def tolerance_report(got, ref, atol, rtol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    ratio = err / (atol + rtol * np.abs(ref))
    return dict(max_ratio=float(np.nanmax(ratio)) if ratio.size else 0.0,
                max_abs=float(np.nanmax(err)) if err.size else 0.0,
                finite=bool(np.all(np.isfinite(got))))


def assert_within(got, ref, kv_dtype, what=""):
    atol, rtol = TOL[kv_dtype]
    r = tolerance_report(got, ref, atol, rtol)
    assert r["finite"], f"{what}: non-finite output"
    assert r["max_ratio"] <= 1.0, f"{what}: {r}"
    return r


def ensure_built():
    if not os.path.exists(LIB):
        from load_balanced_split_amd.build import build
        build()

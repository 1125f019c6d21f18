"""Pins of the oracle's number formats against PyTorch's dtypes and the OCP spec table."""

import json
import os

import numpy as np
import pytest
import torch

from oracle.formats import bf16_to_f64, e4m3_encode, e4m3_to_f64
from oracle.prologue import bf16_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = e4m3_to_f64(codes), torch_e4m3(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.isnan(ours).sum() == 2          # only S.1111.111


def test_e4m3_decode_ocp_named_values():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3_ocp_values.json")))
    for code, val in spec["values"].items():
        got = float(e4m3_to_f64(np.array([int(code, 16)]))[0])
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == val and np.signbit(got) == np.signbit(val), code


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_to_f64(codes)), codes)


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000) * 50,
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(100000) * 0.01,            # subnormal range
    ]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


def test_e4m3_encode_midpoints_ties_to_even_brute_force():
    vals = e4m3_to_f64(np.arange(0x7F))               # non-negative finite values, increasing
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([mids, -mids, mids * (1 + 1e-9), mids * (1 - 1e-9)])
    got = e4m3_encode(x)
    for xi, gi in zip(x, got):
        d = np.abs(vals - abs(xi))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        want = int(want) | (0x80 if xi < 0 else 0)
        assert gi == want, (xi, gi, want)


def test_e4m3_encode_saturates_and_nan():
    got = e4m3_encode(np.array([448.0, 464.0, 479.9, 1e4, np.inf, -1e30, np.nan]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = bf16_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[ok], ref[ok])
    assert bf16_to_f64(np.array([0x3F80, 0xC000]))[0] == 1.0


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-20, 20, 300000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_encode(x.astype(np.float64)), ref)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert bf16_encode(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8]))[0] == 0x3F80
    assert bf16_encode(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82

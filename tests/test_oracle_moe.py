"""Pins of the fused FP8 MoE oracle: the quantiser against PyTorch's E4M3 cast and
the nearest-value definition, one-hot inputs that select single weight columns
exactly, the activation's closed forms, a gate driven far negative, and the
invariants of routing and merging."""

import math

import numpy as np
import pytest

from load_balanced_split_amd import inputs
from oracle import moe
from oracle.formats import e4m3_to_f64

torch = pytest.importorskip("torch")


def test_token_quantiser_matches_torch_cast_and_nearest_value():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 100, size=(64, 1))).astype(np.float32)
    v[3] = 0.0                                    # a zero row: scale 0, zero codes
    v[5, 7] = 0.0
    codes, s = moe.quantize_fp32(v)
    assert s[3] == 0 and not codes[3].any()
    for r in range(64):
        if s[r] == 0:
            continue
        assert s[r] == np.float32(np.max(np.abs(v[r])) / np.float32(448))
        q = (v[r] / s[r]).astype(np.float32)
        want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[r], want), r
        # every code is a nearest representable value of v / s
        all_vals = e4m3_to_f64(np.arange(0, 0x7F))
        d = np.abs(np.abs(q.astype(np.float64))[:, None] - all_vals[None, :]).min(axis=1)
        assert np.all(np.abs(np.abs(e4m3_to_f64(codes[r])) - np.abs(q)) <= d + 1e-12)
        assert np.max(np.abs(e4m3_to_f64(codes[r]))) == 448.0     # the largest element maps to 448


def _tiny(seed, H=32, I=16, E=3, T=1, K=1):
    return inputs.moe_workload(T, E, K, H, I, seed=seed)


def test_one_hot_token_selects_one_column_of_w1():
    """x = c e_j: the token's codes are 448 e_j with scale c / 448, so g = c * s1 * W1[:, j]
    exactly. W1 is square here (2I = H) and its row scales differ, so a transposed
    operand or a per-column scale gives another vector."""
    w = _tiny(1)
    j, c = 11, 3.0
    x = np.zeros(32, np.float32)
    x[j] = c
    x8, sx = moe.quantize_fp32(x[None])
    assert x8[0, j] == 0x7E and np.count_nonzero(x8) == 1           # 448
    e = 2
    g = moe.gate_up(x8[0], float(sx[0]), w.w1[e], w.s1[e].astype(np.float64))
    want = float(sx[0]) * 448.0 * w.s1[e].astype(np.float64) * e4m3_to_f64(w.w1[e][:, j])
    assert np.array_equal(g, want)
    assert not np.allclose(g, float(sx[0]) * 448.0 * w.s1[e] * e4m3_to_f64(w.w1[e][j, :]))


def test_one_hot_activation_code_selects_one_column_of_w2():
    """An activation with one non-zero code i: y = sa * s2 * dec(code) * W2[:, i] exactly (W2
    square here: H = I)."""
    w = _tiny(2, H=32, I=32)
    a8 = np.zeros(32, np.uint8)
    i, code, sa = 5, 0x3A, 0.125                       # 0x3A = 1.25
    a8[i] = code
    e = 1
    y = moe.down(a8, sa, w.w2[e], w.s2[e].astype(np.float64))
    want = sa * 1.25 * w.s2[e].astype(np.float64) * e4m3_to_f64(w.w2[e][:, i])
    assert np.array_equal(y, want)
    assert not np.allclose(y, sa * 1.25 * w.s2[e] * e4m3_to_f64(w.w2[e][i, :]))


def test_activation_closed_forms():
    assert moe.silu(0.0) == 0.0
    assert moe.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(moe.silu(-40.0)) < 40 * math.exp(-40) * 1.01
    assert moe.silu(1.0) == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    g = np.array([0.0, 2.0, -1.0, 40.0, 3.0, 0.5, 7.0, -2.0])       # I = 4: gate | up
    a = moe.activation(g)
    assert np.allclose(a, [0.0, moe.silu(2.0) * 0.5, moe.silu(-1.0) * 7.0, 40.0 * -2.0], rtol=1e-12)


def test_gate_far_negative_gives_zero_layer():
    """All gate codes at -448 and a positive token: every gate value is very negative,
    silu is ~0, the layer output is ~0. Swapped gate and up halves would not be."""
    w = _tiny(3, H=64, I=32, T=2, K=2)
    w.x[:] = inputs.bf16_bits(np.abs(np.random.default_rng(4).standard_normal((2, 64))).astype(np.float32) + 0.5)
    w.w1[:, :32, :] = 0xFE                             # -448 in every gate row
    w.s1[:, :32] = 1.0
    out = moe.fused_moe(w.x, w.ids, w.weights, w.w1, w.s1, w.w2, w.s2)
    assert np.max(np.abs(out)) < 1e-30
    w.w1[:, :32, :], w.w1[:, 32:, :] = w.w1[:, 32:, :].copy(), 0xFE     # now the up half
    assert np.max(np.abs(moe.fused_moe(w.x, w.ids, w.weights, w.w1, w.s1, w.w2, w.s2))) > 1e-3


def test_routing_and_merge_invariants():
    w = inputs.moe_workload(6, 5, 2, 64, 32, seed=5)
    base = moe.fused_moe(w.x, w.ids, w.weights, w.w1, w.s1, w.w2, w.s2)
    # permuting tokens permutes the output rows
    p = np.random.default_rng(6).permutation(6)
    out = moe.fused_moe(w.x[p], w.ids[p], w.weights[p], w.w1, w.s1, w.w2, w.s2)
    assert np.array_equal(out, base[p])
    # relabelling the experts (weights and ids together) changes nothing
    r = np.random.default_rng(7).permutation(5)            # new label of expert e is r[e]
    inv = np.argsort(r)
    out = moe.fused_moe(w.x, r[w.ids].astype(np.int32), w.weights, w.w1[inv], w.s1[inv], w.w2[inv], w.s2[inv])
    assert np.array_equal(out, base)
    # two slots of the same expert with weights u, v == one slot with u + v; scaling the weights
    ids2 = np.stack([w.ids[:, 0], w.ids[:, 0]], axis=1)
    w0 = w.weights[:, 0].astype(np.float64)
    wts2 = np.stack([w0 * 0.25, w0 * 0.75], axis=1)           # exact in fp64
    one = moe.fused_moe(w.x, w.ids[:, :1], w0[:, None], w.w1, w.s1, w.w2, w.s2)
    two = moe.fused_moe(w.x, ids2, wts2, w.w1, w.s1, w.w2, w.s2)
    assert np.allclose(one, two, rtol=1e-12, atol=1e-15)
    assert np.allclose(moe.fused_moe(w.x, w.ids, 3.0 * w.weights.astype(np.float64), w.w1, w.s1, w.w2, w.s2),
                       3.0 * base, rtol=1e-12, atol=1e-15)
    # an expert id outside [0, E) contributes nothing; a zero token gives a zero row
    bad = w.ids.copy()
    bad[:, 1] = 5
    assert np.allclose(moe.fused_moe(w.x, bad, w.weights, w.w1, w.s1, w.w2, w.s2),
                       moe.fused_moe(w.x, w.ids[:, :1], w.weights[:, :1], w.w1, w.s1, w.w2, w.s2), rtol=0, atol=0)
    x0 = w.x.copy()
    x0[2] = 0
    assert not moe.fused_moe(x0, w.ids, w.weights, w.w1, w.s1, w.w2, w.s2)[2].any()


def test_workload_recipe():
    w = inputs.moe_workload(16, 32, 4, 128, 64, seed=0)
    assert w.ids.shape == (16, 4) and w.weights.shape == (16, 4)
    assert all(len(set(r)) == 4 for r in w.ids.tolist())
    assert np.allclose(w.weights.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(w.weights, axis=1) <= 0)             # largest logit first
    # every weight row: its largest magnitude is code 448 * scale
    v = e4m3_to_f64(w.w1[3]) * w.s1[3][:, None]
    assert np.allclose(np.abs(v).max(axis=1), 448.0 * w.s1[3])

"""Pins of the prologue oracle: PyTorch's rms_norm, the complex form of RoPE, closed forms."""

import numpy as np
import pytest
import torch

from load_balanced_split_amd import inputs
from oracle import prologue as opro
from oracle.kv_layout import page_rows
from oracle.formats import bf16_to_f64, e4m3_encode

D = 128


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, D)) * 3
    w = rng.uniform(0.5, 1.5, D)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(opro.rms_norm(x, w, 1e-6), ref, rtol=1e-14, atol=1e-15)


def test_rms_norm_constant_vector_closed_form():
    w = np.linspace(0.5, 1.5, D)
    for c in (-3.0, 0.25, 7.0):
        np.testing.assert_allclose(opro.rms_norm(np.full(D, c), w, 1e-6), w * c / np.sqrt(c * c + 1e-6), rtol=1e-15)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((20, D))
    pos = rng.integers(0, 131073, 20)
    theta = 1e6
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * pos[:, None] * theta ** (-np.arange(64) / 64.0))
    out = opro.rope_rotate_half(x, pos, theta)
    np.testing.assert_allclose(out[:, :64], z.real, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(out[:, 64:], z.imag, rtol=1e-9, atol=1e-9)


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, D))
    assert np.array_equal(opro.rope_rotate_half(x, np.zeros(10), 1e6), x)
    out = opro.rope_rotate_half(x, rng.integers(0, 131072, 10), 1e6)
    np.testing.assert_allclose(np.linalg.norm(out, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    m, n = 1000, 37
    base = opro.rope_rotate_half(q, m, 1e6) @ opro.rope_rotate_half(k, n, 1e6)
    for delta in (1, 64, 5000, 100000):
        shifted = opro.rope_rotate_half(q, m + delta, 1e6) @ opro.rope_rotate_half(k, n + delta, 1e6)
        assert abs(shifted - base) < 1e-9


def test_rope_unit_vector_closed_form():
    for i in (0, 5, 63):
        e = np.zeros(D)
        e[i] = 1.0
        pos = 12345
        ang = pos * 1e6 ** (-2 * i / D)
        out = opro.rope_rotate_half(e, pos, 1e6)
        want = np.zeros(D)
        want[i], want[i + 64] = np.cos(ang), np.sin(ang)
        np.testing.assert_allclose(out, want, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_prologue_appends_at_live_length(kv_dtype):
    w = inputs.build_workload("p", [0, 5, 63, 64, 200], 8, 2, kv_dtype, seed=4, prologue=True)
    r = opro.prologue(w)
    assert list(r["seq_lens"]) == [1, 6, 64, 65, 201]
    for b, L in enumerate(w.seq_lens):
        p = w.page_table[b, L // 64]
        for g in range(w.hkv):
            assert np.array_equal(page_rows(r["k_cache"][p, g], "k", kv_dtype)[L % 64], r["k_codes"][b, g])
            assert np.array_equal(page_rows(r["v_cache"][p, g], "v", kv_dtype)[L % 64], r["v_codes"][b, g])
    changed = (r["k_cache"] != w.k_cache).any(axis=(1, 2))
    assert changed.sum() <= w.batch
    if kv_dtype == "fp8":
        np.testing.assert_array_equal(r["k_codes"], e4m3_encode(r["k_rot"] / w.k_scale[None, :, None]))
    # the rotated query keeps the normalised norm (RoPE is a rotation)
    qn = opro.rms_norm(bf16_to_f64(w.q_new), w.q_norm_w, w.eps)
    np.testing.assert_allclose(np.linalg.norm(r["q_rot"], axis=-1), np.linalg.norm(qn, axis=-1), rtol=1e-12)

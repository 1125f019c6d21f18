"""Pins of the fp64 attention oracle: a library routine, closed forms, invariants."""

import math

import numpy as np
import pytest
import scipy.special
import torch

from load_balanced_split_amd import inputs
from oracle import attention as oa
from oracle.formats import bf16_to_f64, e4m3_to_f64
from oracle.kv_layout import page_rows

D = 128
SCALE = 1.0 / math.sqrt(D)


def paged_from_contiguous(Ks, Vs, rng, extra_pages=3, dtype=np.uint16):
    """Test-side scatter of contiguous per-request K/V codes [Hkv, L, D] into pages,
    then into the cache's tiled in-page order (the input generator's tiling)."""
    hkv = Ks[0].shape[0]
    npages = [(k.shape[1] + 63) // 64 for k in Ks]
    P = sum(npages) + extra_pages
    perm = rng.permutation(P)
    kc = np.zeros((P, hkv, 64, D), dtype)
    vc = np.zeros((P, hkv, 64, D), dtype)
    pt = np.full((len(Ks), max(1, max(npages))), -1, np.int32)
    off = 0
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        for t in range(npages[b]):
            p = perm[off]
            off += 1
            pt[b, t] = p
            rows = K[:, t * 64:(t + 1) * 64, :]
            kc[p, :, :rows.shape[1], :] = rows
            vc[p, :, :rows.shape[1], :] = V[:, t * 64:(t + 1) * 64, :]
    kv_dtype = "bf16" if dtype == np.uint16 else "fp8"
    return inputs.tile_k(kc, kv_dtype), inputs.tile_v(vc, kv_dtype), pt


def sdpa(q, K, V, scale):
    """torch's scaled_dot_product_attention, fp64, one request: q [Hq, D], K/V [Hkv, L, D]."""
    hq, hkv = q.shape[0], K.shape[0]
    G = hq // hkv
    kt = torch.from_numpy(np.repeat(K, G, axis=0))
    vt = torch.from_numpy(np.repeat(V, G, axis=0))
    qt = torch.from_numpy(q)[:, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :].numpy()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_matches_torch_sdpa(seed, kv_dtype):
    rng = np.random.default_rng(100 + seed)
    hkv, G = 2, 4
    lens = [1, 63, 64, 65, 130, int(rng.integers(1, 300))]
    qb = inputs.bf16_bits(rng.standard_normal((len(lens), hkv * G, D)).astype(np.float32))
    if kv_dtype == "bf16":
        Ks = [inputs.bf16_bits(rng.standard_normal((hkv, L, D)).astype(np.float32)) for L in lens]
        Vs = [inputs.bf16_bits(rng.standard_normal((hkv, L, D)).astype(np.float32)) for L in lens]
        ks = vs = None
        dec = lambda c, s: bf16_to_f64(c)
        kc, vc, pt = paged_from_contiguous(Ks, Vs, rng)
    else:
        Ks = [rng.integers(0, 256, (hkv, L, D)).astype(np.uint8) for L in lens]
        Vs = [rng.integers(0, 256, (hkv, L, D)).astype(np.uint8) for L in lens]
        for arr in Ks + Vs:                       # no NaN codes in live tokens
            arr[(arr & 0x7F) == 0x7F] = 0x7E
        ks = np.array([0.01, 0.02], np.float32)
        vs = np.array([0.03, 0.005], np.float32)
        dec = lambda c, s: e4m3_to_f64(c) * s[:, None, None].astype(np.float64)
        kc, vc, pt = paged_from_contiguous(Ks, Vs, rng, dtype=np.uint8)
    out = oa.decode_attention(qb, kc, vc, np.array(lens, np.int32), pt, hkv, SCALE, kv_dtype, ks, vs)
    for b, L in enumerate(lens):
        ref = sdpa(bf16_to_f64(qb[b]), dec(Ks[b], ks), dec(Vs[b], vs), SCALE)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_oracle_tiny_workload_matches_sdpa():
    w = inputs.config_workload(0)
    out = oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, 1, w.sm_scale)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        pages = w.page_table[b, :(L + 63) // 64]
        K = np.concatenate([bf16_to_f64(page_rows(w.k_cache[p, 0], "k", "bf16")) for p in pages])[:L][None]
        V = np.concatenate([bf16_to_f64(page_rows(w.v_cache[p, 0], "v", "bf16")) for p in pages])[:L][None]
        np.testing.assert_allclose(out[b], sdpa(bf16_to_f64(w.q[b]), K, V, w.sm_scale), rtol=1e-12, atol=1e-13)


def _one(q, K, V):
    rng = np.random.default_rng(0)
    kc, vc, pt = paged_from_contiguous([inputs.bf16_bits(K[None].astype(np.float32))],
                                       [inputs.bf16_bits(V[None].astype(np.float32))], rng)
    qb = inputs.bf16_bits(q[None, None].astype(np.float32))
    return oa.decode_attention(qb, kc, vc, np.array([K.shape[0]], np.int32), pt, 1, SCALE)[0, 0]


def _bf(x):
    return bf16_to_f64(inputs.bf16_bits(np.asarray(x, np.float32)))


def test_single_token_returns_v0():
    rng = np.random.default_rng(3)
    K, V, q = _bf(rng.standard_normal((1, D))), _bf(rng.standard_normal((1, D))), _bf(rng.standard_normal(D))
    assert np.array_equal(_one(q, K, V), V[0])


def test_zero_query_gives_mean_of_live_rows():
    rng = np.random.default_rng(4)
    for L in (2, 64, 77, 200):
        K, V = _bf(rng.standard_normal((L, D))), _bf(rng.standard_normal((L, D)))
        np.testing.assert_allclose(_one(np.zeros(D), K, V), V.mean(axis=0), rtol=0, atol=1e-14)


def test_constant_v_returns_it():
    rng = np.random.default_rng(5)
    u = _bf(rng.standard_normal(D))
    for L in (1, 65, 300):
        K = _bf(rng.standard_normal((L, D)))
        np.testing.assert_allclose(_one(_bf(rng.standard_normal(D)), K, np.tile(u, (L, 1))), u, rtol=1e-14, atol=1e-15)


def test_one_hot_v_gives_scipy_softmax_row():
    rng = np.random.default_rng(6)
    for L in (3, 64, 100, 128):
        K, q = _bf(rng.standard_normal((L, D))), _bf(rng.standard_normal(D))
        V = np.eye(D)[:L]
        out = _one(q, K, V)
        np.testing.assert_allclose(out[:L], scipy.special.softmax(SCALE * (K @ q)), rtol=1e-12, atol=1e-15)
        assert np.all(out[L:] == 0)
        assert abs(out.sum() - 1.0) < 1e-12


def test_two_tokens_logistic_weights():
    rng = np.random.default_rng(7)
    K, V, q = _bf(rng.standard_normal((2, D))), _bf(rng.standard_normal((2, D))), _bf(rng.standard_normal(D))
    z0, z1 = SCALE * K @ q
    want = scipy.special.expit(z0 - z1) * V[0] + scipy.special.expit(z1 - z0) * V[1]
    np.testing.assert_allclose(_one(q, K, V), want, rtol=1e-13, atol=1e-14)


def test_huge_logits_pick_argmax_row_without_overflow():
    rng = np.random.default_rng(8)
    L = 150
    K, V = _bf(rng.standard_normal((L, D))), _bf(rng.standard_normal((L, D)))
    q = _bf(rng.standard_normal(D) * 1e3)
    K[17] = np.sign(q)                         # row 17 leads every other logit by thousands
    out = _one(q, K, V)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, V[np.argmax(K @ q)], rtol=1e-6, atol=1e-6)


def test_physical_page_permutation_is_bit_identical():
    w = inputs.build_workload("t", [5, 64, 129, 300, 0, 1], 8, 2, "bf16", seed=9, pool_pages=30)
    out = oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, 2, w.sm_scale)
    perm = np.random.default_rng(10).permutation(w.num_pages)
    kc = np.empty_like(w.k_cache)
    vc = np.empty_like(w.v_cache)
    kc[perm] = w.k_cache
    vc[perm] = w.v_cache
    pt = np.where(w.page_table >= 0, perm[np.maximum(w.page_table, 0)], -1).astype(np.int32)
    out2 = oa.decode_attention(w.q, kc, vc, w.seq_lens, pt, 2, w.sm_scale)
    assert np.array_equal(out, out2)
    assert np.all(out[4] == 0)                  # empty request -> zero row


def test_query_head_permutation_within_group_permutes_output():
    w = inputs.build_workload("t", [70, 200], 8, 2, "bf16", seed=11)
    out = oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, 2, w.sm_scale)
    perm = np.concatenate([np.random.default_rng(12).permutation(4), 4 + np.random.default_rng(13).permutation(4)])
    out2 = oa.decode_attention(w.q[:, perm], w.k_cache, w.v_cache, w.seq_lens, w.page_table, 2, w.sm_scale)
    assert np.array_equal(out[:, perm], out2)


def test_split_then_merge_equals_unsplit():
    rng = np.random.default_rng(14)
    for trial in range(20):
        L = int(rng.integers(2, 700))
        K, V, q = rng.standard_normal((L, D)), rng.standard_normal((L, D)), rng.standard_normal(D) * 3
        cuts = np.sort(rng.choice(np.arange(1, L), size=min(L - 1, int(rng.integers(1, 9))), replace=False))
        bounds = [0, *cuts.tolist(), L]
        states = [oa.partial_state(q, K[a:b], V[a:b], SCALE) for a, b in zip(bounds[:-1], bounds[1:])]
        np.testing.assert_allclose(oa.lse_combine(states), oa.softmax_attention(q, K, V, SCALE), rtol=1e-12, atol=1e-13)

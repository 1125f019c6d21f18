"""The seeded generators: shapes, seed-0 lengths, page tables, poison."""

import numpy as np

from load_balanced_split_amd import inputs
from oracle.kv_layout import page_rows


def test_seed0_lengths():
    l3 = inputs.config_lengths_only(3)
    assert (l3.sum(), l3.min(), l3.max()) == (572570, 1036, 64780)
    l4 = inputs.config_lengths_only(4)
    assert ((l4 + 1).sum(), l4.min(), l4.max()) == (1702440, 801, 60676)
    assert int(((l4 + 1 + 63) // 64).sum()) == 26660


def test_tiny_layout_and_determinism():
    w = inputs.config_workload(0)
    w2 = inputs.config_workload(0)
    assert np.array_equal(w.k_cache, w2.k_cache) and np.array_equal(w.page_table, w2.page_table)
    assert w.k_cache.shape == (16, 1, 8192) and w.v_cache.shape == (16, 1, 8192)
    assert w.page_table.shape == (4, 9)
    used = w.page_table[w.page_table >= 0]
    assert len(used) == 15 and len(set(used.tolist())) == 15
    assert w.kv_bytes() == 416768


def test_poison_marks_only_unreadable_slots():
    w = inputs.build_workload("p", [37, 64, 0, 129], 8, 1, "bf16", seed=1, pool_pages=8, poison=True)
    nan = w.k_cache == inputs.BF16_NAN
    vnan = w.v_cache == inputs.BF16_NAN
    for b, L in enumerate(w.seq_lens):
        for t in range((L + 63) // 64):
            p = w.page_table[b, t]
            n = min(64, L - 64 * t)
            for g in range(w.hkv):
                kr = page_rows(nan[p, g], "k", "bf16")
                vr = page_rows(vnan[p, g], "v", "bf16")
                assert not kr[:n].any() and kr[n:].all()
                assert not vr[:n].any() and vr[n:].all()
    used = set(w.page_table[w.page_table >= 0].tolist())
    for p in range(w.num_pages):
        if p not in used:
            assert nan[p].all() and vnan[p].all()


def test_fp8_scales_cover_pool():
    w = inputs.build_workload("f", [100, 700], 8, 2, "fp8", seed=2, prologue=True)
    assert w.k_cache.dtype == np.uint8 and w.k_scale.shape == (2,)
    assert (w.k_cache & 0x7F).max() <= 0x7E            # no NaN codes, 448 reached
    assert ((w.k_cache & 0x7F) == 0x7E).any()
    assert w.page_table[1, 700 // 64] >= 0              # page for the appended token exists


def test_untile_undoes_tile_and_matches_the_layout_formulas():
    """untile_k / untile_v (the row-major pages a caller of hpa_kv_pack_pages holds)
    invert tile_k / tile_v, and agree with the element-by-element layout decoder."""
    from oracle.kv_layout import page_rows
    rng = np.random.default_rng(3)
    for dt, top, dtype in (("bf16", 65535, np.uint16), ("fp8", 255, np.uint8)):
        x = rng.integers(0, top, size=(3, 2, 64, 128)).astype(dtype)
        for tile, untile, kind in ((inputs.tile_k, inputs.untile_k, "k"), (inputs.tile_v, inputs.untile_v, "v")):
            y = tile(x, dt)
            assert np.array_equal(untile(y, dt), x)
            for p in range(3):
                for g in range(2):
                    assert np.array_equal(page_rows(y[p, g], kind, dt), x[p, g])

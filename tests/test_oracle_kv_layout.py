"""Pins of the cache's in-page order (oracle.kv_layout): hand-worked indices, bijection,
and agreement with the input generator's reshape form of the same order."""

import json
import os

import numpy as np
import pytest

from load_balanced_split_amd import inputs
from oracle import kv_layout as kl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_hand_worked_indices(kv_dtype):
    g = json.load(open(os.path.join(GOLDEN, "kv_layout_indices.json")))[kv_dtype]
    for kind, f in (("k", kl.k_index), ("v", kl.v_index)):
        for t, d, idx in g[kind]:
            assert f(t, d, kv_dtype) == idx, (kind, t, d)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_bijection(kv_dtype, kind):
    tab = kl.index_table(kind, kv_dtype)
    assert sorted(tab.ravel().tolist()) == list(range(64 * 128))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_generator_tiling_matches(kv_dtype):
    rng = np.random.default_rng(3)
    x = rng.integers(0, 60000, size=(3, 2, 64, 128)).astype(np.uint16)
    for kind, tile in (("k", inputs.tile_k), ("v", inputs.tile_v)):
        y = tile(x, kv_dtype)
        assert y.shape == (3, 2, 8192)
        for p in range(3):
            for g in range(2):
                assert np.array_equal(kl.page_rows(y[p, g], kind, kv_dtype), x[p, g])


def test_load_structure_bf16():
    """Each 1 KB load (512 bf16) of K holds, for lane l = 16j + m, 8 consecutive dims
    of one token; the 4 lanes of one m hold 4 consecutive 8-dim pieces (one MFMA
    k-chunk of 32 dims), and one load covers 16 tokens."""
    tab = kl.index_table("k", "bf16")
    where = {int(tab[t, d]): (t, d) for t in range(64) for d in range(128)}
    for load in range(16):
        toks = set()
        for lane in range(64):
            elems = [where[load * 512 + lane * 8 + e] for e in range(8)]
            t0, d0 = elems[0]
            assert all(t == t0 for t, _ in elems) and [d for _, d in elems] == list(range(d0, d0 + 8))
            toks.add(t0)
            m, j = lane % 16, lane // 16
            tm, dm = where[load * 512 + m * 8]
            assert t0 == tm and d0 == dm + 8 * j
        assert len(toks) == 16

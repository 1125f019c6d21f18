"""Where a (token, dim) element of a KV page sits in the library's cache format.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages only say the KV cache is paged (openai-hub.com "腾讯混元HPC-Ops升级：
五大算子直击推理痛点", section "五大算子覆盖了哪些场景"); the in-page order is
the library's own, documented in its C header: every (page, KV head) block holds
64 tokens x 128 dims, and element (t, d) sits at the index below. This module
writes that definition out element by element; it never calls the input
generator's tiling, which expresses the same order as array reshapes.

    bf16 K:  r = t mod 32 = 8a + 4b + q,  d = 32c + 8j + e
             index = 4096 * (t div 32) + 512 * (4b + c) + 8 * (16j + 4a + q) + e
    bf16 V:  r = t mod 32 = 8j + e,       d = 16n + m
             index = 4096 * (t div 32) + 512 * n + 8 * (16j + m) + e
    E4M3 K:  t = 16a + 4b + q,            d = 64p + 16j + e
             index = 1024 * (2b + p) + 16 * (16j + 4a + q) + e
    E4M3 V:  t = 16j + e,                 d = 16n + m
             index = 1024 * n + 16 * (16j + m) + e

Pins (tests/test_oracle_kv_layout.py): hand-worked indices
(tests/golden/kv_layout_indices.json); each map is a bijection onto 0..8191;
round trip against the input generator's independent reshape form.
"""

import numpy as np

PAGE = 64
HEAD_DIM = 128


def k_index(t, d, kv_dtype):
    if kv_dtype == "bf16":
        r = t % 32
        a, b, q = r // 8, (r // 4) % 2, r % 4
        c, j, e = d // 32, (d // 8) % 4, d % 8
        return 4096 * (t // 32) + 512 * (4 * b + c) + 8 * (16 * j + 4 * a + q) + e
    a, b, q = t // 16, (t // 4) % 4, t % 4
    p, j, e = d // 64, (d // 16) % 4, d % 16
    return 1024 * (2 * b + p) + 16 * (16 * j + 4 * a + q) + e


def v_index(t, d, kv_dtype):
    if kv_dtype == "bf16":
        r = t % 32
        j, e = r // 8, r % 8
        n, m = d // 16, d % 16
        return 4096 * (t // 32) + 512 * n + 8 * (16 * j + m) + e
    j, e = t // 16, t % 16
    n, m = d // 16, d % 16
    return 1024 * n + 16 * (16 * j + m) + e


_TABLES = {}


def index_table(kind, kv_dtype):
    """int64 [64, 128]: block index of every (token, dim), by the formulas above."""
    key = (kind, kv_dtype)
    if key not in _TABLES:
        f = k_index if kind == "k" else v_index
        tab = np.empty((PAGE, HEAD_DIM), np.int64)
        for t in range(PAGE):
            for d in range(HEAD_DIM):
                tab[t, d] = f(t, d, kv_dtype)
        _TABLES[key] = tab
    return _TABLES[key]


def page_rows(block, kind, kv_dtype):
    """One stored block [8192] -> its logical [64 tokens, 128 dims] array."""
    return np.asarray(block)[index_table(kind, kv_dtype)]

"""Exact paged decode attention in fp64: gather the pages, then a two-pass softmax.

TEST INFRASTRUCTURE ONLY (see the package header).

What is computed (the plain definition the load-balanced kernel must reach up
to rounding order; the pages speak of split-KV decode attention over a paged
KV cache -- xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
"为什么 batch 越大，数字越漂亮"; openai-hub.com "腾讯混元HPC-Ops升级：五大算子直击
推理痛点", section "五大算子覆盖了哪些场景", the paged varlen call):

For request b, query head h, KV head g = h // (Hq/Hkv) and token j < L_b,
page p = page_table[b, j // 64], slot r = j % 64:
    K_j = row r of block k_cache[p, g]   V_j = row r of block v_cache[p, g]
    (blocks decoded by kv_layout; fp8: code value * scale_g)
    z_j = sm_scale * <q[b,h], K_j>,  m = max_j z_j,  w_j = exp(z_j - m)
    out[b,h] = sum_j w_j V_j / sum_j w_j;  L_b == 0 gives a zero row.

The split-KV decomposition the method relies on (never printed on the pages; it
is the only exact way to combine softmax over disjoint token ranges): each
range yields (acc = sum w_j V_j, m, l = sum w_j) relative to its own max, and
ranges combine by rescaling with exp(m_k - M), M = max_k m_k.

Parity pins (tests/test_oracle_attention.py): PyTorch's
scaled_dot_product_attention in fp64 on the unpaged tensors; closed forms
(L=1 -> V_0; q=0 -> mean of V; constant V -> that vector; one-hot V -> scipy's
softmax row; two tokens -> logistic weights; huge logits -> V_argmax);
invariants (physical page permutation bit-identical; permuting query heads
within a group permutes outputs; split-then-merge equals unsplit to 1e-12).
"""

import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64
from .kv_layout import HEAD_DIM, page_rows

PAGE = 64


def decode_kv(codes, kv_dtype, scale=None):
    if kv_dtype == "bf16":
        return bf16_to_f64(codes)
    return e4m3_to_f64(codes) * float(scale)


def gather_kv(k_cache, v_cache, page_table, b, g, L, kv_dtype, k_scale=None, v_scale=None):
    """Contiguous fp64 K [L, D] and V [L, D] of request b, KV head g."""
    D = HEAD_DIM
    K = np.empty((L, D))
    V = np.empty((L, D))
    for j0 in range(0, L, PAGE):
        n = min(PAGE, L - j0)
        p = int(page_table[b, j0 // PAGE])
        K[j0:j0 + n] = decode_kv(page_rows(k_cache[p, g], "k", kv_dtype)[:n], kv_dtype,
                                 None if k_scale is None else k_scale[g])
        V[j0:j0 + n] = decode_kv(page_rows(v_cache[p, g], "v", kv_dtype)[:n], kv_dtype,
                                 None if v_scale is None else v_scale[g])
    return K, V


def softmax_attention(qh, K, V, sm_scale):
    """One query row over contiguous K, V (two passes: max, then weights)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = sm_scale * (K @ qh)
    m = z.max()
    w = np.exp(z - m)
    return (w @ V) / w.sum()


def decode_attention(q, k_cache, v_cache, seq_lens, page_table, hkv, sm_scale,
                     kv_dtype="bf16", k_scale=None, v_scale=None):
    """fp64 out [B, Hq, D]. ``q`` is bf16 bits (uint16) or already fp64."""
    qf = bf16_to_f64(q) if q.dtype == np.uint16 else np.asarray(q, np.float64)
    B, Hq, D = qf.shape
    G = Hq // hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(hkv):
            K, V = gather_kv(k_cache, v_cache, page_table, b, g, L, kv_dtype, k_scale, v_scale)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = softmax_attention(qf[b, h], K, V, sm_scale)
    return out


def partial_state(qh, K, V, sm_scale):
    """(acc, m, l) of one token range: acc = sum_j e^(z_j - m) V_j, l = sum_j e^(z_j - m)."""
    z = sm_scale * (K @ qh)
    m = z.max()
    w = np.exp(z - m)
    return w @ V, m, w.sum()


def lse_combine(states):
    """Combine partial states in the given order; returns the normalised output row."""
    M = max(m for _, m, _ in states)
    acc = sum(np.exp(m - M) * a for a, m, _ in states)
    l = sum(np.exp(m - M) * s for _, m, s in states)
    return acc / l

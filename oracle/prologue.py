"""Fused decode prologue in fp64: q/k RMSNorm, rotate-half RoPE, quantise, paged append.

TEST INFRASTRUCTURE ONLY (see the package header).

bitbyai.com "vLLM × HPC-Ops: High-Performance Attention and MoE Backends from
Tencent Hunyuan", section "Breaking Down the Kernels": the attention backend
folds RoPE, query-key normalisation and the KV write into one prologue ahead of
attention. The pages give no formulas; the readings taken are:

* RMSNorm (Zhang & Sennrich 2019) per head row of D = 128:
  y = x / sqrt(mean(x^2) + eps) * w, one weight vector [D] for all q heads and
  one for all k heads; v is not normalised. Normalise first, then rotate.
* RoPE (Su et al., RoFormer, 2021) in the rotate-half pairing (i, i + 64):
  f_i = theta^(-2i/D), angle = pos * f_i, pos = the request's live length
  before the append (0-based index of the new token).
* KV write: the new k (after norm and RoPE) and v land in slot pos % 64 of
  page page_table[b, pos // 64]; an fp8 cache stores round-to-nearest-even,
  saturating E4M3 codes of value / scale_g with the cache's existing per-head
  scale; a bf16 cache stores the round-to-nearest-even bf16 value.
* attention then covers L_b + 1 tokens and reads q as the fp64 rotated q.

Parity pins (tests/test_oracle_prologue.py): PyTorch's rms_norm in fp64;
RMSNorm of a constant vector in closed form; RoPE against the complex-number
form (x_i + i x_{i+64}) * exp(i * angle); pos 0 identity; norm preservation;
relative-position invariance of <RoPE_m q, RoPE_n k>; a unit vector's closed
form; the E4M3 encoder's own pins (formats).
"""

import numpy as np

from .formats import bf16_to_f64, e4m3_encode
from .kv_layout import index_table

PAGE = 64


def rms_norm(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def rope_rotate_half(x, pos, theta):
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    inv_freq = np.power(float(theta), -2.0 * np.arange(half) / D)
    ang = np.asarray(pos, np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def bf16_encode(x):
    """fp64 -> nearest bf16 bit pattern, ties to even (normal range only)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def prologue(w):
    """Apply the prologue to a workload (read-only); returns a dict with
    q_rot (fp64 [B,Hq,D]), k_rot (fp64 [B,Hkv,D]), k_codes / v_codes (what is
    written for each request and KV head), the updated caches and lengths."""
    B, Hq, Hkv = w.batch, w.hq, w.hkv
    pos = w.seq_lens.astype(np.int64)
    qn = rms_norm(bf16_to_f64(w.q_new), w.q_norm_w, w.eps)
    kn = rms_norm(bf16_to_f64(w.k_new), w.k_norm_w, w.eps)
    q_rot = rope_rotate_half(qn, pos[:, None], w.rope_theta)
    k_rot = rope_rotate_half(kn, pos[:, None], w.rope_theta)
    v = bf16_to_f64(w.v_new)
    if w.kv_dtype == "fp8":
        k_codes = e4m3_encode(k_rot / w.k_scale[None, :, None].astype(np.float64))
        v_codes = e4m3_encode(v / w.v_scale[None, :, None].astype(np.float64))
    else:
        k_codes = bf16_encode(k_rot)
        v_codes = bf16_encode(v)
    k_cache = w.k_cache.copy()
    v_cache = w.v_cache.copy()
    kt, vt = index_table("k", w.kv_dtype), index_table("v", w.kv_dtype)
    for b in range(B):
        p = int(w.page_table[b, pos[b] // PAGE])
        r = int(pos[b] % PAGE)
        k_cache[p][:, kt[r]] = k_codes[b]
        v_cache[p][:, vt[r]] = v_codes[b]
    return dict(q_rot=q_rot, k_rot=k_rot, k_codes=k_codes, v_codes=v_codes,
                k_cache=k_cache, v_cache=v_cache, seq_lens=(pos + 1).astype(np.int32))

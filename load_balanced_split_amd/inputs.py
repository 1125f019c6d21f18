"""Seeded synthetic inputs for paged decode attention (and for the router GEMM:
``router_workload`` at the end).

This module only draws random numbers and lays them out in the cache formats the
library consumes. It holds none of the attention, softmax, planning, RMSNorm or
rotary arithmetic; both the HIP path and the fp64 oracle read what it produces.
Value encodings (fp32 -> bf16, fp32 -> OCP E4M3) are delegated to PyTorch's own
dtype casts, so no rounding rule is restated here.

Layouts (little-endian bit patterns held in numpy integer arrays):

* ``q``        uint16 bf16 bits, ``[B, Hq, D]``
* ``k_cache``, ``v_cache``  ``[num_pages, Hkv, 64 * D]``: one block of 64 tokens
  x 128 dims per (page, KV head), in the library's tiled in-page order (see
  ``tile_k`` / ``tile_v``); uint16 bf16 bits, or uint8 OCP E4M3 codes with
  per-KV-head fp32 scales
* ``page_table`` int32 ``[B, max_pages]``; entries past a request's pages are -1
* ``seq_lens`` int32 ``[B]`` live KV length of each request (for workloads with
  the fused prologue: the length before the new token is appended)

Draw order for one workload (one fresh ``numpy.random.default_rng(seed)``):
lengths (one vectorised call of size B, when drawn) -> page permutation -> q ->
K -> V -> (new q, new k, new v, q-norm weight, k-norm weight). K and V are drawn
in their logical [page, head, token, dim] shape, in chunks of ``_CHUNK_PAGES``
pages, as standard normal float32, and tiled after encoding.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAGE = 64
HEAD_DIM = 128
_CHUNK_PAGES = 1024
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
E4M3_MAX = 448.0


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    kv_dtype: str                  # "bf16" or "fp8"
    seq_lens: np.ndarray           # int32 [B]
    page_table: np.ndarray         # int32 [B, max_pages]
    num_pages: int
    q: np.ndarray                  # uint16 [B, Hq, D]
    k_cache: np.ndarray            # uint16|uint8 [P, Hkv, 64 * D], tiled (tile_k)
    v_cache: np.ndarray            # uint16|uint8 [P, Hkv, 64 * D], tiled (tile_v)
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray] = None
    sm_scale: float = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))
    # fused-prologue inputs (None when the workload has no prologue)
    q_new: Optional[np.ndarray] = None     # uint16 [B, Hq, D]
    k_new: Optional[np.ndarray] = None     # uint16 [B, Hkv, D]
    v_new: Optional[np.ndarray] = None     # uint16 [B, Hkv, D]
    q_norm_w: Optional[np.ndarray] = None  # float32 [D]
    k_norm_w: Optional[np.ndarray] = None  # float32 [D]
    eps: float = 1e-6
    rope_theta: float = 1e6
    seed: int = 0

    @property
    def head_dim(self) -> int:
        return HEAD_DIM

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def has_prologue(self) -> bool:
        return self.q_new is not None

    def attended_lens(self) -> np.ndarray:
        """Tokens attention covers: the live length, plus one when a token is appended."""
        return self.seq_lens + (1 if self.has_prologue else 0)

    def kv_bytes(self) -> int:
        """Bytes of valid K and V tokens (padding rows excluded)."""
        e = 2 if self.kv_dtype == "bf16" else 1
        return int(self.attended_lens().astype(np.int64).sum()) * self.hkv * 2 * HEAD_DIM * e


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (PyTorch's round-to-nearest-even cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 already within [-448, 448] -> OCP E4M3 codes (PyTorch's float8_e4m3fn cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.clip(x, -E4M3_MAX, E4M3_MAX), dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# --- the tiled in-page order -------------------------------------------------
# A page block X[t, d] (64 tokens x 128 dims) is stored as a reordering of its
# elements: split t and d into digit groups and permute the groups. Token and
# dim digits (most significant first):
#   bf16 K:  t -> (h:2, a:4, b:2, q:4), d -> (c:4, j:4, e:8); stored as (h, b, c, j, a, q, e)
#   bf16 V:  t -> (h:2, j:4, e:8),      d -> (n:8, m:16);     stored as (h, n, j, m, e)
#   E4M3 K:  t -> (a:4, b:4, q:4),      d -> (p:2, j:4, e:16); stored as (b, p, j, a, q, e)
#   E4M3 V:  t -> (j:4, e:16),          d -> (n:8, m:16);     stored as (n, j, m, e)

def tile_k(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """[..., 64, 128] logical K pages -> [..., 8192] in the tiled order."""
    lead = x.shape[:-2]
    k = len(lead)
    if kv_dtype == "bf16":
        y = x.reshape(*lead, 2, 4, 2, 4, 4, 4, 8)
        perm = (0, 2, 4, 5, 1, 3, 6)
    else:
        y = x.reshape(*lead, 4, 4, 4, 2, 4, 16)
        perm = (1, 3, 4, 0, 2, 5)
    y = y.transpose(*range(k), *(k + i for i in perm))
    return np.ascontiguousarray(y).reshape(*lead, PAGE * HEAD_DIM)


def tile_v(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """[..., 64, 128] logical V pages -> [..., 8192] in the tiled order."""
    lead = x.shape[:-2]
    k = len(lead)
    if kv_dtype == "bf16":
        y = x.reshape(*lead, 2, 4, 8, 8, 16)
        perm = (0, 3, 1, 4, 2)
    else:
        y = x.reshape(*lead, 4, 16, 8, 16)
        perm = (2, 0, 3, 1)
    y = y.transpose(*range(k), *(k + i for i in perm))
    return np.ascontiguousarray(y).reshape(*lead, PAGE * HEAD_DIM)


def _untile(y: np.ndarray, shape, perm) -> np.ndarray:
    lead = y.shape[:-1]
    k = len(lead)
    stored = [shape[i] for i in perm]
    x = y.reshape(*lead, *stored)
    inv = [perm.index(i) for i in range(len(perm))]
    x = x.transpose(*range(k), *(k + i for i in inv))
    return np.ascontiguousarray(x).reshape(*lead, PAGE, HEAD_DIM)


def untile_k(y: np.ndarray, kv_dtype: str) -> np.ndarray:
    """[..., 8192] tiled K blocks -> [..., 64, 128] logical (row-major) pages: tile_k undone."""
    if kv_dtype == "bf16":
        return _untile(y, (2, 4, 2, 4, 4, 4, 8), (0, 2, 4, 5, 1, 3, 6))
    return _untile(y, (4, 4, 4, 2, 4, 16), (1, 3, 4, 0, 2, 5))


def untile_v(y: np.ndarray, kv_dtype: str) -> np.ndarray:
    """[..., 8192] tiled V blocks -> [..., 64, 128] logical (row-major) pages: tile_v undone."""
    if kv_dtype == "bf16":
        return _untile(y, (2, 4, 8, 8, 16), (0, 3, 1, 4, 2))
    return _untile(y, (4, 16, 8, 16), (2, 0, 3, 1))


def _draw_pool(rng, num_pages, hkv):
    """Standard normal float32 [num_pages, hkv, 64, D], drawn in page chunks."""
    out = np.empty((num_pages, hkv, PAGE, HEAD_DIM), np.float32)
    for p0 in range(0, num_pages, _CHUNK_PAGES):
        n = min(_CHUNK_PAGES, num_pages - p0)
        out[p0:p0 + n] = rng.standard_normal((n, hkv, PAGE, HEAD_DIM), dtype=np.float32)
    return out


def _draw_pool_bf16(rng, num_pages, hkv, tile):
    out = np.empty((num_pages, hkv, PAGE * HEAD_DIM), np.uint16)
    for p0 in range(0, num_pages, _CHUNK_PAGES):
        n = min(_CHUNK_PAGES, num_pages - p0)
        x = rng.standard_normal((n, hkv, PAGE, HEAD_DIM), dtype=np.float32)
        out[p0:p0 + n] = tile(bf16_bits(x), "bf16")
    return out


def build_workload(name: str, seq_lens, hq: int, hkv: int, kv_dtype: str = "bf16",
                   seed: int = 0, rng=None, pool_pages: Optional[int] = None,
                   poison: bool = False, prologue: bool = False) -> Workload:
    """Lay out a paged KV cache for the given live lengths.

    ``rng`` continues an existing generator (lengths already drawn from it);
    otherwise a fresh ``default_rng(seed)`` is used. Pages are handed to requests
    in request order from one random permutation of the pool. With
    ``prologue=True`` every request also owns the page its new token lands in.
    With ``poison=True`` every padding slot and unused page holds NaN.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = int(seq_lens.shape[0])
    assert kv_dtype in ("bf16", "fp8")
    assert hq % hkv == 0
    owned = seq_lens + (1 if prologue else 0)
    npages = (owned + PAGE - 1) // PAGE
    used = int(npages.sum())
    num_pages = used if pool_pages is None else int(pool_pages)
    assert num_pages >= used
    max_pages = max(1, int(npages.max()) if B else 1)

    perm = rng.permutation(num_pages).astype(np.int32)
    page_table = np.full((B, max_pages), -1, np.int32)
    off = 0
    for b in range(B):
        n = int(npages[b])
        page_table[b, :n] = perm[off:off + n]
        off += n

    q = bf16_bits(rng.standard_normal((B, hq, HEAD_DIM), dtype=np.float32))
    k_scale = v_scale = None
    if kv_dtype == "bf16":
        k_cache = _draw_pool_bf16(rng, num_pages, hkv, tile_k)
        v_cache = _draw_pool_bf16(rng, num_pages, hkv, tile_v)
    else:
        kf = _draw_pool(rng, num_pages, hkv)
        vf = _draw_pool(rng, num_pages, hkv)
        # one scale per KV head, fixed when the cache is built: amax / 448
        k_scale = (np.abs(kf).max(axis=(0, 2, 3)) / E4M3_MAX).astype(np.float32)
        v_scale = (np.abs(vf).max(axis=(0, 2, 3)) / E4M3_MAX).astype(np.float32)
        k_cache = np.empty((num_pages, hkv, PAGE * HEAD_DIM), np.uint8)
        v_cache = np.empty((num_pages, hkv, PAGE * HEAD_DIM), np.uint8)
        for p0 in range(0, num_pages, _CHUNK_PAGES):
            sl = slice(p0, min(num_pages, p0 + _CHUNK_PAGES))
            k_cache[sl] = tile_k(e4m3_codes(kf[sl] / k_scale[None, :, None, None]), "fp8")
            v_cache[sl] = tile_v(e4m3_codes(vf[sl] / v_scale[None, :, None, None]), "fp8")
        del kf, vf

    w = Workload(name=name, batch=B, hq=hq, hkv=hkv, kv_dtype=kv_dtype,
                 seq_lens=seq_lens.astype(np.int32), page_table=page_table, num_pages=num_pages,
                 q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale, seed=seed)
    if prologue:
        w.q_new = bf16_bits(rng.standard_normal((B, hq, HEAD_DIM), dtype=np.float32))
        w.k_new = bf16_bits(rng.standard_normal((B, hkv, HEAD_DIM), dtype=np.float32))
        w.v_new = bf16_bits(rng.standard_normal((B, hkv, HEAD_DIM), dtype=np.float32))
        w.q_norm_w = rng.uniform(0.5, 1.5, HEAD_DIM).astype(np.float32)
        w.k_norm_w = rng.uniform(0.5, 1.5, HEAD_DIM).astype(np.float32)
    if poison:
        poison_padding(w)
    return w


def poison_padding(w: Workload) -> None:
    """Fill every KV slot no request may read (padding rows, unused pages) with NaN.

    For a workload with a prologue the append slot counts as padding too: the
    prologue must overwrite it before attention reads it.
    """
    nan = BF16_NAN if w.kv_dtype == "bf16" else E4M3_NAN
    used = np.zeros(w.num_pages, bool)
    rows = np.arange(PAGE)[:, None] + np.zeros((1, HEAD_DIM), np.int64)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        n = (L + (1 if w.has_prologue else 0) + PAGE - 1) // PAGE
        pages = w.page_table[b, :n]
        used[pages] = True
        if n == 0:
            continue
        last = int(pages[-1])
        valid_in_last = L - (n - 1) * PAGE       # may be 0..64 (0: new token starts the page)
        if valid_in_last < PAGE:
            pad = rows >= valid_in_last          # logical [64, 128] mask of padding rows
            w.k_cache[last][:, tile_k(pad, w.kv_dtype)] = nan
            w.v_cache[last][:, tile_v(pad, w.kv_dtype)] = nan
    w.k_cache[~used] = nan
    w.v_cache[~used] = nan


# --- the five workloads -----------------------------------------------------

CONFIG_NAMES = {
    0: "tiny: B=4 lens{37,64,200,513} Hq8:Hkv1 D128 page64 bf16, pool 16 pages",
    1: "uniform: B=64 x 512 Hq8:Hkv1 D128 page64 bf16",
    2: "skewed: B=32 1x131072+31x4096 Hq8:Hkv1 D128 page64 bf16",
    3: "mix: B=32 log-uniform[1024,65536] Hq32:Hkv4 D128 page64 bf16",
    4: "fp8+prologue: B=128 lognormal(8192,1)[128,131072] Hq8:Hkv1 D128 page64 e4m3",
}


def config_lengths(index: int, rng) -> np.ndarray:
    if index == 0:
        return np.array([37, 64, 200, 513], np.int64)
    if index == 1:
        return np.full(64, 512, np.int64)
    if index == 2:
        return np.array([131072] + [4096] * 31, np.int64)
    if index == 3:
        u = rng.uniform(math.log(1024), math.log(65536), size=32)
        return np.clip(np.rint(np.exp(u)), 1024, 65536).astype(np.int64)
    if index == 4:
        x = rng.lognormal(mean=math.log(8192), sigma=1.0, size=128)
        return np.clip(np.rint(x), 128, 131072).astype(np.int64)
    raise ValueError(f"no workload {index}")


def config_workload(index: int, seed: int = 0, poison: bool = False) -> Workload:
    rng = np.random.default_rng(seed)
    lens = config_lengths(index, rng)
    if index == 0:
        return build_workload("cfg0_tiny", lens, 8, 1, "bf16", seed, rng, pool_pages=16, poison=poison)
    if index == 1:
        return build_workload("cfg1_uniform", lens, 8, 1, "bf16", seed, rng, poison=poison)
    if index == 2:
        return build_workload("cfg2_skewed", lens, 8, 1, "bf16", seed, rng, poison=poison)
    if index == 3:
        return build_workload("cfg3_mix", lens, 32, 4, "bf16", seed, rng, poison=poison)
    if index == 4:
        return build_workload("cfg4_fp8_prologue", lens, 8, 1, "fp8", seed, rng,
                              poison=poison, prologue=True)
    raise ValueError(index)


def config_lengths_only(index: int, seed: int = 0) -> np.ndarray:
    """The lengths a workload would draw, without building its cache."""
    return config_lengths(index, np.random.default_rng(seed))


# ------------------------------------------------------------------ router ---

@dataclasses.dataclass
class RouterWorkload:
    """Inputs of the split-precision router GEMM: activations x (bf16 bits,
    [tokens, hidden]) and the router weight w (fp32, [experts, hidden])."""
    name: str
    tokens: int
    experts: int
    hidden: int
    x: np.ndarray
    w: np.ndarray


def router_workload(tokens: int, experts: int, hidden: int, seed: int = 0, name: str = "router") -> RouterWorkload:
    """x ~ N(0, 1) rounded to bf16 by PyTorch's cast; w ~ N(0, 1/hidden) in fp32, so
    that logits are of order 1. Draw order: x, then w, from one default_rng(seed)."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((tokens, hidden), dtype=np.float32))
    w = (rng.standard_normal((experts, hidden), dtype=np.float32) / np.float32(math.sqrt(hidden))).astype(np.float32)
    return RouterWorkload(name=name, tokens=tokens, experts=experts, hidden=hidden, x=x, w=w)


# ------------------------------------------------------------------- MoE ---

@dataclasses.dataclass
class MoeWorkload:
    """Inputs of the fused FP8 MoE layer: hidden states x (bf16 bits, [T, H]), the
    routing (expert ids [T, K] int32, weights [T, K] fp32), the expert weights as OCP
    E4M3 codes with one fp32 scale per output channel: W1 [E, 2I, H] (gate rows, then
    up rows) with s1 [E, 2I], W2 [E, H, I] with s2 [E, H]."""
    name: str
    tokens: int
    experts: int
    top_k: int
    hidden: int
    inter: int
    x: np.ndarray
    ids: np.ndarray
    weights: np.ndarray
    w1: np.ndarray
    s1: np.ndarray
    w2: np.ndarray
    s2: np.ndarray

    def weight_bytes_read(self) -> int:
        """Bytes of W1 and W2 codes of the experts some token is routed to."""
        used = np.unique(self.ids[(self.ids >= 0) & (self.ids < self.experts)])
        return int(len(used)) * 3 * self.inter * self.hidden


def _per_row_fp8(rng, rows, cols, std):
    """N(0, std^2) float32 rows -> (E4M3 codes, fp32 scale amax / 448 per row)."""
    f = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    s = (np.abs(f).max(axis=1) / np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_codes(f / s[:, None]), s


def moe_workload(tokens: int, experts: int, top_k: int, hidden: int, inter: int, seed: int = 0,
                 name: str = "moe") -> MoeWorkload:
    """x ~ N(0, 1) -> bf16; routing: per token the top_k of E N(0, 1) logits (distinct
    experts, largest first) with softmax weights over those k; W1 ~ N(0, 1/H), W2 ~ N(0, 1/I),
    each row quantised to E4M3 with scale amax / 448 (PyTorch's casts). Draw order, one
    default_rng(seed): x, logits, then W1 and W2 expert by expert."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((tokens, hidden), dtype=np.float32))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    top = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    ew = np.exp(top - top.max(axis=1, keepdims=True))
    weights = (ew / ew.sum(axis=1, keepdims=True)).astype(np.float32)
    w1 = np.empty((experts, 2 * inter, hidden), np.uint8)
    s1 = np.empty((experts, 2 * inter), np.float32)
    w2 = np.empty((experts, hidden, inter), np.uint8)
    s2 = np.empty((experts, hidden), np.float32)
    for e in range(experts):
        w1[e], s1[e] = _per_row_fp8(rng, 2 * inter, hidden, 1.0 / math.sqrt(hidden))
        w2[e], s2[e] = _per_row_fp8(rng, hidden, inter, 1.0 / math.sqrt(inter))
    return MoeWorkload(name=name, tokens=tokens, experts=experts, top_k=top_k, hidden=hidden, inter=inter,
                       x=x, ids=ids, weights=weights, w1=w1, s1=s1, w2=w2, s2=s2)

"""Split-precision router GEMM in fp64: logits of every token for every expert,
and the top-k experts per token.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: xiaodao.ai, "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
"从实验表走到 SLA，还差一轮负载测试": to keep the router's choice of its top-k
experts intact, the router's fp32 weight is cut into a bf16 high part and a bf16
residual, each goes through its own tensor-core product, and the two results are
summed; the page validates the scheme by its error, by greedy outputs and by
cosine similarity. The same page, section "局部快两倍，整条链只快一点",
gives the kernel's gain on one model's shapes, which are not stated.

The page prints no formula. Readings (each a plain one the passage supports):

* activations x are bf16, [tokens, hidden]; the weight W is fp32, [experts, hidden];
* hi = the bf16 value nearest to W (ties to the even significand), lo = the bf16
  value nearest to W - hi (W - hi is exact in fp32), elementwise;
* logits[t, e] = sum_k x[t, k] hi[e, k] + sum_k x[t, k] lo[e, k] -- each product is
  exact in fp32, the sums are fp32 accumulations; one pass (hi only) is the plain
  bf16 router the split improves on;
* the top-k experts of a token are the k largest logits, equal logits ordered by the
  lower expert index, listed from the largest down;
* the page's checks: the error against the exact fp32-weight logits, the greedy
  choice (top-1 and the whole top-k set) and the cosine similarity of each token's
  logit vector with the exact one.

What the computed logits are held to (``error_bound``): the representation error
sum_k |x_k| |W_k - hi_k - lo_k| (with one pass, |W_k - hi_k|) plus the worst-case
error of any order of fp32 summation of the n = passes * hidden exact products and
a few partial sums, gamma_n * sum_k |x_k| (|hi_k| + |lo_k|) with gamma_n = n u / (1 - n u),
u = 2^-24 (the standard bound for recursive summation in any order).

Parity pins (tests/test_oracle_router.py): the bf16 rounding against PyTorch's
bfloat16 cast and hand-worked ties; the split's closed-form bound |W - hi - lo| <=
2^-16 |W| and its exact cases; integer-valued GEMMs against exact Python integers;
top-k against brute-force sorting with forced ties; the summation bound against
fp32 summation in random orders; the metrics on vectors with known answers.
"""

import numpy as np

BF16_UNIT_ROUNDOFF = 2.0 ** -8      # half the spacing of bf16 significands (8 bits)
FP32_UNIT_ROUNDOFF = 2.0 ** -24


def bf16_values(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their values in fp64 (the upper half of a binary32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def nearest_bf16(a) -> np.ndarray:
    """The bf16 value nearest to each element of `a` (fp32-representable, finite,
    below the bf16 overflow threshold), ties to the even significand; in fp64.

    The two candidates are the bf16 neighbours of a: its binary32 pattern with the
    low 16 bits cleared (towards zero) and the next bf16 away from zero."""
    a64 = np.asarray(a, np.float64)
    a32 = a64.astype(np.float32)
    if not np.array_equal(a32.astype(np.float64), a64, equal_nan=True):
        raise ValueError("nearest_bf16 takes fp32-representable values")
    bits = a32.view(np.uint32)
    toward = bits & np.uint32(0xFFFF0000)
    away = toward + np.uint32(0x10000)
    v_toward = toward.view(np.float32).astype(np.float64)
    v_away = away.view(np.float32).astype(np.float64)
    d_toward = np.abs(a64 - v_toward)
    d_away = np.abs(a64 - v_away)
    toward_even = (toward >> np.uint32(16)) & np.uint32(1) == 0
    pick_toward = (d_toward < d_away) | ((d_toward == d_away) & toward_even)
    out = np.where(pick_toward, v_toward, v_away)
    if not np.all(np.isfinite(out[np.isfinite(a64)])):
        raise ValueError("value beyond the bf16 range")
    return out


def split_weights(w):
    """fp32 weight -> (hi, lo) in fp64, both bf16 values: hi nearest to w, lo nearest
    to the residual w - hi."""
    w64 = np.asarray(w, np.float32).astype(np.float64)
    hi = nearest_bf16(w64)
    lo = nearest_bf16(w64 - hi)          # the residual is exact in fp32
    return hi, lo


def router_logits_exact(x_bits, w) -> np.ndarray:
    """x [T, H] (bf16 bits) times the fp32 weight [E, H] transposed, exactly (fp64
    products of bf16 and fp32 values are exact; the fp64 sum rounds at 2^-53)."""
    return bf16_values(x_bits) @ np.asarray(w, np.float32).astype(np.float64).T


def router_logits_split(x_bits, w, passes: int = 2) -> np.ndarray:
    """What the split method sums before its own fp32 rounding: x hi^T (+ x lo^T), fp64."""
    hi, lo = split_weights(w)
    x = bf16_values(x_bits)
    out = x @ hi.T
    if passes == 2:
        out = out + x @ lo.T
    return out


def error_bound(x_bits, w, passes: int = 2, extra_adds: int = 64) -> np.ndarray:
    """Per-logit bound on |computed - exact| for a computation that forms the exact
    products of x with hi (and lo) and sums them in fp32 in any order, with up to
    `extra_adds` further fp32 additions of partial sums."""
    hi, lo = split_weights(w)
    w64 = np.asarray(w, np.float32).astype(np.float64)
    ax = np.abs(bf16_values(x_bits))
    kept = hi + lo if passes == 2 else hi
    representation = ax @ np.abs(w64 - kept).T
    n = passes * ax.shape[1] + extra_adds
    gamma = n * FP32_UNIT_ROUNDOFF / (1.0 - n * FP32_UNIT_ROUNDOFF)
    magnitude = ax @ (np.abs(hi) + (np.abs(lo) if passes == 2 else 0.0)).T
    return representation + gamma * magnitude


def top_k(logits, k: int):
    """Per row: the k largest values, equal values ordered by the lower index, listed
    from the largest down. Returns (indices int64 [T, k], values [T, k])."""
    v = np.asarray(logits)
    T, E = v.shape
    idx = np.empty((T, k), np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -v[t].astype(np.float64)))   # by -value, then index
        idx[t] = order[:k]
    return idx, np.take_along_axis(v, idx, axis=1)


def topk_valid(chosen, exact, bound) -> np.ndarray:
    """Per row: is `chosen` (k distinct indices) a top-k of `exact` that the error
    bound cannot tell apart from the true one? Holds when every chosen logit, raised
    by its bound, reaches every unchosen logit lowered by its bound."""
    chosen = np.asarray(chosen)
    T, E = exact.shape
    ok = np.zeros(T, bool)
    for t in range(T):
        c = chosen[t]
        if len(set(c.tolist())) != len(c) or c.min() < 0 or c.max() >= E:
            continue
        mask = np.ones(E, bool)
        mask[c] = False
        if not mask.any():
            ok[t] = True
            continue
        lowest_chosen = np.min(exact[t, c] + bound[t, c])
        highest_other = np.max(exact[t, mask] - bound[t, mask])
        ok[t] = lowest_chosen >= highest_other
    return ok


def cosine_rows(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.sum(a * b, axis=1)
    den = np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 1.0)


def page_checks(computed, exact, k: int) -> dict:
    """The page's three checks of a router's logits against the exact ones: the
    error (largest absolute, and largest relative to the row's largest |logit|),
    the greedy choice (fraction of tokens whose top-1 and whose top-k set match)
    and the cosine similarity (smallest over tokens)."""
    computed = np.asarray(computed, np.float64)
    err = np.abs(computed - exact)
    scale = np.maximum(np.max(np.abs(exact), axis=1, keepdims=True), np.finfo(np.float64).tiny)
    ci, _ = top_k(computed, k)
    ei, _ = top_k(exact, k)
    same_set = np.array([set(a.tolist()) == set(b.tolist()) for a, b in zip(ci, ei)])
    return {"max_abs_err": float(err.max()) if err.size else 0.0,
            "max_rel_err": float((err / scale).max()) if err.size else 0.0,
            "top1_match": float(np.mean(ci[:, 0] == ei[:, 0])) if len(ci) else 1.0,
            "topk_set_match": float(np.mean(same_set)) if len(ci) else 1.0,
            "min_cosine": float(cosine_rows(computed, exact).min()) if len(ci) else 1.0}

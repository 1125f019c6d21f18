"""Fused FP8 mixture-of-experts layer for decode batches, in plain numpy.

TEST INFRASTRUCTURE ONLY (see the package header).

What the pipeline computes (xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半",
section "为什么 batch 越大，数字越漂亮", the MoE paragraph: routing index, Gate-Up,
activation with requantisation, Down GEMM and the top-k merge run as one fused
chain with no standalone gather; bitbyai.com "vLLM × HPC-Ops …", section
"Breaking Down the Kernels", MoE backend: token rearrangement, FP8 expert GEMMs,
activation and result gathering in one pipeline):

For token t and each of its k routed experts e = ids[t, k] with weight w[t, k]:

    x8, sx  = quantize(x[t])                           FP8 activations, one scale per token
    g[j]    = sx * s1[e, j] * sum_h dec(x8[h]) dec(W1[e, j, h])     j < 2I (gate: j < I, up: I + i)
    a[i]    = silu(g[i]) * g[I + i],  silu(z) = z / (1 + e^-z)       i < I
    a8, sa  = quantize(a)                              requantised, one scale per (token, k)
    y[n]    = sa * s2[e, n] * sum_i dec(a8[i]) dec(W2[e, n, i])      n < H
    out[t]  = sum over k (in k order) of w[t, k] * y               -> bf16 by the caller

quantize(v) = (codes, s) with s = max|v| / 448 and codes = E4M3(v / s) (nearest,
ties to even, OCP E4M3); a zero vector gives s = 0 and zero codes. dec() is the
exact value of a code. Weights are FP8 codes with one fp32 scale per output
channel (W1: [E, 2I, H] with s1 [E, 2I]; W2: [E, H, I] with s2 [E, H]).

Readings where the pages are silent: SwiGLU (silu(gate) * up) as the
activation, gate rows first in W1; per-token activation scales and
per-output-channel weight scales; the routing (ids, weights) is an input, as in
the pages' illustrative fused_moe call; the k results of a token are summed in
k order. Precision: the token quantisation is defined in fp32 (amax / 448 and
the division rounded to fp32, as the kernel computes it) so that both sides
take the same code decisions; everything after it is fp64 here.

Parity pins (tests/test_oracle_moe.py): the quantiser against PyTorch's
float8_e4m3fn cast and the nearest-value definition; a one-hot token selects
one column of W1 exactly (a transposed operand, a per-column scale or a swapped
gate/up half fails it); a one-hot activation code selects one column of W2
exactly; the activation's closed forms (silu(0) = 0, silu(z) -> z and -> 0);
gate rows driven far negative give a zero layer; token permutation, expert
relabelling, splitting a routing weight over two slots of the same expert and
scaling the weights are the invariants of the composition.
"""

import numpy as np

from .formats import bf16_to_f64, e4m3_encode, e4m3_to_f64

E4M3_MAX = 448.0


def quantize_fp32(v):
    """Rows of v (fp32 values) -> (E4M3 codes, fp32 scale per row): s = amax / 448 and
    v / s both rounded to fp32, then the nearest E4M3 code."""
    v = np.asarray(v, np.float32)
    amax = np.max(np.abs(v), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1))
    q = (v / safe[..., None]).astype(np.float32)
    codes = e4m3_encode(q.astype(np.float64))
    codes = np.where((s > 0)[..., None], codes, np.uint8(0))
    return codes.astype(np.uint8), s


def quantize_f64(v):
    """Rows of v (fp64) -> (E4M3 codes, scale): s = amax / 448, codes of v / s, in fp64."""
    v = np.asarray(v, np.float64)
    s = np.max(np.abs(v), axis=-1) / E4M3_MAX
    safe = np.where(s > 0, s, 1.0)
    codes = e4m3_encode(v / safe[..., None])
    codes = np.where((s > 0)[..., None], codes, np.uint8(0))
    return codes.astype(np.uint8), s


def silu(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):             # e^-z = inf for very negative z: the limit -0
        return z / (1.0 + np.exp(-z))


def gate_up(x8, sx, W1e, s1e):
    """g [2I] of one token for one expert: dequantised token row times dequantised W1 rows."""
    return sx * s1e * (e4m3_to_f64(W1e) @ e4m3_to_f64(x8))


def activation(g):
    I = g.shape[-1] // 2
    return silu(g[..., :I]) * g[..., I:]


def down(a8, sa, W2e, s2e):
    """y [H] of one (token, expert) from its requantised activation."""
    return sa * s2e * (e4m3_to_f64(W2e) @ e4m3_to_f64(a8))


def fused_moe(x_bits, ids, weights, W1, s1, W2, s2, details=False):
    """out [T, H] fp64 (before the bf16 rounding). ids [T, K] int, weights [T, K];
    a pair whose expert id is outside [0, E) contributes nothing. With details, also
    the token codes and scales and the per-pair activations, codes and scales."""
    x = bf16_to_f64(x_bits).astype(np.float32)
    T, K = ids.shape
    E = W1.shape[0]
    H = W2.shape[1]
    x8, sx = quantize_fp32(x)
    out = np.zeros((T, H))
    acts, a8s, sas = {}, {}, {}
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            if not 0 <= e < E:
                continue
            g = gate_up(x8[t], float(sx[t]), W1[e], s1[e].astype(np.float64))
            a = activation(g)
            a8, sa = quantize_f64(a)
            y = down(a8, float(sa), W2[e], s2[e].astype(np.float64))
            out[t] += float(weights[t, k]) * y
            if details:
                acts[(t, k)], a8s[(t, k)], sas[(t, k)] = a, a8, float(sa)
    if details:
        return out, dict(x8=x8, sx=sx, act=acts, act_codes=a8s, act_scale=sas)
    return out

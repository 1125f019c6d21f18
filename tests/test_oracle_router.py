"""Pins of the router-GEMM oracle (oracle/router.py) to things other than itself:
PyTorch's bfloat16 cast, hand-worked rounding ties, the split's closed-form bound
and exact cases, integer GEMMs in exact Python arithmetic, brute-force top-k with
forced ties, fp32 summation in random orders against the error bound, and the
page's checks on inputs with known answers."""

import itertools

import numpy as np
import pytest
import torch

from load_balanced_split_amd import inputs
from oracle import router as orr


def _torch_bf16(a32):
    return torch.from_numpy(np.asarray(a32, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_nearest_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(50000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(50000) * 1e30).astype(np.float32)])
    # exact ties: the low 16 bits are 0x8000, with even and odd kept bits
    tie = ((rng.integers(0x3000, 0x4800, 20000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    a = np.concatenate([a, tie, -tie, np.float32([0.0, -0.0, 1.0, -1.0])])
    assert np.array_equal(orr.nearest_bf16(a), _torch_bf16(a))


def test_nearest_bf16_hand_worked_ties():
    # bf16 keeps 8 significant bits: near 1 the spacing is 2^-7
    assert orr.nearest_bf16(np.float32(1 + 2 ** -8)) == 1.0                     # tie, 1.0 is even
    assert orr.nearest_bf16(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6         # tie, 1 + 2^-7 is odd
    assert orr.nearest_bf16(np.float32(1 + 2 ** -8 + 2 ** -20)) == 1 + 2 ** -7  # just past the tie
    assert orr.nearest_bf16(np.float32(-(1 + 3 * 2 ** -8))) == -(1 + 2 ** -6)
    assert orr.nearest_bf16(np.float32(255.5)) == 256.0                          # 255.5 -> spacing 1 at 2^7: tie to 256 (even)
    with pytest.raises(ValueError):
        orr.nearest_bf16(np.float64(1 + 2 ** -40))                               # not fp32


def test_split_bound_and_exact_cases():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 512)) * 10.0 ** rng.uniform(-6, 3, (64, 1))).astype(np.float32)
    hi, lo = orr.split_weights(w)
    w64 = w.astype(np.float64)
    # |w - hi| <= 2^-8 |w| and |w - hi - lo| <= 2^-16 |w| (closed forms of two roundings)
    assert np.all(np.abs(w64 - hi) <= 2.0 ** -8 * np.abs(w64))
    assert np.all(np.abs(w64 - hi - lo) <= 2.0 ** -16 * np.abs(w64))
    # both halves are bf16 values (their binary32 patterns have a zero low half)
    for part in (hi, lo):
        assert np.all(part.astype(np.float32).view(np.uint32) & 0xFFFF == 0)
    # a weight already in bf16 has no residual; one that is bf16 + bf16 is split exactly
    b = _torch_bf16(w)
    hb, lb = orr.split_weights(b.astype(np.float32))
    assert np.array_equal(hb, b) and np.all(lb == 0)
    exact = np.float32([1 + 2 ** -12, -3 * (1 + 2 ** -10), 2 ** -3 + 2 ** -14])
    he, le = orr.split_weights(exact)
    assert np.array_equal(he + le, exact.astype(np.float64))
    assert np.array_equal(he, [1.0, -3.0, 2 ** -3])


def _int_bits(vals):
    return inputs.bf16_bits(np.asarray(vals, np.float32))


def test_integer_gemm_is_exact():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, (5, 96))
    w = rng.integers(-8, 9, (7, 96))
    got = orr.router_logits_exact(_int_bits(x), w.astype(np.float32))
    want = [[sum(int(a) * int(b) for a, b in zip(x[t], w[e])) for e in range(7)] for t in range(5)]
    assert np.array_equal(got, np.array(want, np.float64))
    # integer weights are bf16 values: both passes give the exact logits, the residual is 0
    assert np.array_equal(orr.router_logits_split(_int_bits(x), w.astype(np.float32), 2), got)
    assert np.array_equal(orr.router_logits_split(_int_bits(x), w.astype(np.float32), 1), got)


def test_one_pass_and_two_pass_errors_on_a_worked_case():
    # w = 1 + 2^-12 in every entry, x = 1: the exact logit is H (1 + 2^-12); one pass
    # sees only the high part 1 (loses H 2^-12), two passes recover it exactly
    H = 64
    x = _int_bits(np.ones((1, H)))
    w = np.full((1, H), 1 + 2 ** -12, np.float32)
    assert orr.router_logits_exact(x, w)[0, 0] == H * (1 + 2 ** -12)
    assert orr.router_logits_split(x, w, 1)[0, 0] == H
    assert orr.router_logits_split(x, w, 2)[0, 0] == H * (1 + 2 ** -12)


def test_top_k_against_brute_force_with_ties():
    rng = np.random.default_rng(4)
    for trial in range(200):
        E = int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        v = rng.integers(-3, 4, (1, E)).astype(np.float64)     # many equal values
        idx, vals = orr.top_k(v, k)
        want = sorted(range(E), key=lambda e: (-v[0, e], e))[:k]
        assert idx[0].tolist() == want
        assert np.array_equal(vals[0], v[0, want])


def test_topk_valid_accepts_ties_within_the_bound_only():
    exact = np.array([[3.0, 2.0, 2.0 + 1e-9, 0.0]])
    bound = np.full_like(exact, 1e-6)
    assert orr.topk_valid(np.array([[0, 1]]), exact, bound)[0]          # 1 vs 2 cannot be told apart
    assert orr.topk_valid(np.array([[0, 2]]), exact, bound)[0]
    assert not orr.topk_valid(np.array([[0, 3]]), exact, bound)[0]      # 3 is certainly below 1 and 2
    assert not orr.topk_valid(np.array([[0, 0]]), exact, bound)[0]      # repeated index
    tight = np.full_like(exact, 1e-12)
    assert not orr.topk_valid(np.array([[0, 1]]), exact, tight)[0]


def test_error_bound_holds_for_fp32_summation_in_random_orders():
    rng = np.random.default_rng(5)
    w = inputs.router_workload(3, 4, 256, seed=6)
    hi, lo = orr.split_weights(w.w)
    x = orr.bf16_values(w.x)
    exact = orr.router_logits_exact(w.x, w.w)
    for passes in (1, 2):
        bound = orr.error_bound(w.x, w.w, passes)
        for t, e in itertools.product(range(3), range(4)):
            terms = list((x[t] * hi[e]).astype(np.float32))            # exact products in fp32
            if passes == 2:
                terms += list((x[t] * lo[e]).astype(np.float32))
            for _ in range(20):
                rng.shuffle(terms)
                acc = np.float32(0.0)
                for v in terms:
                    acc = np.float32(acc + v)
                assert abs(float(acc) - exact[t, e]) <= bound[t, e]
    # the two-pass bound is far tighter than the one-pass one on typical weights
    assert np.median(orr.error_bound(w.x, w.w, 2)) < np.median(orr.error_bound(w.x, w.w, 1)) / 8


def test_page_checks_on_known_answers():
    a = np.array([[1.0, 2.0, 3.0], [0.0, 1.0, 0.0]])
    c = orr.page_checks(a, a, 2)
    assert c["max_abs_err"] == 0 and c["top1_match"] == 1 and c["topk_set_match"] == 1
    assert c["min_cosine"] == pytest.approx(1.0)
    assert orr.cosine_rows(np.array([[1.0, 0.0]]), np.array([[0.0, 2.0]]))[0] == 0.0
    assert orr.cosine_rows(np.array([[1.0, 2.0]]), np.array([[3.0, 6.0]]))[0] == pytest.approx(1.0)
    swapped = np.array([[1.0, 3.0, 2.0], [0.0, 1.0, 0.0]])
    c2 = orr.page_checks(swapped, a, 1)
    assert c2["top1_match"] == 0.5 and c2["max_abs_err"] == 1.0

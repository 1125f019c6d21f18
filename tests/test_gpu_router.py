"""The split-precision router GEMM through the C ABI against the fp64 oracle
(oracle/router.py): every logit within the oracle's error bound of the exact
fp32-weight logits, the top-k the oracle's top-k of the kernel's own fp32 logits
(bit-exact indices), and a valid top-k of the exact logits within the bound; the
packed weight decoded by its documented layout equals the oracle's split bit for
bit; the page's checks (error, greedy choice, cosine) for one and two passes."""

import numpy as np
import pytest

from load_balanced_split_amd import _lib, inputs
from oracle import router as orr
from tests.helpers import ensure_built

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    _lib.lib()


def run(rw, passes, top_k=8):
    from load_balanced_split_amd.runner import RouterStep
    print(f"router T={rw.tokens} E={rw.experts} H={rw.hidden} passes={passes} k={top_k}", flush=True)
    r = RouterStep(rw, top_k=top_k)
    r.run(passes)
    return r, r.results()


def check(rw, passes, top_k=8):
    r, (logits, idx, val) = run(rw, passes, top_k)
    exact = orr.router_logits_exact(rw.x, rw.w)
    bound = orr.error_bound(rw.x, rw.w, passes)
    assert np.all(np.isfinite(logits))
    assert np.all(np.abs(logits - exact) <= bound), float(np.max(np.abs(logits - exact) / bound))
    if top_k:
        want_idx, want_val = orr.top_k(logits.astype(np.float32), top_k)   # the kernel's own fp32 logits
        assert np.array_equal(idx, want_idx)
        assert np.array_equal(val, want_val.astype(np.float64))
        assert np.all(orr.topk_valid(idx, exact, bound))
    return r, logits, exact


# decode (K ranges per wave), medium (expert groups per wave) and LDS-tiled shapes (more
# than 256 tokens, experts a multiple of 128), with ragged token counts and K ranges of
# 1, 2 and 3 K-steps in the tiled pipeline; the largest hidden size (65536)
SHAPES = [(1, 256, 7168), (5, 64, 96), (16, 16, 32), (17, 128, 256), (64, 256, 1024), (65, 48, 160),
          (300, 256, 2048), (8, 1024, 512), (33, 32, 64), (257, 128, 64), (1000, 384, 32), (300, 128, 96),
          (520, 1024, 256), (3, 16, 65536)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("passes", [1, 2])
def test_router_logits_and_topk_against_oracle(shape, passes):
    T, E, H = shape
    rw = inputs.router_workload(T, E, H, seed=T * 7 + E + H)
    check(rw, passes, top_k=min(8, E))


def test_router_full_prefill_shape():
    rw = inputs.router_workload(4096, 256, 7168, seed=11)
    for passes in (1, 2):
        check(rw, passes)


def test_packed_weight_is_the_oracle_split_in_the_documented_layout():
    rw = inputs.router_workload(1, 48, 160, seed=3)
    r, _ = run(rw, 2)
    packed = r.packed.cpu().numpy().view(np.uint16)
    E, H = rw.experts, rw.hidden
    hi, lo = orr.split_weights(rw.w)
    e, k = np.meshgrid(np.arange(E), np.arange(H), indexing="ij")
    tile = (e // 16) * (H // 32) + k // 32
    lane = 16 * ((k % 32) // 8) + e % 16
    off = (2048 * tile + 16 * lane + 2 * (k % 8)) // 2          # in uint16 units
    assert np.array_equal(orr.bf16_values(packed[off]), hi)
    assert np.array_equal(orr.bf16_values(packed[off + 512]), lo)


def test_two_passes_are_far_more_accurate_than_one():
    rw = inputs.router_workload(2048, 256, 4096, seed=5)
    _, l1, exact = check(rw, 1)
    _, l2, _ = check(rw, 2)
    c1 = orr.page_checks(l1, exact, 8)
    c2 = orr.page_checks(l2, exact, 8)
    print("one pass", c1, "two passes", c2, flush=True)
    assert c2["max_abs_err"] * 16 < c1["max_abs_err"]
    assert c2["min_cosine"] >= c1["min_cosine"] and c2["min_cosine"] > 1 - 1e-10
    assert c2["topk_set_match"] >= c1["topk_set_match"] and c2["top1_match"] >= c1["top1_match"]


def test_router_edge_cases():
    # equal weight rows give bit-equal logits: the top-k lists the lower expert first
    rw = inputs.router_workload(20, 32, 256, seed=9)
    rw.w[7] = rw.w[3]
    rw.w[30] = rw.w[3]
    r, (logits, idx, _) = run(rw, 2, top_k=32)
    assert np.array_equal(logits[:, 3], logits[:, 7]) and np.array_equal(logits[:, 3], logits[:, 30])
    for t in range(20):
        pos = [list(idx[t]).index(e) for e in (3, 7, 30)]
        assert pos == sorted(pos)
    # the same with enough tokens for the one-wave-per-token top-k
    rw = inputs.router_workload(600, 32, 256, seed=19)
    rw.w[7] = rw.w[3]
    rw.w[30] = rw.w[3]
    r, (logits, idx, _) = run(rw, 2, top_k=32)
    assert np.array_equal(logits[:, 3], logits[:, 7]) and np.array_equal(logits[:, 3], logits[:, 30])
    for t in range(0, 600, 37):
        pos = [list(idx[t]).index(e) for e in (3, 7, 30)]
        assert pos == sorted(pos)
    # top_k == experts, top_k == 0 (both top-k kernels), and a second run is bit-identical
    check(inputs.router_workload(3, 16, 64, seed=1), 2, top_k=16)
    check(inputs.router_workload(3, 16, 64, seed=1), 2, top_k=0)
    check(inputs.router_workload(700, 16, 64, seed=4), 2, top_k=16)
    check(inputs.router_workload(700, 16, 64, seed=4), 2, top_k=0)
    rw = inputs.router_workload(100, 256, 1024, seed=2)
    r, (l_a, i_a, _) = run(rw, 2)
    r.run(2)
    l_b, i_b, _ = r.results()
    assert np.array_equal(l_a, l_b) and np.array_equal(i_a, i_b)
    # no tokens: nothing is launched, nothing is read
    from load_balanced_split_amd.runner import RouterStep
    RouterStep(inputs.router_workload(0, 64, 64, seed=0)).run(2)
    torch.cuda.synchronize()

"""GPU parity of the fused FP8 MoE layer (hpa_moe_fused, through the C ABI) against
the oracle.

Tolerance (derived from the arithmetic; the pages give none for this path): both
sides take the same E4M3 decisions for the tokens (fp32 scale and division on
both), and every FP8 x FP8 product is exact in fp32, so Gate-Up differs only by how
the MFMA sums the products (measured: within ~4e-5 of the row's largest activation,
coarser than an fp32 sum). The requantised activation codes can then differ by one
code where a / sa lies within that distance of a rounding midpoint (measured: 9 of
5120 codes on a 20-token call); each such code moves one of I terms of a Down row by
at most one E4M3 step (2^-3 relative). With outputs of order 0.1-1,
|gpu - ref| <= 1e-2 + 1e-2 |ref| per element (the bf16 rounding of the output, 2^-9
relative, included) covers these and fails any wrong term. The fp32 activations are checked against the oracle's at
1e-4 relative to the row's largest magnitude."""

import numpy as np
import pytest

from load_balanced_split_amd import _lib, inputs
from oracle import moe as om
from tests.helpers import ensure_built

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL = RTOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    _lib.lib()


def _check(mw, tokens=None, act=True):
    from load_balanced_split_amd.runner import MoeStep
    d = MoeStep(mw)
    print(f"moe T={mw.tokens} E={mw.experts} K={mw.top_k} H={mw.hidden} I={mw.inter}", flush=True)
    d.workspace.fill_(0xFF)                     # NaN everywhere the kernels do not write
    d.run()
    torch.cuda.synchronize()
    got = d.output_f64()
    assert np.all(np.isfinite(got))
    rows = range(mw.tokens) if tokens is None else tokens
    sel = list(rows)
    ref, det = om.fused_moe(mw.x[sel], mw.ids[sel], mw.weights[sel], mw.w1, mw.s1, mw.w2, mw.s2, details=True)
    err = np.abs(got[sel] - ref)
    ratio = float(np.max(err / (ATOL + RTOL * np.abs(ref))))
    print(f"   max |err| {err.max():.3e}, max err/tol {ratio:.3f}, max |ref| {np.abs(ref).max():.3f}", flush=True)
    assert ratio <= 1.0
    if act:
        a_gpu = d.activations()
        for i, t in enumerate(sel):
            for k in range(mw.top_k):
                if (i, k) in det["act"]:
                    want = det["act"][(i, k)]
                    scale = max(np.abs(want).max(), 1e-30)
                    assert np.max(np.abs(a_gpu[t, k] - want)) <= 1e-4 * scale, (t, k)
    if mw.tokens * mw.top_k > 16:           # the routing pass wrote the token codes: bit-exact
        x8, sx = d.token_codes()
        want8, wants = om.quantize_fp32(inputs_f32(mw.x))
        assert np.array_equal(sx, wants) and np.array_equal(x8, want8)
        _check_routing(d, mw)
    assert int(d.err.item()) == 0
    return d, got


def _check_routing(d, mw):
    """The routing index: every valid pair listed once, grouped by expert in expert
    order and in pair order inside a group; the pair blocks cut each group into runs of
    at most 16, in list order."""
    lst, be, bf, bn = d.routing()
    ids = mw.ids.reshape(-1)
    want, blocks = [], []
    for e in range(mw.experts):
        pairs = np.flatnonzero(ids == e)
        for j in range(0, len(pairs), 16):
            blocks.append((e, len(want) + j, min(16, len(pairs) - j)))
        want.extend(pairs.tolist())
    n = len(want)
    assert np.array_equal(lst[:n], np.array(want, dtype=np.int32))
    assert list(zip(be.tolist(), bf.tolist(), bn.tolist())) == blocks


def inputs_f32(x_bits):
    from oracle.formats import bf16_to_f64
    return bf16_to_f64(x_bits).astype(np.float32)


@pytest.mark.parametrize("shape", [(1, 4, 1, 128, 128), (5, 4, 2, 256, 128), (33, 16, 8, 384, 256),
                                   (17, 8, 3, 128, 384), (64, 32, 4, 512, 256), (40, 1, 1, 128, 256),
                                   (300, 1024, 2, 128, 128)])
def test_moe_small_shapes_against_oracle(shape):
    """Every token against the oracle. The grouped kernels take two row blocks per
    Gate-Up wave when pairs >= 4 x experts (one expert holding all 40 pairs: three pair
    blocks), one otherwise (1024 experts: the largest routing table)."""
    T, E, K, H, I = shape
    _check(inputs.moe_workload(T, E, K, H, I, seed=sum(shape)))


@pytest.mark.parametrize("T", [1, 32, 128])
def test_moe_decode_shape_sampled_tokens(T):
    """The benchmark's decode shapes (1, 32 and 128 tokens, 128 experts, top 8, hidden
    2048, inter 768, the bench's seeds) on sampled tokens, and two runs give identical
    bits."""
    mw = inputs.moe_workload(T, 128, 8, 2048, 768, seed=T)
    d, got = _check(mw, tokens=sorted({0, T // 4, T // 2, T - 1}), act=True)
    d.run()
    torch.cuda.synchronize()
    assert np.array_equal(d.output_f64(), got)


@pytest.mark.parametrize("shape", [(1, 32, 16, 256, 4096), (2, 8, 8, 512, 2048), (16, 4, 1, 128, 384),
                                   (1, 16, 8, 2048, 768)])
def test_moe_few_pair_shapes(shape):
    """Calls of at most 16 pairs (Gate-Up quantises the token; one Down launch
    requantises, multiplies and merges, one workgroup of top_k waves per token and 16
    rows): the widest workgroup (top 16, inter 4096: 1024 threads, 64 KB of codes), the
    middle activation width, one-wave workgroups (16 tokens x top 1), the bench's
    one-token shape on every row."""
    T, E, K, H, I = shape
    _check(inputs.moe_workload(T, E, K, H, I, seed=3 * sum(shape)))


def test_moe_edge_cases():
    """A zero token gives a zero row; an expert id out of range adds nothing and is
    reported; a token routed twice to one expert adds both slots; more than 16 tokens
    on one expert span several pair blocks."""
    from load_balanced_split_amd.runner import MoeStep
    mw = inputs.moe_workload(40, 6, 3, 256, 128, seed=9)
    mw.x[3] = 0
    mw.ids[5, 1] = mw.ids[5, 0]                 # the same expert twice
    mw.ids[:, 2] = 2                             # every token on expert 2 (40 > 16 pairs)
    mw.ids[5, 2] = 2
    mw.ids[0, 0], mw.ids[1, 2] = 6, -1           # out of range: skipped
    d = MoeStep(mw)
    d.run()
    torch.cuda.synchronize()
    assert int(d.err.item()) & _lib.DEVERR_MOE_EXPERT
    got = d.output_f64()
    ref = om.fused_moe(mw.x, mw.ids, mw.weights, mw.w1, mw.s1, mw.w2, mw.s2)
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))
    assert not got[3].any()
    _check_routing(d, mw)                        # out-of-range ids are not listed
    # the same cases with few enough pairs (<= 16) that every pair is its own block and
    # Gate-Up quantises the tokens itself
    mw = inputs.moe_workload(4, 6, 3, 256, 128, seed=10)
    mw.x[1] = 0
    mw.ids[2, 1] = mw.ids[2, 0]
    mw.ids[0, 2], mw.ids[3, 0] = 6, -2
    d = MoeStep(mw)
    d.workspace.fill_(0xFF)
    d.run()
    torch.cuda.synchronize()
    assert int(d.err.item()) & _lib.DEVERR_MOE_EXPERT
    got = d.output_f64()
    ref = om.fused_moe(mw.x, mw.ids, mw.weights, mw.w1, mw.s1, mw.w2, mw.s2)
    assert np.all(np.isfinite(got)) and np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))
    assert not got[1].any()


def test_moe_weight_packing_layout():
    """hpa_moe_pack_weights places byte (e, r, col) of a row-major [E][rows][cols] array
    at tile ((e rows/16 + r/16) cols/128 + col/128) * 2048, lane l = r%16 + 16 q with
    q = (col%128)/32, byte 16 l + j (j = col%32 < 16) or 1024 + 16 l + j - 16."""
    E, R, C = 3, 48, 384
    w = np.random.default_rng(1).integers(0, 256, size=(E, R, C), dtype=np.uint8)
    wd = torch.from_numpy(w).cuda()
    packed = torch.empty_like(wd)
    _lib.hpa_moe_pack_weights(wd, packed)
    torch.cuda.synchronize()
    got = packed.cpu().numpy().reshape(-1)
    e, r, col = np.meshgrid(np.arange(E), np.arange(R), np.arange(C), indexing="ij")
    tile = (e * (R // 16) + r // 16) * (C // 128) + col // 128
    lane = r % 16 + 16 * ((col % 128) // 32)
    j = col % 32
    dest = tile * 2048 + np.where(j < 16, 16 * lane + j, 1024 + 16 * lane + j - 16)
    assert np.array_equal(np.sort(dest.reshape(-1)), np.arange(E * R * C))   # a permutation
    assert np.array_equal(got[dest], w)
    with pytest.raises(RuntimeError):
        _lib.hpa_moe_pack_weights(torch.empty((1, 24, 128), dtype=torch.uint8, device="cuda"),
                                  torch.empty((1, 24, 128), dtype=torch.uint8, device="cuda"))


def test_moe_maximum_sizes():
    """The limits: 1024 tokens x top 16 (16384 pairs, the most the workspace plans for;
    16 experts, so each has ~1024 pairs in ~64 pair blocks), sampled tokens; and hidden =
    inter = 4096 (the largest rows) with every token checked."""
    mw = inputs.moe_workload(1024, 16, 16, 256, 128, seed=21)
    _check(mw, tokens=[0, 333, 777, 1023], act=True)
    mw = inputs.moe_workload(3, 2, 2, 4096, 4096, seed=22)
    _check(mw, act=True)


def test_moe_few_pair_path_equals_grouped_path():
    """Two tokens x top 8 (16 pairs: every pair its own block, tokens quantised inside
    Gate-Up) give the same bits as the same two tokens inside a three-token batch (24
    pairs: the routing index, pairs grouped by expert with other tokens' pairs)."""
    from load_balanced_split_amd.runner import MoeStep
    big = inputs.moe_workload(3, 8, 8, 256, 256, seed=12)
    small = inputs.moe_workload(2, 8, 8, 256, 256, seed=12)
    small.x, small.ids, small.weights = big.x[:2].copy(), big.ids[:2].copy(), big.weights[:2].copy()
    small.w1, small.s1, small.w2, small.s2 = big.w1, big.s1, big.w2, big.s2
    outs = []
    for mw in (small, big):
        d = MoeStep(mw)
        d.run()
        torch.cuda.synchronize()
        outs.append(d.output_f64()[:2])
    assert np.array_equal(outs[0], outs[1])

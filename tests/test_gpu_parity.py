"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Planner work lists must be bit-identical to the CPU planner; attention outputs
must match the oracle within |gpu - ref| <= atol + rtol |ref| per element
(bf16 KV: 1e-2 / 1e-2, E4M3 KV: 3e-2 / 3e-2).
"""

import math

import numpy as np
import pytest

from load_balanced_split_amd import _lib, inputs
from oracle import attention as oa
from oracle import planner as op
from oracle import prologue as opro
from oracle.kv_layout import index_table
from tests.helpers import TOL, assert_within, ensure_built, tolerance_report

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PLAN_KEYS = ("C", "worker_off", "item_s", "item_t0", "item_t1", "item_split", "item_slot",
             "num_splits", "partial_base", "merge_list")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    _lib.lib()
    return torch.device("cuda")


def device_plan(lens, hkv, W, min_tiles, item_cost=0, tail_den=0, tail_chunk=1, item_order=0):
    """Run the GPU planner on a length vector; return its arrays as host lists."""
    B = len(lens)
    maxp = max(1, max([(int(L) + 63) // 64 for L in lens] or [1]))
    desc = _lib.make_desc(B, hkv, hkv, maxp, 1)
    size = _lib.hpa_plan_workspace_size(desc, W)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    _lib.hpa_plan(desc, sl, W, min_tiles, item_cost, tail_den, tail_chunk, ws, item_order=item_order)
    torch.cuda.synchronize()
    lay = _lib.hpa_plan_workspace_layout(desc, W)
    h = ws.cpu().numpy().view(np.int32)
    hdr = h[:16]
    Wp, N, S, nit, nm, npart = (int(x) for x in hdr[:6])
    D, Ws = int(hdr[8]), int(hdr[9])
    g = lambda k, n: h[lay[k] // 4: lay[k] // 4 + n].tolist()
    return dict(Wp=Wp, Ws=Ws, D=D, N=N, S=S, n_items=nit, n_partials=npart, err=int(hdr[6]),
                C=g("C", S + 1), worker_off=g("worker_off", Ws + D + 1), item_s=g("item_s", nit),
                item_t0=g("item_t0", nit), item_t1=g("item_t1", nit), item_split=g("item_split", nit),
                item_slot=g("item_slot", nit), num_splits=g("num_splits", S),
                partial_base=g("partial_base", S), merge_list=g("merge_list", nm))


def check_plan(lens, hkv, W, mt, cost=0, den=0, chunk=1, order=0):
    got = device_plan(lens, hkv, W, mt, cost, den, chunk, order)
    want = op.balanced_plan(lens, hkv, W, mt, cost, den, chunk, order)
    assert got["err"] == 0
    for k in ("Wp", "Ws", "D", "N", "n_items", "n_partials") + PLAN_KEYS:
        assert got[k] == want[k], (k, lens, hkv, W, mt, cost, den, chunk, order)


# ---------------------------------------------------------------- planner ---

@pytest.mark.parametrize("tail", [(0, 1), (8, 8), (3, 1)])
@pytest.mark.parametrize("cost", [0, 3])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("W,mt", [(0, 1), (1, 1), (7, 1), (512, 1), (512, 4), (1024, 1), (3000, 2)])
def test_plan_bit_exact_workload_lengths(cfg, W, mt, cost, tail):
    lens = inputs.config_lengths_only(cfg) + (1 if cfg == 4 else 0)
    hkv = 4 if cfg == 3 else 1
    if W == 0:
        W = _lib.hpa_default_num_workers(0)
    print(f"plan cfg{cfg} W={W} mt={mt} cost={cost} tail={tail}", flush=True)
    for order in (0, 1, 2):
        check_plan(lens.tolist(), hkv, W, mt, cost, *tail, order)


def test_plan_bit_exact_random_lengths():
    rng = np.random.default_rng(123)
    for trial in range(300):
        B = int(rng.integers(1, 300))
        hkv = int(rng.integers(1, 5))
        lens = rng.integers(0, 20000, size=B)
        lens[rng.random(B) < 0.3] = 0
        if trial % 5 == 0:
            lens[:] = rng.choice([0, 1, 63, 64, 65, 4096, 65535, 65536, 65537], size=B)
        W = int(rng.integers(1, 4000))
        mt = int(rng.integers(1, 6))
        cost = int(rng.integers(0, 6)) if trial % 2 else 0
        den = int(rng.integers(1, 17)) if trial % 3 else 0
        chunk = int(rng.integers(1, 40))
        check_plan(lens.tolist(), hkv, W, mt, cost, den, chunk, trial % 3)
    check_plan([0, 0, 0], 2, 16, 1)              # N == 0: no active workers
    check_plan([0, 0, 0], 2, 16, 1, 4)
    check_plan([5000], 1, 100000 // 64, 1)       # W > N tiles
    check_plan([64, 64], 1, 4, 1, 2)             # workers owning only virtual tiles get no item
    check_plan([64] * 40, 1, 300, 1, 64)         # the largest cost
    check_plan([192], 1, 4, 1, 0, 2, 1)          # fewer static workers than active ones
    check_plan([5000, 64, 0, 3000], 2, 9, 1, 2, 1, 1)   # everything in the tail, 4 W chunks
    check_plan([5000, 64, 0, 3000], 2, 9, 1, 2, 1, 1000)  # everything in one chunk
    check_plan([0, 0], 1, 9, 1, 0, 4, 2)         # N == 0 with a tail


# -------------------------------------------------------------- attention ---

def run_and_compare(w, sched="balanced", W=0, min_tiles=_lib.FUSED_MIN_TILES, ref=None, what=""):
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w, num_workers=W)
    print(f"attn {what} {w.name} sched={sched} W={d.num_workers}", flush=True)
    if sched == "single":
        scrub_partials(d)
    d.step(sched, min_tiles)
    torch.cuda.synchronize()
    assert d.device_error() == 0
    if ref is None:
        ref = oracle_out(w)
    got = d.output_f64()
    r = assert_within(got, ref, w.kv_dtype, f"{w.name} {sched} W={W}")
    return got, r, d


def scrub_partials(d):
    """Fill the partial workspace with NaN (all bits set) before a single-launch step:
    a fold that read a partial before its producer's stores were visible would then
    give a non-finite or different output instead of an earlier run's equal bits."""
    d.partial_ws.fill_(0xFF)


def oracle_out(w):
    if w.has_prologue:
        pr = opro.prologue(w)
        return oa.decode_attention(pr["q_rot"], pr["k_cache"], pr["v_cache"], pr["seq_lens"], w.page_table,
                                   w.hkv, w.sm_scale, w.kv_dtype, w.k_scale, w.v_scale)
    return oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, w.hkv, w.sm_scale,
                               w.kv_dtype, w.k_scale, w.v_scale)


EDGE_LENS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 700, 1000]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [(8, 1), (32, 4), (4, 1), (16, 1), (2, 2)])
def test_edge_lengths_all_schedules(kv_dtype, heads):
    hq, hkv = heads
    w = inputs.build_workload("edge", EDGE_LENS, hq, hkv, kv_dtype, seed=5, pool_pages=60, poison=True)
    ref = oracle_out(w)
    outs = {}
    for sched, W in [("balanced", 0), ("balanced", 1), ("balanced", 3), ("balanced", 37),
                     ("fused", 0), ("fused", 1), ("fused", 3), ("fused", 37),
                     ("single", 0), ("single", 1), ("single", 3), ("single", 37),
                     ("static_splits", 0), ("static_splits", 5), ("static_chunk", 0), ("static_chunk", 9)]:
        got, r, _ = run_and_compare(w, sched, W, ref=ref, what=f"{kv_dtype} {hq}:{hkv}")
        assert np.all(got[0] == 0)                      # empty request -> zero row
        outs[(sched, W)] = got
    # the fused schedules compute the planner's work list in-kernel (and the single-launch
    # one merges in-kernel, in the merge kernel's order): identical bits
    for W in (0, 1, 3, 37):
        assert np.array_equal(outs[("balanced", W)], outs[("fused", W)])
        assert np.array_equal(outs[("balanced", W)], outs[("single", W)])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_random_batches(kv_dtype):
    rng = np.random.default_rng(77)
    for trial in range(6):
        B = int(rng.integers(1, 24))
        lens = rng.integers(0, 3000, size=B)
        w = inputs.build_workload("rand", lens, 8, 1, kv_dtype, seed=int(rng.integers(1 << 30)), poison=trial % 2 == 0)
        ref = oracle_out(w)
        W_r = int(rng.integers(1, 50))
        for sched, W in [("balanced", 0), ("balanced", W_r), ("fused", W_r), ("static_splits", 0)]:
            run_and_compare(w, sched, W, min_tiles=int(rng.integers(1, 4)), ref=ref, what=f"trial{trial}")


def test_tiny_workload():
    w = inputs.config_workload(0)
    ref = oracle_out(w)
    for sched in ("balanced", "static_splits", "static_chunk"):
        run_and_compare(w, sched, ref=ref)
    run_and_compare(w, "balanced", W=4, ref=ref)


@pytest.mark.parametrize("case", ["three_blocks_256_threads", "two_blocks_128_threads"])
def test_many_splits_combine_blocks(case):
    """One sequence split more than 256 ways: its 16-split groups form more than one
    block of 16 group results, so every level of the combine runs (group, block, and
    the in-order fold of block results), in the merge kernel (256-thread blocks with
    two-pass prefetch, or 128-thread blocks whose block spans four passes) and in the
    single-launch in-kernel merge. Planned, fused and single-launch bits agree and
    match the oracle. The split counts come from the CPU planner."""
    if case == "three_blocks_256_threads":
        lens, hq, hkv, W = [80000, 700, 3000], 8, 1, 4000
    else:
        lens, hq, hkv, W = [40000] + [100] * 63, 32, 4, 2000
    plan = op.balanced_plan(lens, hkv, W, _lib.FUSED_MIN_TILES, _lib.FUSED_ITEM_COST, 0, 1, 0)
    groups = -(-max(plan["num_splits"]) // 16)
    two = len(lens) * hkv * (hq // hkv) <= W          # the merge kernel's 256-thread blocks
    assert groups > 16 and two == (case == "three_blocks_256_threads"), (groups, two)
    w = inputs.build_workload("many_splits", lens, hq, hkv, "bf16", seed=61, poison=True)
    ref = oracle_out(w)
    outs = {s: run_and_compare(w, s, W, ref=ref, what=case)[0] for s in ("balanced", "fused", "single")}
    assert np.array_equal(outs["balanced"], outs["fused"])
    assert np.array_equal(outs["balanced"], outs["single"])


@pytest.mark.parametrize("W,splits", [(16, 16), (17, 17), (260, 256), (261, 257)])
def test_combine_group_and_block_boundaries(W, splits):
    """A sequence split exactly 16, 17, 256 and 257 ways: one full group, a group and a
    single split, one full block of 16 groups, a block and a single group (plus a
    short request and an empty one). Planned, fused and single-launch bits agree and
    match the oracle; the split counts come from the CPU planner."""
    lens = [38400, 100, 0]
    plan = op.balanced_plan(lens, 1, W, _lib.FUSED_MIN_TILES, _lib.FUSED_ITEM_COST, 0, 1, 0)
    assert plan["num_splits"][0] == splits
    w = inputs.build_workload("combine_edges", lens, 8, 1, "bf16", seed=62, poison=True)
    ref = oracle_out(w)
    outs = {s: run_and_compare(w, s, W, ref=ref, what=f"{splits} splits")[0] for s in ("balanced", "fused", "single")}
    assert np.array_equal(outs["balanced"], outs["fused"])
    assert np.array_equal(outs["balanced"], outs["single"])


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_full_size_bf16_workloads(cfg):
    w = inputs.config_workload(cfg)
    ref = oracle_out(w)
    outs = {}
    for sched in ("balanced", "fused", "single", "static_splits", "static_chunk"):
        got, r, _ = run_and_compare(w, sched, ref=ref, what=f"cfg{cfg}")
        print(f"cfg{cfg} {sched}: {r}", flush=True)
        outs[sched] = got
    assert np.array_equal(outs["balanced"], outs["fused"])
    assert np.array_equal(outs["balanced"], outs["single"])
    # one worker (no split at all) agrees with the default within tolerance
    if cfg != 3:
        run_and_compare(w, "balanced", W=1, ref=ref, what=f"cfg{cfg} single worker")


def test_fp8_prologue_workload():
    w = inputs.config_workload(4)
    pr = opro.prologue(w)
    ref = oa.decode_attention(pr["q_rot"], pr["k_cache"], pr["v_cache"], pr["seq_lens"], w.page_table, w.hkv,
                              w.sm_scale, w.kv_dtype, w.k_scale, w.v_scale)
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w)
    print(f"cfg4 W={d.num_workers}", flush=True)
    d.step("balanced")
    torch.cuda.synchronize()
    assert d.device_error() == 0
    assert np.array_equal(d.lens_after.cpu().numpy(), pr["seq_lens"])
    # rotated q: bf16 rounding of the fp64 value
    q_rot = d.q_rot.float().cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(q_rot, pr["q_rot"], rtol=2 ** -8, atol=1e-6)
    # appended codes: equal except a neighbouring code at rounding ties (fp32 vs fp64)
    kc = d.k_cache.cpu().numpy()
    vc = d.v_cache.cpu().numpy()
    diffs = 0
    for b, L in enumerate(w.seq_lens):
        p, r = w.page_table[b, L // 64], L % 64
        kt, vt = index_table("k", "fp8")[r], index_table("v", "fp8")[r]
        for got, want in ((kc[p][:, kt], pr["k_codes"][b]), (vc[p][:, vt], pr["v_codes"][b])):
            dif = np.abs(got.astype(int) - want.astype(int))
            assert dif.max() <= 1
            diffs += int((dif > 0).sum())
    print(f"cfg4 appended E4M3 codes off by one code: {diffs}", flush=True)
    assert diffs <= 4
    got = d.output_f64()
    r = assert_within(got, ref, "fp8", "cfg4")
    print(f"cfg4 attention: {r}", flush=True)
    # the other schedules on the same (already appended) cache
    for sched in ("fused", "single", "static_splits", "static_chunk"):
        d.attend(sched)
        torch.cuda.synchronize()
        assert_within(d.output_f64(), ref, "fp8", f"cfg4 {sched}")


def _plan_of(d):
    pa = d.plan_arrays()
    return {k: pa[k] for k in ("Wp", "Ws", "D", "N", "S", "n_items", "n_partials") + PLAN_KEYS}


def _prologue_plan_matches_separate(w, W=0, break_request=None):
    """One launch (prologue + planner) against two (prologue, then hpa_plan over
    seq_lens_out): same plan, same output bits, and the oracle's plan over the
    appended lengths."""
    from load_balanced_split_amd.runner import DeviceStep
    one, two = DeviceStep(w, num_workers=W), DeviceStep(w, num_workers=W)
    for d in (one, two):
        d.lens_after.copy_(d.seq_lens)               # what a failed append leaves in place
        if break_request is not None:
            b = break_request
            d.page_table[b, int(w.seq_lens[b]) // 64] = w.num_pages + 3
    print(f"prologue+plan {w.name} B={w.batch} hkv={w.hkv} W={one.num_workers}", flush=True)
    one.step("balanced")
    two.step("balanced", prologue_plans=False)
    torch.cuda.synchronize()
    assert _plan_of(one) == _plan_of(two)
    # a failed append leaves that request's rotated q unwritten: compare the others
    keep = [b for b in range(w.batch) if b != break_request]
    assert torch.equal(one.out[keep], two.out[keep])
    assert torch.equal(one.lens_after, two.lens_after)
    want = op.balanced_plan(one.lens_after.cpu().numpy().tolist(), w.hkv, one.num_workers,
                            _lib.FUSED_MIN_TILES, _lib.FUSED_ITEM_COST, _lib.FUSED_TAIL_DEN, _lib.FUSED_TAIL_CHUNK)
    got = _plan_of(one)
    for k in ("Wp", "Ws", "D", "n_items", "n_partials") + PLAN_KEYS:
        assert got[k] == want[k], k
    return one, two


def test_prologue_plan_one_launch_equals_two():
    w = inputs.config_workload(4)
    one, _ = _prologue_plan_matches_separate(w)
    assert one.device_error() == 0
    # and the fused schedule on the same appended cache gives the same bits
    one.attend("fused")
    torch.cuda.synchronize()
    fused = one.out.clone()
    one.attend("balanced")
    torch.cuda.synchronize()
    assert torch.equal(one.out, fused)


def test_prologue_plan_failed_append_and_large_batch():
    """A request whose append fails keeps its old length in the plan (and the error is
    reported); above 3072 sequences the plan is made by a second launch."""
    w = inputs.build_workload("pplan", [0, 5, 63, 64, 127, 128, 1000, 4000], 16, 2, "bf16", seed=19,
                              prologue=True, poison=True)
    one, two = _prologue_plan_matches_separate(w, W=13, break_request=3)
    assert one.device_error(clear=True) & _lib.DEVERR_PROLOGUE
    lens = np.random.default_rng(20).integers(0, 100, size=3100)
    wl = inputs.build_workload("pplan_big", lens, 8, 1, "bf16", seed=21, prologue=True)
    one, _ = _prologue_plan_matches_separate(wl, W=100)
    assert one.device_error() == 0


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_bf16_and_fp8_prologue_small(kv_dtype):
    w = inputs.build_workload("pro", [0, 5, 63, 64, 127, 128, 1000, 4000], 16, 2, kv_dtype, seed=9,
                              prologue=True, poison=True)
    pr = opro.prologue(w)
    got, r, d = run_and_compare(w, "balanced", what="prologue")
    q_rot = d.q_rot.float().cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(q_rot, pr["q_rot"], rtol=2 ** -8, atol=1e-6)


def test_page_permutation_bit_identical_on_gpu():
    w = inputs.build_workload("perm", [70, 300, 1, 129, 1500], 8, 1, "bf16", seed=3, pool_pages=60)
    g1, _, _ = run_and_compare(w, "balanced", W=5)
    perm = np.random.default_rng(4).permutation(w.num_pages)
    kc = np.empty_like(w.k_cache)
    vc = np.empty_like(w.v_cache)
    kc[perm] = w.k_cache
    vc[perm] = w.v_cache
    w.k_cache, w.v_cache = kc, vc
    w.page_table = np.where(w.page_table >= 0, perm[np.maximum(w.page_table, 0)], -1).astype(np.int32)
    g2, _, _ = run_and_compare(w, "balanced", W=5)
    assert np.array_equal(g1, g2)


def test_constant_v_returns_it_on_gpu():
    w = inputs.build_workload("constv", [1, 64, 333, 2000], 8, 1, "bf16", seed=6)
    u = inputs.bf16_bits(np.random.default_rng(7).standard_normal(128).astype(np.float32))
    w.v_cache[:] = inputs.tile_v(np.broadcast_to(u, (64, 128)), "bf16")[None, None, :]
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w, num_workers=9)
    d.step("balanced")
    torch.cuda.synchronize()
    want = (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = d.output_f64()
    for b in range(4):
        np.testing.assert_allclose(got[b], np.broadcast_to(want, (8, 128)), rtol=2 ** -7, atol=1e-6)


def test_device_errors_are_reported_not_faulted():
    w = inputs.build_workload("bad", [100, 200, 300], 8, 1, "bf16", seed=8)
    w.page_table[1, 2] = w.num_pages + 5            # out-of-range page id for request 1
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w, num_workers=6)
    d.step("balanced")
    torch.cuda.synchronize()
    assert d.device_error(clear=True) & _lib.DEVERR_PAGE_ID
    assert d.device_error() == 0
    ref = oracle_out(inputs.build_workload("bad", [100, 200, 300], 8, 1, "bf16", seed=8))
    got = d.output_f64()
    assert_within(got[[0, 2]], ref[[0, 2]], "bf16", "requests with valid pages")
    # a length beyond the page table is reported by the planner
    d.seq_lens[0] = 64 * w.max_pages + 1
    d.step("balanced")
    torch.cuda.synchronize()
    assert d.device_error(clear=True) & _lib.DEVERR_SEQ_LEN
    # attention launched with a different worker count than the plan
    _lib.hpa_plan(d.desc, d.seq_lens, 5, 1, 0, 0, 1, d.plan_ws)
    d.attend("balanced")
    torch.cuda.synchronize()
    assert d.device_error(clear=True) & _lib.DEVERR_PLAN


def test_plan_for_another_batch_shape_is_refused():
    """A plan made for B = 3 (or for the same B x Hkv split differently) used by a
    B = 4 launch with the same worker count: the device reports HPA_DEVERR_PLAN and
    neither the attention nor the merge kernel writes an output row."""
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.build_workload("shape", [700, 64, 3000, 129], 8, 1, "bf16", seed=18)
    d = DeviceStep(w, num_workers=6)
    d.step("balanced")
    torch.cuda.synchronize()
    assert d.device_error() == 0
    good = d.out.clone()
    for B, hkv, hq in ((3, 1, 8), (2, 2, 16)):
        desc = _lib.make_desc(B, hq, hkv, w.max_pages, w.num_pages)
        lens = d.seq_lens[:B].contiguous()
        print(f"plan shape B={B} hkv={hkv} against B=4 hkv=1", flush=True)
        _lib.hpa_plan(desc, lens, 6, _lib.FUSED_MIN_TILES, _lib.FUSED_ITEM_COST, 0, 1, d.plan_ws)
        d.out.fill_(7.0)
        d.attend("balanced")
        torch.cuda.synchronize()
        assert d.device_error(clear=True) & _lib.DEVERR_PLAN, (B, hkv)
        assert torch.all(d.out == 7.0), (B, hkv)
    # a plan of the right shape works again on the same workspace
    d.step("balanced")
    torch.cuda.synchronize()
    assert d.device_error() == 0 and torch.equal(d.out, good)


@pytest.mark.parametrize("hkv", [1, 2])
def test_fused_schedule_both_planners(hkv):
    """Up to 256 sequences the fused kernel plans in registers, above that in LDS: both
    give the planned schedule's bits, with empty requests and a bad length among them."""
    rng = np.random.default_rng(31)
    for B in (250 // hkv, 300 // hkv):
        lens = rng.integers(0, 400, size=B)
        lens[rng.random(B) < 0.1] = 0
        w = inputs.build_workload("fusedplan", lens, 4 * hkv, hkv, "bf16", seed=int(B), poison=True)
        ref = oracle_out(w)
        W = int(rng.integers(20, 300))
        g_bal, _, _ = run_and_compare(w, "balanced", W, ref=ref, what=f"S={B * hkv}")
        g_fus, _, _ = run_and_compare(w, "fused", W, ref=ref, what=f"S={B * hkv}")
        g_one, _, _ = run_and_compare(w, "single", W, ref=ref, what=f"S={B * hkv}")
        assert np.array_equal(g_bal, g_fus) and np.array_equal(g_bal, g_one)


def test_single_launch_merge_counters_reset_across_steps():
    """The in-kernel merge's arrival counters return to zero: repeated steps (and a
    different batch on the same workspace) keep giving the planned schedule's bits."""
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.build_workload("repeat", [5000, 64, 3000, 1, 700], 8, 1, "bf16", seed=12)
    d = DeviceStep(w, num_workers=23)
    d.step("balanced")
    torch.cuda.synchronize()
    want = d.out.clone()
    for rep in range(4):
        d.out.zero_()
        scrub_partials(d)
        d.step("single")
        torch.cuda.synchronize()
        assert torch.equal(d.out, want), rep
    # shorter lengths on the same buffers: other split structure, same workspace
    d.seq_lens.copy_(torch.tensor([4000, 0, 2900, 1, 1], dtype=torch.int32))
    d.step("balanced")
    torch.cuda.synchronize()
    want2 = d.out.clone()
    scrub_partials(d)
    d.step("single")
    torch.cuda.synchronize()
    assert torch.equal(d.out, want2)
    assert d.device_error() == 0


@pytest.mark.parametrize("tail", [(0, 1), (1, 1), (2, 3), (8, 8), (4, 1000)])
def test_planned_dynamic_tails_against_oracle(tail):
    """Any dynamic tail (none, the whole list claimed tile by tile, one chunk, ...) gives
    the oracle's output; the fused schedules (which use their own fixed tail) agree with
    the planner run with theirs."""
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.build_workload("tail", [9000, 64, 3000, 1, 0, 700, 130, 4096], 8, 2, "bf16", seed=21, poison=True)
    ref = oracle_out(w)
    for W in (1, 7, 40):
        d = DeviceStep(w, num_workers=W)
        print(f"tail {tail} W={W}", flush=True)
        d.step("balanced", tail_den=tail[0], tail_chunk=tail[1])
        torch.cuda.synchronize()
        assert d.device_error() == 0
        assert_within(d.output_f64(), ref, "bf16", f"tail {tail} W={W}")
        pa = d.plan_arrays()
        want = op.balanced_plan(w.seq_lens.tolist(), w.hkv, W, _lib.FUSED_MIN_TILES, _lib.FUSED_ITEM_COST, *tail)
        assert (pa["Ws"], pa["D"], pa["n_items"]) == (want["Ws"], want["D"], want["n_items"])


def test_tail_claim_counters_reset_across_launches():
    """Tail chunks are claimed on a counter in the plan workspace that the last workgroup
    returns to zero: repeated launches on one plan (no planner call in between) keep
    giving the same bits, and so do the fused schedules when they plan with a tail."""
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.build_workload("claims", [20000, 64, 3000, 1, 700, 129], 8, 2, "fp8", seed=13)
    d = DeviceStep(w, num_workers=31)
    d.step("balanced", tail_den=3, tail_chunk=2)
    torch.cuda.synchronize()
    want = d.out.clone()
    assert d.plan_arrays()["D"] > 0
    for rep in range(4):
        d.out.zero_()
        d.attend("balanced")
        torch.cuda.synchronize()
        assert torch.equal(d.out, want), rep
    assert d.device_error() == 0
    if _lib.FUSED_TAIL_DEN == 0:
        return
    d.step("balanced")
    torch.cuda.synchronize()
    want = d.out.clone()
    for rep in range(3):
        for sched in ("fused", "single", "balanced"):
            d.out.zero_()
            if sched == "single":
                scrub_partials(d)
            d.attend(sched)
            torch.cuda.synchronize()
            assert torch.equal(d.out, want), (rep, sched)
    assert d.device_error() == 0


def test_fused_reports_bad_lengths():
    w = inputs.build_workload("badf", [100, 200, 300], 8, 1, "bf16", seed=8)
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w, num_workers=6)
    d.seq_lens[1] = 64 * w.max_pages + 1
    d.step("fused")
    torch.cuda.synchronize()
    assert d.device_error(clear=True) & _lib.DEVERR_SEQ_LEN
    # the same on a batch planned in LDS (more than 256 sequences)
    wl = inputs.build_workload("badl", [100] * 300, 2, 1, "bf16", seed=8)
    dl = DeviceStep(wl, num_workers=40)
    dl.seq_lens[7] = -3
    dl.step("fused")
    torch.cuda.synchronize()
    assert dl.device_error(clear=True) & _lib.DEVERR_SEQ_LEN


def test_all_empty_and_zero_batch():
    w = inputs.build_workload("empty", [0, 0, 0], 8, 1, "bf16", seed=1, pool_pages=2)
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w, num_workers=4)
    d.out.fill_(1.0)
    d.step("balanced")
    torch.cuda.synchronize()
    assert np.all(d.output_f64() == 0)
    for sched in ("static_splits", "fused"):
        d.out.fill_(1.0)
        d.step(sched)
        torch.cuda.synchronize()
        assert np.all(d.output_f64() == 0)


def test_stream_read_probe_reads_every_slice():
    """The plain-read probe covers the whole buffer, ragged last slice included: a
    slice whose XOR equals the probe's constant (only the buffer's last 16 bytes are
    non-zero) is the only one that writes its sink word."""
    n16 = 1000
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    buf[-4] = int(np.array(0x9E3779B9, np.uint32).view(np.int32))
    for wgs, hit in ((3, 2), (1, 0), (7, 6)):
        sink = torch.zeros(16, dtype=torch.int32, device="cuda")
        print(f"probe wgs={wgs}", flush=True)
        _lib.hpa_probe_stream_read(buf, wgs, sink)
        torch.cuda.synchronize()
        want = np.zeros(16, np.int32)
        want[hit] = buf[-4].item()
        assert np.array_equal(sink.cpu().numpy(), want), (wgs, sink.cpu().numpy())


def _partials(d, W):
    """(acc [slots, G, 128], m [slots, G], l [slots, G]) of the partial workspace laid
    out for W workers (acc, then m, then l; m in log2 units)."""
    w = d.w
    S, G = w.batch * w.hkv, w.hq // w.hkv
    slots = 5 * W + S
    raw = d.partial_ws.cpu().numpy()
    f = raw[: slots * G * 130 * 4].view(np.float32)
    acc = f[: slots * G * 128].reshape(slots, G, 128)
    m = f[slots * G * 128: slots * G * 129].reshape(slots, G)
    l = f[slots * G * 129: slots * G * 130].reshape(slots, G)
    return acc.astype(np.float64), m.astype(np.float64), l.astype(np.float64)


@pytest.mark.parametrize("flavour", ["static_splits", "static_chunk"])
def test_static_schedule_structure_matches_oracle(flavour):
    """The GPU static split-KV schedule fills exactly the partial slots of
    oracle.planner.static_partition (S_split, chunk sizes, slot numbers), each with the
    softmax state (acc / l, max, sum) of its own tile range, and writes the rows of
    sequences with a single chunk directly -- checked on the hand-worked case and on
    the skewed workload at the default static worker count."""
    from load_balanced_split_amd.runner import DeviceStep
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "static_partitions.json")))
    cases = [(inputs.build_workload("static_golden", g["seq_lens"], 8, 1, "bf16", seed=14), g["num_workers"]),
             (inputs.config_workload(2), 0)]
    for w, W in cases:
        d = DeviceStep(w, num_workers=W)
        Ws = d.static_workers
        part = op.static_partition(w.seq_lens.tolist(), w.hkv, Ws, w.max_pages, flavour.split("_")[1])
        if W:
            assert [list(it) for it in part["items"]] == g[flavour.split("_")[1]]
        print(f"static structure {flavour} {w.name} W={Ws} S_split={part['S_split']}", flush=True)
        d.partial_ws.fill_(0xFF)                     # NaN everywhere: unwritten slots stay NaN
        d.out.fill_(float("nan"))
        d.attend(flavour, flags=_lib.ATTN_NO_MERGE)
        torch.cuda.synchronize()
        assert d.device_error() == 0
        acc, m, l = _partials(d, Ws)
        written = set(np.nonzero(np.isfinite(m[:, 0]))[0].tolist())
        assert written == {it[4] for it in part["items"] if it[4] >= 0}
        out = d.output_f64()
        qf = (w.q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        G = w.hq // w.hkv
        full = {}
        for s, k, t0, t1, slot in part["items"]:
            b, gh = divmod(s, w.hkv)
            L = int(w.seq_lens[b])
            if s not in full:
                full[s] = oa.gather_kv(w.k_cache, w.v_cache, w.page_table, b, gh, L, w.kv_dtype)
            K, V = full[s]
            lo, hi = t0 * 64, min(t1 * 64, L)
            for h in range(G):
                qh = qf[b, gh * G + h]
                if slot < 0:
                    want = oa.softmax_attention(qh, K, V, w.sm_scale)
                    assert np.all(np.abs(out[b, gh * G + h] - want) <= 1e-2 + 1e-2 * np.abs(want))
                    continue
                a_ref, m_ref, l_ref = oa.partial_state(qh, K[lo:hi], V[lo:hi], w.sm_scale)
                assert abs(m[slot, h] * np.log(2.0) - m_ref) <= 1e-3 * (1 + abs(m_ref)), (s, k, h)
                assert abs(l[slot, h] - l_ref) <= 1e-2 * l_ref, (s, k, h)
                o_ref = a_ref / l_ref
                assert np.all(np.abs(acc[slot, h] / l[slot, h] - o_ref) <= 1e-2 + 1e-2 * np.abs(o_ref)), (s, k, h)


def test_fused_and_single_schedules_above_the_lds_plan_limit():
    """4096 sequences (B = 512, Hkv = 8) -- more than the fused kernels plan in LDS: the
    fused and single-launch schedules plan in the workspace first and give the planned
    schedule's bits, empty requests and a bad length included."""
    rng = np.random.default_rng(52)
    lens = rng.integers(0, 200, size=512)
    lens[rng.random(512) < 0.1] = 0
    lens[7] = 9000
    w = inputs.build_workload("big_s", lens, 16, 8, "bf16", seed=53, poison=True)
    ref = oracle_out(w)
    outs = {}
    for sched in ("balanced", "fused", "single"):
        got, _, _ = run_and_compare(w, sched, 0, ref=ref, what="S=4096")
        outs[sched] = got
    assert np.array_equal(outs["balanced"], outs["fused"]) and np.array_equal(outs["balanced"], outs["single"])
    from load_balanced_split_amd.runner import DeviceStep
    d = DeviceStep(w, num_workers=100)
    d.seq_lens[3] = 64 * w.max_pages + 1
    for sched in ("fused", "single"):
        d.out.fill_(1.0)
        d.step(sched)
        torch.cuda.synchronize()
        assert d.device_error(clear=True) & _lib.DEVERR_SEQ_LEN, sched
        assert not bool(d.out[3].float().abs().sum()), sched        # a bad length gives a zero row


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_item_orders_and_in_kernel_merge_give_the_same_bits(cfg):
    """Every item order, with the merge kernel or merged inside the planned kernel
    (HPA_ATTN_MERGE_IN_KERNEL), gives the list-order planned schedule's bits (the
    E4M3 workload plans inside the prologue launch; its append is idempotent); the
    partial workspace is NaN-filled before every step."""
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.config_workload(cfg)
    d = DeviceStep(w)
    d.step("balanced")
    torch.cuda.synchronize()
    want = d.out.clone()
    assert_within(d.output_f64(), oracle_out(w), w.kv_dtype, f"cfg{cfg}")
    for order in (0, 1, 2):
        for sched in ("balanced", "balanced_inmerge"):
            print(f"cfg{cfg} order {order} {sched}", flush=True)
            d.out.zero_()
            scrub_partials(d)
            d.step(sched, item_order=order)
            torch.cuda.synchronize()
            assert d.device_error() == 0
            assert torch.equal(d.out, want), (order, sched)

"""Pins of the CPU planner: a hand-worked plan, brute force over tiles, properties."""

import json
import os

import numpy as np
import pytest

from oracle import planner as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_tiny_plan():
    g = json.load(open(os.path.join(GOLDEN, "plan_tiny_w4.json")))
    p = op.balanced_plan(g["seq_lens"], g["hkv"], g["num_workers"], g["min_tiles"])
    for key in ("C", "N", "Wp", "worker_off", "item_s", "item_t0", "item_t1", "item_split",
                "item_slot", "num_splits", "partial_base", "n_partials", "merge_list"):
        assert p[key] == g[key], key


def test_hand_worked_item_cost_plans():
    g = json.load(open(os.path.join(GOLDEN, "plan_item_cost.json")))
    for case in g["cases"]:
        p = op.balanced_plan(case["seq_lens"], case["hkv"], case["num_workers"], case["min_tiles"],
                             case["item_cost"])
        for key in ("C", "N", "Np", "Wp", "worker_off", "item_s", "item_t0", "item_t1", "item_split",
                    "item_slot", "num_splits", "partial_base", "n_partials", "merge_list"):
            assert p[key] == case[key], key


def brute_force_cost_plan(seq_lens, hkv, W, min_tiles, cost):
    """Lay the global list out position by position (cost virtual entries, then the
    real tiles, for every non-empty sequence), give each position to the worker whose
    range holds it by scanning the boundaries, then group real tiles by (worker, seq)."""
    seqs = [-(-int(L) // 64) for L in seq_lens for _ in range(hkv)]
    layout = []
    for s, n in enumerate(seqs):
        if n:
            layout += [None] * cost + [(s, t) for t in range(n)]
    Np = len(layout)
    if sum(seqs) == 0:
        return []
    Wp = min(W, max(1, Np // min_tiles))
    bounds = [w * Np // Wp for w in range(Wp + 1)]
    groups = {}
    for k, e in enumerate(layout):
        w = max(i for i in range(Wp) if bounds[i] <= k)
        if e is not None:
            groups.setdefault((w, e[0]), []).append(e[1])
    return [(w, s, ts[0], ts[-1] + 1) for (w, s), ts in sorted(groups.items())]


def test_item_cost_against_brute_force_random():
    rng = np.random.default_rng(1)
    for trial in range(300):
        B = int(rng.integers(1, 9))
        hkv = int(rng.integers(1, 4))
        lens = rng.choice([0, 1, 63, 64, 65, 127, 128, 129, 500, 1000], size=B)
        W = int(rng.integers(1, 40))
        mt = int(rng.integers(1, 4))
        c = int(rng.integers(0, 5))
        p = op.balanced_plan(lens, hkv, W, mt, c)
        items = []
        for w in range(p["Wp"]):
            for i in range(p["worker_off"][w], p["worker_off"][w + 1]):
                items.append((w, p["item_s"][i], p["item_t0"][i], p["item_t1"][i]))
        assert items == brute_force_cost_plan(lens, hkv, W, mt, c)


@pytest.mark.parametrize("seed", range(3))
def test_item_cost_properties(seed):
    """Every tile once; a worker's charged work (tiles + cost per item) is within
    one item cost of its share of the extended list; cost 0 is the plain plan."""
    rng = np.random.default_rng(100 + seed)
    for trial in range(200):
        B = int(rng.integers(0, 30))
        hkv = int(rng.integers(1, 5))
        lens = rng.integers(0, 5000, size=B)
        lens[rng.random(B) < 0.2] = 0
        W = int(rng.integers(1, 600))
        mt = int(rng.integers(1, 5))
        c = int(rng.integers(0, 9))
        p = op.balanced_plan(lens, hkv, W, mt, c)
        n = op.tile_counts(lens, hkv)
        if p["N"] == 0:
            assert p["Wp"] == 0 and p["n_items"] == 0
            continue
        assert p["Np"] == p["N"] + c * sum(1 for x in n if x > 0)
        cover = [np.zeros(x, int) for x in n]
        for s, t0, t1 in zip(p["item_s"], p["item_t0"], p["item_t1"]):
            cover[s][t0:t1] += 1
        assert all((x == 1).all() for x in cover)
        Np, Wp = p["Np"], p["Wp"]
        for w in range(Wp):
            share = (w + 1) * Np // Wp - w * Np // Wp
            idx = range(p["worker_off"][w], p["worker_off"][w + 1])
            charged = sum(p["item_t1"][i] - p["item_t0"][i] for i in idx) + c * len(idx)
            assert share - c <= charged <= share + c
        if c == 0:
            q = op.balanced_plan(lens, hkv, W, mt)
            assert all(p[k] == q[k] for k in q)


def test_hand_worked_dynamic_tail_plans():
    g = json.load(open(os.path.join(GOLDEN, "plan_dynamic_tail.json")))
    for case in g["cases"]:
        p = op.balanced_plan(case["seq_lens"], case["hkv"], case["num_workers"], case["min_tiles"],
                             case["item_cost"], case["tail_den"], case["tail_chunk"])
        for key in ("Np", "Wp", "Ws", "D", "V", "worker_off", "item_s", "item_t0", "item_t1", "item_split",
                    "item_slot", "num_splits", "partial_base", "n_partials", "merge_list"):
            assert p[key] == case[key], key


def brute_force_tail_plan(seq_lens, hkv, W, min_tiles, cost, tail_den, tail_chunk):
    """Position by position: lay out the list, give each position to the last virtual
    worker (W_s static ranges, then D tail chunks) whose boundary is at or before it,
    found by scanning the boundaries, then group real tiles by (virtual worker, sequence)."""
    seqs = [-(-int(L) // 64) for L in seq_lens for _ in range(hkv)]
    layout = []
    for s, n in enumerate(seqs):
        if n:
            layout += [None] * cost + [(s, t) for t in range(n)]
    Np = len(layout)
    if sum(seqs) == 0:
        return []
    Wp = min(W, max(1, Np // min_tiles))
    T = Np // tail_den if tail_den else 0
    D = min(-(-T // tail_chunk), 4 * W) if T else 0
    A = Np - T
    Ws = min(Wp, A)
    bounds = []
    for w in range(Ws):
        bounds.append((w * A) // Ws)
    for c in range(D):
        bounds.append(A + (c * T) // D)
    groups = {}
    for k, e in enumerate(layout):
        v = max(i for i in range(len(bounds)) if bounds[i] <= k)
        if e is not None:
            groups.setdefault((v, e[0]), []).append(e[1])
    return [(v, s, ts[0], ts[-1] + 1) for (v, s), ts in sorted(groups.items())]


def test_dynamic_tail_against_brute_force_random():
    rng = np.random.default_rng(2)
    for trial in range(300):
        B = int(rng.integers(1, 9))
        hkv = int(rng.integers(1, 4))
        lens = rng.choice([0, 1, 63, 64, 65, 127, 128, 129, 500, 1000, 3000], size=B)
        W = int(rng.integers(1, 30))
        mt = int(rng.integers(1, 4))
        c = int(rng.integers(0, 4))
        den = int(rng.integers(2, 9))
        ch = int(rng.integers(1, 5))
        p = op.balanced_plan(lens, hkv, W, mt, c, den, ch)
        items = []
        for v in range(p["V"]):
            for i in range(p["worker_off"][v], p["worker_off"][v + 1]):
                items.append((v, p["item_s"][i], p["item_t0"][i], p["item_t1"][i]))
        assert items == brute_force_tail_plan(lens, hkv, W, mt, c, den, ch)


@pytest.mark.parametrize("seed", range(3))
def test_dynamic_tail_properties(seed):
    """Every tile once; static ranges share A evenly, chunks share T evenly and hold at
    most tail_chunk positions; slots of a sequence consecutive in virtual-worker order."""
    rng = np.random.default_rng(200 + seed)
    for trial in range(200):
        B = int(rng.integers(1, 30))
        hkv = int(rng.integers(1, 5))
        lens = rng.integers(0, 6000, size=B)
        W = int(rng.integers(1, 400))
        c = int(rng.integers(0, 6))
        den = int(rng.integers(2, 17))
        ch = int(rng.integers(1, 9))
        p = op.balanced_plan(lens, hkv, W, 1, c, den, ch)
        n = op.tile_counts(lens, hkv)
        if p["N"] == 0:
            assert p["V"] == 0 and p["n_items"] == 0
            continue
        Np, Wp, D = p["Np"], p["Wp"], p["D"]
        T = Np // den
        Ws = p["Ws"]
        assert D == min(-(-T // ch), 4 * W) and Ws == min(Wp, Np - T) and p["V"] == Ws + D
        # every virtual worker owns at least one position
        bounds = [v * (Np - T) // Ws for v in range(Ws)] + [Np - T + i * T // D for i in range(D)] + [Np]
        assert all(bounds[v] < bounds[v + 1] for v in range(p["V"]))
        cover = [np.zeros(x, int) for x in n]
        for s, t0, t1 in zip(p["item_s"], p["item_t0"], p["item_t1"]):
            cover[s][t0:t1] += 1
        assert all((x == 1).all() for x in cover)
        if D:
            sizes = [(i + 1) * T // D - i * T // D for i in range(D)]
            assert max(sizes) - min(sizes) <= 1
            assert max(sizes) <= ch or D == 4 * W
        per_seq = {}
        for i, s in enumerate(p["item_s"]):
            per_seq.setdefault(s, []).append(i)
        for s, idx in per_seq.items():
            assert [p["item_split"][i] for i in idx] == list(range(len(idx)))
            if len(idx) > 1:
                assert [p["item_slot"][i] for i in idx] == list(range(p["partial_base"][s], p["partial_base"][s] + len(idx)))


def brute_force_plan(seq_lens, hkv, W, min_tiles):
    """Enumerate global tiles one by one: owner worker by scanning the worker
    boundaries, owner sequence by scanning the sequence boundaries, then group."""
    seqs = []
    for b, L in enumerate(seq_lens):
        for g in range(hkv):
            seqs.append(-(-int(L) // 64))
    N = sum(seqs)
    if N == 0:
        return []
    Wp = min(W, max(1, N // min_tiles))
    bounds = [w * N // Wp for w in range(Wp + 1)]
    groups = {}
    k = 0
    for s, n in enumerate(seqs):
        for t in range(n):
            w = max(i for i in range(Wp) if bounds[i] <= k)
            groups.setdefault((w, s), []).append(t)
            k += 1
    return [(w, s, ts[0], ts[-1] + 1) for (w, s), ts in sorted(groups.items())]


def test_against_brute_force_random():
    rng = np.random.default_rng(0)
    for trial in range(300):
        B = int(rng.integers(1, 9))
        hkv = int(rng.integers(1, 4))
        lens = rng.choice([0, 1, 63, 64, 65, 127, 128, 129, 500, 1000], size=B)
        W = int(rng.integers(1, 40))
        mt = int(rng.integers(1, 4))
        p = op.balanced_plan(lens, hkv, W, mt)
        items = []
        for w in range(p["Wp"]):
            for i in range(p["worker_off"][w], p["worker_off"][w + 1]):
                items.append((w, p["item_s"][i], p["item_t0"][i], p["item_t1"][i]))
        assert items == brute_force_plan(lens, hkv, W, mt)


@pytest.mark.parametrize("seed", range(5))
def test_plan_properties(seed):
    rng = np.random.default_rng(seed)
    for trial in range(200):
        B = int(rng.integers(0, 40))
        hkv = int(rng.integers(1, 5))
        lens = rng.integers(0, 5000, size=B)
        lens[rng.random(B) < 0.2] = 0
        W = int(rng.integers(1, 600))
        mt = int(rng.integers(1, 9))
        p = op.balanced_plan(lens, hkv, W, mt)
        N, Wp = p["N"], p["Wp"]
        n = op.tile_counts(lens, hkv)
        assert N == sum(n)
        if N == 0:
            assert Wp == 0 and p["n_items"] == 0
            continue
        assert 1 <= Wp <= W and (Wp == 1 or N // Wp >= mt or Wp == W)
        # every (s, tile) covered exactly once
        cover = [np.zeros(x, int) for x in n]
        for s, t0, t1 in zip(p["item_s"], p["item_t0"], p["item_t1"]):
            assert 0 <= t0 < t1 <= n[s]
            cover[s][t0:t1] += 1
        assert all((c == 1).all() for c in cover)
        # per-worker load differs by at most one tile
        loads = [sum(p["item_t1"][i] - p["item_t0"][i] for i in range(p["worker_off"][w], p["worker_off"][w + 1]))
                 for w in range(Wp)]
        assert set(loads) <= {N // Wp, -(-N // Wp)}
        # items of a sequence: consecutive ranks, contiguous tiles, consecutive slots
        per_seq = {}
        for i, s in enumerate(p["item_s"]):
            per_seq.setdefault(s, []).append(i)
        slots = []
        for s, idx in per_seq.items():
            assert [p["item_split"][i] for i in idx] == list(range(len(idx)))
            assert p["num_splits"][s] == len(idx)
            assert p["item_t0"][idx[0]] == 0 and p["item_t1"][idx[-1]] == n[s]
            for a, b in zip(idx[:-1], idx[1:]):
                assert p["item_t1"][a] == p["item_t0"][b]
            if len(idx) == 1:
                assert p["item_slot"][idx[0]] == -1
            else:
                sl = [p["item_slot"][i] for i in idx]
                assert sl == list(range(p["partial_base"][s], p["partial_base"][s] + len(idx)))
                slots += sl
        assert sorted(slots) == list(range(p["n_partials"]))
        assert p["n_items"] <= Wp + len(n)
        assert p["merge_list"] == [s for s in range(len(n)) if p["num_splits"][s] != 1]


@pytest.mark.parametrize("flavour", ["splits", "chunk"])
def test_static_partition_covers_every_tile(flavour):
    rng = np.random.default_rng(7)
    for trial in range(200):
        B = int(rng.integers(1, 20))
        hkv = int(rng.integers(1, 3))
        lens = rng.integers(0, 3000, size=B)
        maxp = max(1, int(-(-lens.max() // 64)))
        W = int(rng.integers(1, 300))
        p = op.static_partition(lens, hkv, W, maxp, flavour)
        n = op.tile_counts(lens, hkv)
        cover = [np.zeros(x, int) for x in n]
        nslot = {}
        for s, k, t0, t1, slot in p["items"]:
            assert k < p["S_split"]
            cover[s][t0:t1] += 1
            nslot.setdefault(s, []).append(slot)
        assert all((c == 1).all() for c in cover)
        for s, sl in nslot.items():
            assert (sl == [-1]) if len(sl) == 1 else all(x >= 0 for x in sl)


def test_skewed_workload_static_vs_balanced_shape():
    """1 x 131072 + 31 x 4096 tokens, 512 workers: the balanced plan gives every
    worker 7 or 8 tiles, the static one leaves the long request's 16 chunks at
    128 tiles each -- the long tail the pages describe."""
    lens = [131072] + [4096] * 31
    p = op.balanced_plan(lens, 1, 512, 1)
    loads = [sum(p["item_t1"][i] - p["item_t0"][i] for i in range(p["worker_off"][w], p["worker_off"][w + 1]))
             for w in range(p["Wp"])]
    assert p["N"] == 4032 and max(loads) == 8 and min(loads) == 7
    st = op.static_partition(lens, 1, 512, 2048, "splits")
    assert st["S_split"] == 16
    assert max(t1 - t0 for _, _, t0, t1, _ in st["items"]) == 128


def test_static_partitions_hand_worked():
    """Both static flavours against a hand-worked case in which they differ (a
    'chunk' partition that split nothing, or split like 'splits', fails)."""
    g = json.load(open(os.path.join(GOLDEN, "static_partitions.json")))
    for flavour in ("splits", "chunk"):
        p = op.static_partition(g["seq_lens"], g["hkv"], g["num_workers"], g["max_pages"], flavour)
        assert p["S_split"] == g["S_split"]
        assert [list(it) for it in p["items"]] == g[flavour], flavour


def test_hand_worked_item_orders():
    """Item orders on a hand-worked case: ranks and slots travel with their items."""
    g = json.load(open(os.path.join(GOLDEN, "plan_item_order.json")))
    for case in g["cases"]:
        p = op.balanced_plan(case["seq_lens"], case["hkv"], case["num_workers"], case["min_tiles"],
                             case["item_cost"], 0, 1, case["item_order"])
        for key in ("worker_off", "item_s", "item_t0", "item_t1", "item_split", "item_slot", "num_splits",
                    "partial_base"):
            assert p[key] == case[key], (case["item_order"], key)


def test_item_orders_permute_only_within_workers():
    """Any order holds the same (worker, item) set as list order, each worker's items
    split into whole sequences and shared pieces in the stated order, each class in
    sequence order, with unchanged ranks and slots."""
    rng = np.random.default_rng(7)
    for trial in range(300):
        B = int(rng.integers(0, 40))
        hkv = int(rng.integers(1, 4))
        lens = rng.integers(0, 4000, size=B)
        lens[rng.random(B) < 0.2] = 0
        W = int(rng.integers(1, 200))
        mt, c = int(rng.integers(1, 5)), int(rng.integers(0, 6))
        den = int(rng.integers(0, 5)) if trial % 2 else 0
        ch = int(rng.integers(1, 9))
        base = op.balanced_plan(lens, hkv, W, mt, c, den, ch, 0)
        for order in (1, 2):
            p = op.balanced_plan(lens, hkv, W, mt, c, den, ch, order)
            assert p["worker_off"] == base["worker_off"] and p["n_items"] == base["n_items"]
            for w in range(p["V"]):
                lo, hi = p["worker_off"][w], p["worker_off"][w + 1]
                got = list(zip(*(p[k][lo:hi] for k in ("item_s", "item_t0", "item_t1", "item_split", "item_slot"))))
                want = list(zip(*(base[k][lo:hi] for k in ("item_s", "item_t0", "item_t1", "item_split", "item_slot"))))
                assert sorted(got) == sorted(want)
                split = [p["num_splits"][it[0]] > 1 for it in got]
                first = [not x for x in split] if order == 1 else split
                assert first == sorted(first, reverse=True)          # one class, then the other
                for cls in (True, False):
                    ss = [it[0] for it, x in zip(got, split) if x == cls]
                    assert ss == sorted(ss)

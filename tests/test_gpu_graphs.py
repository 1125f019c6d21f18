"""HIP-graph capture of a whole step: each schedule's step (and the router call)
captured once, then replayed several times with other eager work and
synchronisations between the replays; every replay must reproduce the eager
result bit for bit (counters and workspaces return to their start state within
each launch, and no captured node clears memory)."""

import numpy as np
import pytest

from load_balanced_split_amd import _lib, inputs
from tests.helpers import ensure_built

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    _lib.lib()


def _replays(step, other, out, reps=3, scrub=None):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(reps):
        other()                                   # eager work between replays
        torch.cuda.synchronize()
        for t in out:
            t.zero_()
        if scrub is not None:
            scrub()                               # outside the graph: stale data turns into NaN
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(out, ref):
            assert torch.equal(t, r)
    del g


@pytest.mark.parametrize("kv_dtype,prologue", [("bf16", False), ("fp8", True)])
def test_attention_step_graph_replays_match_eager(kv_dtype, prologue):
    from load_balanced_split_amd.runner import DeviceStep
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 5000, size=24)
    lens[3] = 40000
    w = inputs.build_workload("graph", lens, 8, 1, kv_dtype, seed=4, prologue=prologue)
    d = DeviceStep(w)
    for sched in ("balanced", "fused", "single"):
        print(f"graph {kv_dtype} prologue={prologue} {sched}", flush=True)
        _replays(lambda: d.step(sched), lambda: d.step("static_splits"), [d.out],
                 scrub=(lambda: d.partial_ws.fill_(0xFF)) if sched == "single" else None)
        assert d.device_error() == 0


def test_router_graph_replays_match_eager():
    from load_balanced_split_amd.runner import RouterStep
    for T in (1, 64, 300):
        print(f"graph router T={T}", flush=True)
        r = RouterStep(inputs.router_workload(T, 256, 1024, seed=T), top_k=8)
        _replays(lambda: r.run(2), lambda: r.run(1), [r.logits, r.topk_idx, r.topk_val])


def test_moe_graph_replays_match_eager():
    """The fused MoE call, few-pair (one token) and grouped (20 tokens) paths, captured once
    and replayed with a different batch's call and a NaN-filled workspace between replays."""
    from load_balanced_split_amd.runner import MoeStep
    other = MoeStep(inputs.moe_workload(3, 16, 4, 256, 128, seed=5))
    for T in (1, 20):
        print(f"graph moe T={T}", flush=True)
        m = MoeStep(inputs.moe_workload(T, 16, 4, 256, 128, seed=T))
        _replays(m.run, other.run, [m.out], scrub=lambda: m.workspace.fill_(0xFF))
        assert int(m.err.item()) == 0

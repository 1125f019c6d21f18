"""The allocation-free entry point (hpa_decode_attn_noalloc) through the C ABI:
its output equals hpa_decode_attn's with caller-given workspaces, bit for bit,
on two calls in a row (the second on a smaller batch, so the workspaces inside
the library's scratch array move), for every schedule it runs, and matches the
oracle; oversized shapes are refused before anything is launched."""

import numpy as np
import pytest

from load_balanced_split_amd import _lib, inputs
from oracle import attention as oa
from tests.helpers import assert_within, ensure_built

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    _lib.lib()


def _noalloc_out(d, sched, W, err):
    q, lens = d.attn_inputs()
    out = torch.full_like(d.out, float("nan"))
    _lib.hpa_decode_attn_noalloc(d.desc, sched, q, d.k_cache, d.v_cache, d.k_scale, d.v_scale, lens,
                                 d.page_table, W, out, err)
    return out


@pytest.mark.parametrize("sched", ["fused", "single", "static_splits", "static_chunk"])
def test_noalloc_matches_workspace_call(sched):
    from load_balanced_split_amd.runner import DeviceStep
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    big = inputs.build_workload("noalloc_big", [131072 // 4] + [4096] * 15 + [0, 1, 63, 700], 8, 1, "bf16",
                                seed=41, poison=True)
    small = inputs.build_workload("noalloc_small", [5000, 64, 3000, 129], 16, 2, "fp8", seed=42, poison=True)
    for w, W in ((big, 0), (small, 37)):
        d = DeviceStep(w, num_workers=W)
        Wd = d.static_workers if sched.startswith("static") else d.num_workers
        print(f"noalloc {sched} {w.name} W={Wd}", flush=True)
        d.attend(sched)
        torch.cuda.synchronize()
        want = d.out.clone()
        got = _noalloc_out(d, sched, Wd, err)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (sched, w.name)
        assert int(err.item()) == 0
        ref = oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, w.hkv, w.sm_scale,
                                  w.kv_dtype, w.k_scale, w.v_scale)
        assert_within(got.float().cpu().numpy().astype(np.float64), ref, w.kv_dtype, f"noalloc {sched} {w.name}")


def test_noalloc_reports_device_errors_and_refuses_large_shapes():
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.build_workload("noalloc_bad", [100, 200, 300], 8, 1, "bf16", seed=8)
    w.page_table[1, 2] = w.num_pages + 5
    d = DeviceStep(w, num_workers=6)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _noalloc_out(d, "fused", 6, err)
    torch.cuda.synchronize()
    assert int(err.item()) & _lib.DEVERR_PAGE_ID
    # more workers, sequences or bytes than the scratch array holds: refused, nothing launched
    for desc, W, sched in ((_lib.make_desc(4, 8, 1, 9, 16), 5000, "fused"),
                           (_lib.make_desc(3000, 8, 1, 9, 16), 64, "fused"),
                           (_lib.make_desc(2048, 16, 1, 9, 16), 4096, "single"),
                           (_lib.make_desc(4, 8, 1, 9, 16), 64, "balanced")):
        with pytest.raises(_lib.HpaError) as e:
            _lib.hpa_decode_attn_noalloc(desc, sched, d.q, d.k_cache, d.v_cache, None, None, d.seq_lens,
                                         d.page_table, W, d.out, err)
        assert e.value.status == (1 if sched == "balanced" else 2), (W, sched)

"""The C-ABI library loads, exports every declared symbol, and its host-side
validation answers without touching a GPU."""

import ctypes

import pytest

from load_balanced_split_amd import _lib
from tests.helpers import ensure_built


@pytest.fixture(scope="module")
def L():
    ensure_built()
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = _lib.declared_symbols()
    assert {"hpa_plan", "hpa_decode_attn", "hpa_decode_prologue"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    d = _lib.make_desc(4, 8, 1, 9, 16)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_status_strings(L):
    assert _lib.hpa_status_string(0) == "ok"
    assert "workspace" in _lib.hpa_status_string(3)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 2), ("page_size", 16, 2), ("num_kv_heads", 5, 1), ("num_q_heads", 34, 1),
    ("batch", -1, 1), ("max_pages_per_seq", 0, 1), ("sm_scale", 0.0, 1), ("kv_dtype", 7, 1)])
def test_descriptor_validation(L, field, value, status):
    d = _desc(**{field: value})
    if field == "num_q_heads" and value == 34:
        d.num_kv_heads = 2          # group 17 > 16
        status = 2
    n = ctypes.c_size_t(0)
    assert L.hpa_plan_workspace_size(ctypes.byref(d), 512, ctypes.byref(n)) == status
    assert _lib.hpa_last_error_message()


def test_workspace_sizes_and_layout(L):
    d = _desc()
    lay = _lib.hpa_plan_workspace_layout(d, 512)
    assert lay["max_items"] == 5 * 512 + 4        # at most 4 W tail chunks
    offs = [lay[k] for k in ("header", "C", "worker_off", "item_s", "item_t0", "item_t1", "item_split",
                             "item_slot", "num_splits", "partial_base", "merge_list")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert _lib.hpa_plan_workspace_size(d, 512) == lay["total_bytes"]
    # (5 W + S) slots x G heads x (128 acc + m + l) fp32
    assert _lib.hpa_partial_workspace_size(d, 512) == (5 * 512 + 4) * 8 * (128 + 2) * 4


def test_calls_reject_bad_arguments_before_launching(L):
    d = _desc()
    with pytest.raises(_lib.HpaError) as e:
        L_status = L.hpa_plan(ctypes.byref(d), None, 512, 1, 0, 0, 1, 0, None, 0, None)
        _lib._check(L_status, "hpa_plan")
    assert e.value.status == 1
    # undersized plan workspace -> HPA_ERR_WORKSPACE, nothing launched
    fake = ctypes.c_void_p(0x1000)
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 1, 0, 0, 1, 0, fake, 16, None) == 3
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 0, 0, 0, 1, 0, fake, 1 << 30, None) == 1     # min_tiles < 1
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 1, -1, 0, 1, 0, fake, 1 << 30, None) == 1    # item cost < 0
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 1, 65, 0, 1, 0, fake, 1 << 30, None) == 1    # item cost > 64
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 1, 0, -1, 1, 0, fake, 1 << 30, None) == 1    # tail_den < 0
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 1, 0, 8, 0, 0, fake, 1 << 30, None) == 1     # tail_chunk < 1
    assert L.hpa_plan(ctypes.byref(d), fake, 512, 1, 0, 0, 1, 3, fake, 1 << 30, None) == 1     # item_order > 2
    # sizes beyond the 32-bit plan offsets: more than 2^20 workers, 2^24 sequences
    n = ctypes.c_size_t(0)
    assert L.hpa_plan_workspace_size(ctypes.byref(d), (1 << 20) + 1, ctypes.byref(n)) == 1
    assert L.hpa_plan(ctypes.byref(d), fake, (1 << 20) + 1, 1, 0, 0, 1, 0, fake, 1 << 30, None) == 1
    big = _desc(batch=1 << 22, num_q_heads=8, num_kv_heads=8)
    assert L.hpa_plan_workspace_size(ctypes.byref(big), 512, ctypes.byref(n)) == 1
    # balanced attention without a plan, fp8 without scales
    args = [fake] * 7
    assert L.hpa_decode_attn(ctypes.byref(d), 0, *args, 512, None, 0, fake, 1 << 30, fake, 0, None) == 1
    d8 = _desc(kv_dtype=1)
    assert L.hpa_decode_attn(ctypes.byref(d8), 1, fake, fake, fake, None, None, fake, fake, 512, None, 0,
                             fake, 1 << 30, fake, 0, None) == 1
    # partial workspace too small
    assert L.hpa_decode_attn(ctypes.byref(d), 1, fake, fake, fake, None, None, fake, fake, 512, None, 0,
                             fake, 100, fake, 0, None) == 3
    # unknown flags, both halves switched off, the in-kernel merge flag off the planned schedule
    # or with a half switched off
    assert L.hpa_decode_attn(ctypes.byref(d), 0, fake, fake, fake, None, None, fake, fake, 512, fake, 1 << 30,
                             fake, 1 << 30, fake, 5, None) == 1
    for bad in (3, 4, 8, -1):
        assert L.hpa_decode_attn(ctypes.byref(d), 1, fake, fake, fake, None, None, fake, fake, 512, None, 0,
                                 fake, 1 << 30, fake, bad, None) == 1
    # prologue: aliasing positions / seq_lens_out is refused
    assert L.hpa_decode_prologue(ctypes.byref(d), fake, fake, fake, fake, fake, 1e-6, 1e6, fake, fake, fake,
                                 fake, None, None, fake, fake, None, None) == 1
    # prologue + plan: the rules of both calls, and plan_ws is required
    P = [fake] * 5
    pro = lambda desc, W, mt, cost, den, ch, ws, nbytes: L.hpa_decode_prologue_plan(
        ctypes.byref(desc), *P, 1e-6, 1e6, fake, fake, fake, fake, None, None, fake,
        ctypes.c_void_p(0x2000), W, mt, cost, den, ch, 0, ws, nbytes, None)
    assert pro(d, 512, 1, 4, 0, 1, None, 0) == 1                       # no plan workspace
    assert pro(d, 512, 1, 4, 0, 1, fake, 16) == 3                      # workspace too small
    assert pro(d, 512, 0, 4, 0, 1, fake, 1 << 30) == 1                 # min_tiles < 1
    assert pro(d, 512, 1, 65, 0, 1, fake, 1 << 30) == 1                # item cost > 64
    assert pro(d, 512, 1, 4, 1, 0, fake, 1 << 30) == 1                 # tail_chunk < 1
    assert pro(d8, 512, 1, 4, 0, 1, fake, 1 << 30) == 1                # E4M3 without scales
    assert L.hpa_decode_prologue_plan(ctypes.byref(d), *P, 1e-6, 1e6, fake, fake, fake, fake, None, None, fake,
                                      fake, 512, 1, 4, 0, 1, 0, fake, 1 << 30, None) == 1   # positions = seq_lens_out
    # default worker count: an unknown schedule or a NULL output is refused before any device query
    n = ctypes.c_int32(0)
    assert L.hpa_default_num_workers(0, 7, ctypes.byref(n)) == 1
    assert L.hpa_default_num_workers(0, 0, None) == 1
    # single-launch schedule: partials the in-kernel merge cannot address with 32-bit
    # offsets (16 heads per KV head, 200k workers: > 4 GiB of partial slots) are refused
    d16 = _desc(num_q_heads=16)
    huge = ctypes.c_size_t(1 << 40)
    assert L.hpa_decode_attn(ctypes.byref(d16), 4, fake, fake, fake, None, None, fake, fake, 200000, fake, huge,
                             fake, huge, fake, 0, None) == 2
    assert "32-bit" in _lib.hpa_last_error_message()
    # the same shape on the fused schedule (merge kernel) passes that check
    assert L.hpa_decode_attn(ctypes.byref(d16), 3, fake, fake, fake, None, None, fake, fake, 200000, None, 0,
                             fake, huge, fake, 0, None) == 1            # ... and stops at the missing plan_ws
    # allocation-free call: schedules that need a plan, and shapes beyond its scratch array,
    # are refused before anything touches the device
    na = lambda desc, sched, W: L.hpa_decode_attn_noalloc(ctypes.byref(desc), sched, fake, fake, fake, None, None,
                                                          fake, fake, W, fake, None, None)
    assert na(d, 0, 64) == 1                                          # HPA_SCHED_BALANCED needs hpa_plan
    assert na(d, 3, 5000) == 2                                        # more than 4096 workers
    assert na(_desc(batch=3000), 3, 64) == 2                          # more than 2048 sequences
    assert na(_desc(batch=2048, num_q_heads=16), 4, 4096) == 2        # workspaces beyond 32 MiB
    assert na(_desc(batch=0), 3, 64) == 0                             # empty batch: nothing to do
    # row-major page packing: count must cover the pool without a page list, no in-place
    # conversion through a page list, 16-byte aligned pointers, head_dim 128
    pk = lambda desc, kr, pages, n, kc: L.hpa_kv_pack_pages(ctypes.byref(desc), kr, kr, pages, n, kc, kc, None, None)
    other = ctypes.c_void_p(0x20000)
    assert pk(d, fake, None, 15, other) == 1                      # num_pages is 16
    assert pk(d, fake, fake, 4, fake) == 1                        # in place with a page list
    assert pk(d, ctypes.c_void_p(0x1004), None, 16, other) == 1   # misaligned
    assert pk(d, fake, fake, -1, other) == 1
    assert pk(_desc(head_dim=64), fake, None, 16, other) == 2
    assert pk(d, fake, fake, 0, other) == 0                       # nothing to pack
    # empty batch is a no-op
    d0 = _desc(batch=0)
    assert L.hpa_decode_attn(ctypes.byref(d0), 1, None, None, None, None, None, None, None, 512, None, 0,
                             None, 0, None, 0, None) == 0


def test_valu_product_build_exports_and_limits(L):
    """The comparison build (VALU products) exports the same symbols and refuses
    query groups larger than 8 heads, which the library build accepts."""
    import os
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libhpa_valu.so")
    if not os.path.exists(path):
        pytest.skip("libhpa_valu.so not built")
    V = ctypes.CDLL(path)
    for n in _lib.declared_symbols():
        assert hasattr(V, n), n
    n = ctypes.c_size_t(0)
    for hq, status_valu in ((8, 0), (16, 2)):
        d = _desc(num_q_heads=hq)
        V.hpa_plan_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        assert V.hpa_plan_workspace_size(ctypes.byref(d), 512, ctypes.byref(n)) == status_valu
        assert L.hpa_plan_workspace_size(ctypes.byref(d), 512, ctypes.byref(n)) == 0


def test_stream_read_probe_validation(L):
    buf, sink = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    f = L.hpa_probe_stream_read
    assert f(buf, 17, 4, sink, None) == 1                     # not a multiple of 16
    assert f(buf, 0, 4, sink, None) == 1                      # empty
    assert f(ctypes.c_void_p(4100), 64, 4, sink, None) == 1   # misaligned
    assert f(None, 64, 4, sink, None) == 1
    assert f(buf, 64, 4, None, None) == 1
    assert f(buf, 64, -1, sink, None) == 1


def test_router_validation_and_workspace_size(L):
    n = ctypes.c_size_t(0)
    ws = L.hpa_router_workspace_size
    assert ws(1, 256, 7168, ctypes.byref(n)) == 0
    # one token, 16 expert blocks: 112 K ranges of 2 chunks, 4 per workgroup -> 28 partial sums per logit
    assert n.value == 28 * 1 * 256 * 4
    assert ws(0, 256, 7168, ctypes.byref(n)) == 0 and n.value == 0
    # many tokens: 128 x 128 tiles (2 x 32 of them), 8 K ranges for 512 workgroups -> 8 partial sums
    assert ws(4096, 256, 7168, ctypes.byref(n)) == 0 and n.value == 8 * 4096 * 256 * 4
    for T, E, H, status in ((1, 8, 64, 2), (1, 1040, 64, 2), (1, 24, 64, 2), (1, 16, 48, 2), (1, 16, 0, 2),
                            (1, 16, 1 << 17, 2), (-1, 16, 64, 1), ((1 << 20) + 1, 16, 64, 1)):
        assert ws(T, E, H, ctypes.byref(n)) == status, (T, E, H)
    p, q = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    g = L.hpa_router_gemm
    big = ctypes.c_size_t(1 << 30)
    assert g(p, p, 4, 64, 64, 3, q, 2, q, q, p, big, None) == 1            # passes
    assert g(p, p, 4, 64, 64, 2, q, 33, q, q, p, big, None) == 1           # top_k > 32
    assert g(p, p, 4, 16, 64, 2, q, 17, q, q, p, big, None) == 1           # top_k > experts
    assert g(p, p, 4, 64, 64, 2, q, 2, None, q, p, big, None) == 1         # top-k outputs missing
    assert g(None, p, 4, 64, 64, 2, q, 2, q, q, p, big, None) == 1
    assert g(ctypes.c_void_p(4100), p, 4, 64, 64, 2, q, 2, q, q, p, big, None) == 1   # misaligned x
    assert g(p, p, 4, 64, 64, 2, q, 2, q, q, p, ctypes.c_size_t(16), None) == 3       # workspace
    assert g(None, None, 0, 64, 64, 2, None, 0, None, None, None, ctypes.c_size_t(0), None) == 0   # no tokens
    pk = L.hpa_router_pack_weights
    assert pk(None, 64, 64, p, None) == 1
    assert pk(ctypes.c_void_p(4100), 64, 64, p, None) == 1
    assert pk(p, 20, 64, p, None) == 2


def test_moe_validation_and_workspace_size(L):
    """The MoE calls refuse bad shapes, pointers and workspaces on the host, before any
    launch (no GPU needed)."""
    n = ctypes.c_size_t(0)
    ws = L.hpa_moe_workspace_size
    al = lambda x: (x + 255) // 256 * 256
    T, K, H, I = 32, 8, 2048, 768
    P = T * K
    assert ws(T, K, H, I, ctypes.byref(n)) == 0
    want = (al(T * H) + al(T * 4) + al(P * 4) + al(3 * P * 4) + al(4) + al(P * I * 4) + al(P * (I // 16) * 4)
            + al(P * I) + al(P * 4) + al(P * H * 4))
    assert n.value == want
    for args, status in (((1025, 1, 128, 128), 2), ((1, 0, 128, 128), 2), ((1, 17, 128, 128), 2),
                         ((1, 1, 64, 128), 2), ((1, 1, 128, 200), 2), ((1, 1, 4224, 128), 2),
                         ((1024, 16, 128, 128), 0), ((-1, 1, 128, 128), 2)):
        assert ws(*args, ctypes.byref(n)) == status, args
    assert ws(1, 1, 128, 128, None) == 1
    f = L.hpa_moe_fused
    p, q = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    fp = ctypes.cast(p, ctypes.POINTER(ctypes.c_float))
    ip = ctypes.cast(p, ctypes.POINTER(ctypes.c_int32))
    big = ctypes.c_size_t(1 << 40)
    ok = dict(x=p, ids=ip, wts=fp, w1=p, s1=fp, w2=p, s2=fp, T=4, E=8, K=2, H=128, I=128, out=q, ws=p,
              bytes=big, err=None, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["ids"], a["wts"], a["w1"], a["s1"], a["w2"], a["s2"], a["T"], a["E"], a["K"], a["H"],
                 a["I"], a["out"], a["ws"], a["bytes"], a["err"], a["stream"])
    assert call(E=1025) == 2 and call(K=0) == 2 and call(H=100) == 2 and call(T=1025) == 2
    assert call(x=None) == 1 and call(out=None) == 1 and call(ws=None) == 1
    assert call(out=ctypes.c_void_p(8200)) == 1                           # misaligned
    assert call(bytes=ctypes.c_size_t(1024)) == 3                         # workspace too small
    assert call(T=0) == 0                                                 # nothing to do, nothing launched
    pk = L.hpa_moe_pack_weights
    assert pk(p, 8, 24, 128, q, None) == 2                                # rows not a multiple of 16
    assert pk(p, 8, 32, 100, q, None) == 2                                # cols not a multiple of 128
    assert pk(p, 0, 32, 128, q, None) == 2
    assert pk(None, 8, 32, 128, q, None) == 1
    assert pk(p, 8, 32, 128, p, None) == 1                                # in place
    assert pk(ctypes.c_void_p(4100), 8, 32, 128, q, None) == 1            # misaligned

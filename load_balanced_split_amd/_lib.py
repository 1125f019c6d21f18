"""ctypes binding of libhpa (include/hpa.h): argument marshalling only.

Every call takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI, and raises HpaError on
a non-OK status. All arithmetic happens in the library's HIP kernels; there is
no CPU fallback: if libhpa.so is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# HPA_TRACE=1 selects the instrumented build (per-wave timestamps and CU ids of
# the attention kernels, written after the partial results in the workspace);
# HPA_PRODUCTS=valu the comparison build whose attention kernels compute both
# products with VALU dot products instead of MFMA (query groups of up to 8 heads).
TRACE = os.environ.get("HPA_TRACE", "0") == "1"
PRODUCTS = os.environ.get("HPA_PRODUCTS", "mfma")
if PRODUCTS not in ("mfma", "valu"):
    raise ValueError(f"HPA_PRODUCTS={PRODUCTS!r}: expected mfma or valu")
if TRACE and PRODUCTS != "mfma":
    raise ValueError("HPA_TRACE=1 and HPA_PRODUCTS=valu select different builds")
LIB_PATH = os.path.join(PKG, "libhpa_trace.so" if TRACE else
                        "libhpa_valu.so" if PRODUCTS == "valu" else "libhpa.so")
TRACE_WAVES, TRACE_WORDS, TRACE_START, TRACE_ITEMS, TRACE_UNITS = 4, 68, 4, 4, 48
HEADER = os.path.join(os.path.dirname(PKG), "include", "hpa.h")

HPA_KV_BF16, HPA_KV_FP8_E4M3 = 0, 1
HPA_SCHED_BALANCED, HPA_SCHED_STATIC_SPLITS, HPA_SCHED_STATIC_CHUNK, HPA_SCHED_BALANCED_FUSED = 0, 1, 2, 3
HPA_SCHED_BALANCED_SINGLE = 4
SCHED = {"balanced": 0, "static_splits": 1, "static_chunk": 2, "fused": 3, "single": 4}
DEVERR_SEQ_LEN, DEVERR_PAGE_ID, DEVERR_PROLOGUE, DEVERR_PLAN, DEVERR_MOE_EXPERT = 1, 2, 4, 8, 16
ATTN_NO_MERGE, ATTN_MERGE_ONLY, ATTN_MERGE_IN_KERNEL = 1, 2, 4
HEADER_SLOTS = dict(Wp=0, N=1, S=2, n_items=3, n_merge=4, n_partials=5, error=6, W=7, D=8, Ws=9)


def _header_define(name: str) -> int:
    m = re.search(rf"^#define\s+{name}\s+(\d+)", open(HEADER).read(), re.M)
    if not m:
        raise RuntimeError(f"{name} not defined in {HEADER}")
    return int(m.group(1))


# what the fused schedule plans with (hpa_plan with these gives its items exactly)
FUSED_ITEM_COST = _header_define("HPA_FUSED_ITEM_COST")
FUSED_MIN_TILES = _header_define("HPA_FUSED_MIN_TILES")
FUSED_TAIL_DEN = _header_define("HPA_FUSED_TAIL_DEN")
FUSED_TAIL_CHUNK = _header_define("HPA_FUSED_TAIL_CHUNK")


class HpaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class PlanLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "header", "C", "worker_off", "item_s", "item_t0", "item_t1", "item_split", "item_slot",
        "num_splits", "partial_base", "merge_list", "total_bytes")] + [("max_items", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # One HIP runtime per process: torch brings its own libamdhip64 (same soname as
        # the one libhpa links), so load torch first and libhpa binds to that copy.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise HpaError(-1, "load", f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(AttnDesc)
        sig = {
            "hpa_default_num_workers": [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)],
            "hpa_plan_workspace_size": [D, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hpa_plan_workspace_layout": [D, _I, ctypes.POINTER(PlanLayout)],
            "hpa_partial_workspace_size": [D, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hpa_plan": [D, _P, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P],
            "hpa_decode_attn": [D, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I, _P, ctypes.c_size_t,
                                _P, ctypes.c_size_t, _P, _I, _P],
            "hpa_kv_pack_pages": [D, _P, _P, _P, _I, _P, _P, _P, _P],
            "hpa_moe_workspace_size": [_I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hpa_moe_pack_weights": [_P, _I, _I, _I, _P, _P],
            "hpa_moe_fused": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, ctypes.c_size_t, _P, _P],
            "hpa_decode_attn_noalloc": [D, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P],
            "hpa_decode_prologue": [D, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_double, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _P],
            "hpa_decode_prologue_plan": [D, _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_double, _P, _P,
                                         _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P],
            "hpa_read_device_error": [_P, ctypes.POINTER(ctypes.c_int32), _I, _P],
            "hpa_probe_stream_read": [_P, ctypes.c_size_t, _I, _P, _P],
            "hpa_router_pack_weights": [_P, _I, _I, _P, _P],
            "hpa_router_workspace_size": [_I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
            "hpa_router_gemm": [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, ctypes.c_size_t, _P],
            "hpa_status_string": [ctypes.c_int],
            "hpa_last_error_message": [],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("hpa_status_string", "hpa_last_error_message") else ctypes.c_int
        _lib = L
    return _lib


def declared_symbols() -> list:
    """Names of the functions include/hpa.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hpa_status|const char\*)\s+(hpa_\w+)\s*\(", text, re.M)))


def _check(status: int, where: str):
    if status != 0:
        raise HpaError(status, where, lib().hpa_last_error_message().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(batch, num_q_heads, num_kv_heads, max_pages_per_seq, num_pages, kv_dtype="bf16",
              sm_scale=None) -> AttnDesc:
    import math
    return AttnDesc(batch, num_q_heads, num_kv_heads, 128, 64, max_pages_per_seq, num_pages,
                    HPA_KV_FP8_E4M3 if kv_dtype == "fp8" else HPA_KV_BF16,
                    1.0 / math.sqrt(128) if sm_scale is None else sm_scale)


def hpa_default_num_workers(device: int = 0, sched: str = "balanced") -> int:
    n = ctypes.c_int32(0)
    _check(lib().hpa_default_num_workers(device, SCHED[sched], ctypes.byref(n)), "hpa_default_num_workers")
    return n.value


def hpa_plan_workspace_size(desc: AttnDesc, num_workers: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hpa_plan_workspace_size(ctypes.byref(desc), num_workers, ctypes.byref(n)), "hpa_plan_workspace_size")
    return n.value


def hpa_plan_workspace_layout(desc: AttnDesc, num_workers: int = 0) -> dict:
    lay = PlanLayout()
    _check(lib().hpa_plan_workspace_layout(ctypes.byref(desc), num_workers, ctypes.byref(lay)),
           "hpa_plan_workspace_layout")
    return {name: getattr(lay, name) for name, _ in PlanLayout._fields_}


def hpa_partial_workspace_size(desc: AttnDesc, num_workers: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hpa_partial_workspace_size(ctypes.byref(desc), num_workers, ctypes.byref(n)),
           "hpa_partial_workspace_size")
    return n.value


def hpa_plan(desc, seq_lens, num_workers, min_tiles_per_worker, item_cost, tail_den, tail_chunk, plan_ws,
             stream=None, item_order=0):
    _check(lib().hpa_plan(ctypes.byref(desc), _ptr(seq_lens), num_workers, min_tiles_per_worker, item_cost,
                          tail_den, tail_chunk, item_order, _ptr(plan_ws), plan_ws.numel() * plan_ws.element_size(),
                          _stream(stream)), "hpa_plan")


def hpa_decode_attn(desc, sched, q, k_cache, v_cache, k_scale, v_scale, seq_lens, page_table,
                    num_workers, plan_ws, partial_ws, out, flags=0, stream=None):
    sched = SCHED[sched] if isinstance(sched, str) else int(sched)
    pbytes = 0 if plan_ws is None else plan_ws.numel() * plan_ws.element_size()
    _check(lib().hpa_decode_attn(ctypes.byref(desc), sched, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens), _ptr(page_table),
                                 num_workers, _ptr(plan_ws), pbytes, _ptr(partial_ws),
                                 partial_ws.numel() * partial_ws.element_size(), _ptr(out), flags,
                                 _stream(stream)), "hpa_decode_attn")


def hpa_kv_pack_pages(desc, k_rows, v_rows, pages, k_cache, v_cache, device_error=None, stream=None):
    """Row-major [count, Hkv, 64, 128] pages -> tiled blocks pages[i] of the caches (pages None:
    the whole pool, page i -> block i; may then be the caches themselves)."""
    count = desc.num_pages if pages is None else pages.numel()
    _check(lib().hpa_kv_pack_pages(ctypes.byref(desc), _ptr(k_rows), _ptr(v_rows), _ptr(pages), count,
                                   _ptr(k_cache), _ptr(v_cache), _ptr(device_error), _stream(stream)),
           "hpa_kv_pack_pages")


def hpa_decode_attn_noalloc(desc, sched, q, k_cache, v_cache, k_scale, v_scale, seq_lens, page_table,
                            num_workers, out, device_error=None, stream=None):
    sched = SCHED[sched] if isinstance(sched, str) else int(sched)
    _check(lib().hpa_decode_attn_noalloc(ctypes.byref(desc), sched, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens), _ptr(page_table),
                                         num_workers, _ptr(out), _ptr(device_error), _stream(stream)),
           "hpa_decode_attn_noalloc")


def hpa_decode_prologue(desc, q_in, k_in, v_in, q_norm_w, k_norm_w, eps, rope_theta, positions,
                        page_table, k_cache, v_cache, k_scale, v_scale, q_out, seq_lens_out,
                        plan_ws=None, stream=None):
    _check(lib().hpa_decode_prologue(ctypes.byref(desc), _ptr(q_in), _ptr(k_in), _ptr(v_in),
                                     _ptr(q_norm_w), _ptr(k_norm_w), eps, rope_theta, _ptr(positions),
                                     _ptr(page_table), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(q_out), _ptr(seq_lens_out), _ptr(plan_ws),
                                     _stream(stream)), "hpa_decode_prologue")


def hpa_decode_prologue_plan(desc, q_in, k_in, v_in, q_norm_w, k_norm_w, eps, rope_theta, positions,
                             page_table, k_cache, v_cache, k_scale, v_scale, q_out, seq_lens_out, num_workers,
                             min_tiles_per_worker, item_cost, tail_den, tail_chunk, plan_ws, stream=None,
                             item_order=0):
    _check(lib().hpa_decode_prologue_plan(ctypes.byref(desc), _ptr(q_in), _ptr(k_in), _ptr(v_in),
                                          _ptr(q_norm_w), _ptr(k_norm_w), eps, rope_theta, _ptr(positions),
                                          _ptr(page_table), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                          _ptr(v_scale), _ptr(q_out), _ptr(seq_lens_out), num_workers,
                                          min_tiles_per_worker, item_cost, tail_den, tail_chunk, item_order,
                                          _ptr(plan_ws),
                                          plan_ws.numel() * plan_ws.element_size(), _stream(stream)),
           "hpa_decode_prologue_plan")


def hpa_read_device_error(plan_ws, clear: bool = False, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().hpa_read_device_error(_ptr(plan_ws), ctypes.byref(code), 1 if clear else 0, _stream(stream)),
           "hpa_read_device_error")
    return code.value


def hpa_probe_stream_read(buf, workgroups: int = 0, sink=None, stream=None) -> None:
    """Read all of `buf` (a device tensor) once with the library's plain-read probe."""
    import torch
    if sink is None:
        sink = torch.zeros(max(workgroups, 4096), dtype=torch.int32, device=buf.device)
    _check(lib().hpa_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), workgroups, _ptr(sink),
                                       _stream(stream)), "hpa_probe_stream_read")


def hpa_router_pack_weights(w, packed, stream=None) -> None:
    """w: fp32 [E, H] device tensor -> packed (uint8 device tensor of E * H * 4 bytes)."""
    E, H = w.shape
    _check(lib().hpa_router_pack_weights(_ptr(w), E, H, _ptr(packed), _stream(stream)), "hpa_router_pack_weights")


def hpa_router_workspace_size(tokens: int, experts: int, hidden: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hpa_router_workspace_size(tokens, experts, hidden, ctypes.byref(n)), "hpa_router_workspace_size")
    return n.value


def hpa_router_gemm(x, packed, experts: int, passes: int, logits, top_k: int, topk_idx, topk_val, workspace,
                    stream=None) -> None:
    """x: bf16 [T, H] device tensor; logits fp32 [T, E]; topk_idx int32 / topk_val fp32 [T, top_k]."""
    T, H = x.shape
    _check(lib().hpa_router_gemm(_ptr(x), _ptr(packed), T, experts, H, passes, _ptr(logits), top_k,
                                 _ptr(topk_idx) if top_k else None, _ptr(topk_val) if top_k else None,
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "hpa_router_gemm")


def hpa_moe_pack_weights(w, packed, stream=None) -> None:
    """w: uint8 E4M3 codes [E, rows, cols] (row-major) -> packed (uint8, same size)."""
    E, rows, cols = w.shape
    _check(lib().hpa_moe_pack_weights(_ptr(w), E, rows, cols, _ptr(packed), _stream(stream)), "hpa_moe_pack_weights")


def hpa_moe_workspace_size(tokens: int, top_k: int, hidden: int, inter: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hpa_moe_workspace_size(tokens, top_k, hidden, inter, ctypes.byref(n)), "hpa_moe_workspace_size")
    return n.value


def hpa_moe_fused(x, topk_ids, topk_weights, w1, s1, w2, s2, experts: int, inter: int, out, workspace,
                  device_error=None, stream=None) -> None:
    """x bf16 [T, H]; ids int32 / weights fp32 [T, K]; w1 uint8 [E, 2I, H], s1 fp32 [E, 2I];
    w2 uint8 [E, H, I], s2 fp32 [E, H]; out bf16 [T, H]."""
    T, H = x.shape
    K = topk_ids.shape[1]
    _check(lib().hpa_moe_fused(_ptr(x), _ptr(topk_ids), _ptr(topk_weights), _ptr(w1), _ptr(s1), _ptr(w2), _ptr(s2),
                               T, experts, K, H, inter, _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(device_error), _stream(stream)),
           "hpa_moe_fused")


def hpa_status_string(status: int) -> str:
    return lib().hpa_status_string(status).decode()


def hpa_last_error_message() -> str:
    return lib().hpa_last_error_message().decode()

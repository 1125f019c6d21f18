"""Device-side plumbing around the C ABI: upload a workload, own its workspaces,
run one decode step (prologue -> plan -> attention -> merge) on the GPU.

PyTorch is used only to hold device memory and to name the stream.
"""

from __future__ import annotations

import numpy as np

from . import _lib


class DeviceStep:
    """One workload resident in HBM plus the workspaces its decode step needs."""

    def __init__(self, w, num_workers: int = 0, device: str = "cuda"):
        import torch
        self.torch = torch
        self.w = w
        dev = torch.device(device)
        self.device = dev

        def up(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.view(dtype)
            return t.to(dev)

        self.q = up(w.q.view(np.int16), torch.bfloat16)
        self.k_cache = up(w.k_cache.view(np.int16) if w.kv_dtype == "bf16" else w.k_cache)
        self.v_cache = up(w.v_cache.view(np.int16) if w.kv_dtype == "bf16" else w.v_cache)
        self.k_scale = up(w.k_scale) if w.k_scale is not None else None
        self.v_scale = up(w.v_scale) if w.v_scale is not None else None
        self.seq_lens = up(w.seq_lens)
        self.page_table = up(w.page_table)
        self.desc = _lib.make_desc(w.batch, w.hq, w.hkv, w.max_pages, w.num_pages, w.kv_dtype, w.sm_scale)
        # an explicit worker count serves every schedule; otherwise each schedule takes
        # its own default (persistent grid, or the W static split-KV sizes its splits by)
        di = dev.index or 0
        self.num_workers = num_workers or _lib.hpa_default_num_workers(di, "balanced")
        self.static_workers = num_workers or _lib.hpa_default_num_workers(di, "static_splits")
        ws_workers = max(self.num_workers, self.static_workers)
        self.plan_ws = torch.zeros(_lib.hpa_plan_workspace_size(self.desc, ws_workers),
                                   dtype=torch.uint8, device=dev)
        self.partial_ws = torch.empty(_lib.hpa_partial_workspace_size(self.desc, ws_workers),
                                      dtype=torch.uint8, device=dev)
        self.last_workers = self.num_workers
        self.out = torch.empty((w.batch, w.hq, 128), dtype=torch.bfloat16, device=dev)
        if w.has_prologue:
            self.q_new = up(w.q_new.view(np.int16), torch.bfloat16)
            self.k_new = up(w.k_new.view(np.int16), torch.bfloat16)
            self.v_new = up(w.v_new.view(np.int16), torch.bfloat16)
            self.q_norm_w = up(w.q_norm_w)
            self.k_norm_w = up(w.k_norm_w)
            self.q_rot = torch.empty_like(self.q_new)
            self.lens_after = torch.empty_like(self.seq_lens)

    def prologue(self, stream=None):
        w = self.w
        _lib.hpa_decode_prologue(self.desc, self.q_new, self.k_new, self.v_new, self.q_norm_w, self.k_norm_w,
                                 w.eps, w.rope_theta, self.seq_lens, self.page_table, self.k_cache,
                                 self.v_cache, self.k_scale, self.v_scale, self.q_rot, self.lens_after,
                                 self.plan_ws, stream)

    def prologue_plan(self, min_tiles: int = _lib.FUSED_MIN_TILES, item_cost: int = _lib.FUSED_ITEM_COST,
                      tail_den: int = _lib.FUSED_TAIL_DEN, tail_chunk: int = _lib.FUSED_TAIL_CHUNK, stream=None,
                      item_order: int = 0):
        """The prologue and the planner in one launch (the plan hpa_plan would make over
        the lengths after the append)."""
        w = self.w
        _lib.hpa_decode_prologue_plan(self.desc, self.q_new, self.k_new, self.v_new, self.q_norm_w,
                                      self.k_norm_w, w.eps, w.rope_theta, self.seq_lens, self.page_table,
                                      self.k_cache, self.v_cache, self.k_scale, self.v_scale, self.q_rot,
                                      self.lens_after, self.num_workers, min_tiles, item_cost, tail_den,
                                      tail_chunk, self.plan_ws, stream, item_order)

    def attn_inputs(self):
        if self.w.has_prologue:
            return self.q_rot, self.lens_after
        return self.q, self.seq_lens

    def plan(self, min_tiles: int = _lib.FUSED_MIN_TILES, item_cost: int = _lib.FUSED_ITEM_COST,
             tail_den: int = _lib.FUSED_TAIL_DEN, tail_chunk: int = _lib.FUSED_TAIL_CHUNK, stream=None,
             item_order: int = 0):
        _, lens = self.attn_inputs()
        _lib.hpa_plan(self.desc, lens, self.num_workers, min_tiles, item_cost, tail_den, tail_chunk,
                      self.plan_ws, stream, item_order)

    def attend(self, sched: str = "balanced", stream=None, flags: int = 0):
        """sched: a schedule name of _lib.SCHED, or "balanced_inmerge" (the planned
        schedule with HPA_ATTN_MERGE_IN_KERNEL: one launch over the plan)."""
        q, lens = self.attn_inputs()
        W = self.static_workers if sched.startswith("static") else self.num_workers
        self.last_workers = W
        if sched == "balanced_inmerge":
            sched, flags = "balanced", flags | _lib.ATTN_MERGE_IN_KERNEL
        _lib.hpa_decode_attn(self.desc, sched, q, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                             lens, self.page_table, W, self.plan_ws, self.partial_ws,
                             self.out, flags, stream)

    def step(self, sched: str = "balanced", min_tiles: int = _lib.FUSED_MIN_TILES,
             item_cost: int = _lib.FUSED_ITEM_COST, tail_den: int = _lib.FUSED_TAIL_DEN,
             tail_chunk: int = _lib.FUSED_TAIL_CHUNK, stream=None, prologue_plans: bool = True,
             item_order: int = 0):
        """The whole hot path of one decode step; returns the bf16 output tensor. With a
        prologue, the planned schedules plan inside the prologue launch unless
        prologue_plans is False (then: prologue launch, planner launch)."""
        planned = sched in ("balanced", "balanced_inmerge")
        if self.w.has_prologue and planned and prologue_plans:
            self.prologue_plan(min_tiles, item_cost, tail_den, tail_chunk, stream, item_order)
        else:
            if self.w.has_prologue:
                self.prologue(stream)
            if planned:
                self.plan(min_tiles, item_cost, tail_den, tail_chunk, stream, item_order)
        self.attend(sched, stream)
        return self.out

    def device_error(self, clear: bool = False) -> int:
        return _lib.hpa_read_device_error(self.plan_ws, clear)

    def plan_arrays(self) -> dict:
        """The plan workspace as host int32 arrays (after the stream is synchronised)."""
        lay = _lib.hpa_plan_workspace_layout(self.desc, self.num_workers)
        ws = self.plan_ws.cpu().numpy().view(np.int32)
        hdr = ws[lay["header"] // 4: lay["header"] // 4 + 16]
        Wp, N, S, nit, nm, npart = (int(x) for x in hdr[:6])
        D, Ws = int(hdr[8]), int(hdr[9])
        g = lambda key, n: ws[lay[key] // 4: lay[key] // 4 + n].tolist()
        return dict(Wp=Wp, Ws=Ws, D=D, V=Ws + D, N=N, S=S, n_items=nit, n_partials=npart, error=int(hdr[6]),
                    W=int(hdr[7]), C=g("C", S + 1), worker_off=g("worker_off", Ws + D + 1), item_s=g("item_s", nit),
                    item_t0=g("item_t0", nit), item_t1=g("item_t1", nit), item_split=g("item_split", nit),
                    item_slot=g("item_slot", nit), num_splits=g("num_splits", S),
                    partial_base=g("partial_base", S), merge_list=g("merge_list", nm))

    def trace_records(self) -> np.ndarray:
        """Instrumented build only: per-wave records [blocks, waves, 68] of the last
        attention launch (start, end on the 100 MHz counter; HW_ID | XCC_ID << 32; units;
        4 start-up times; per item: first unit issued, last unit computed, combine done;
        then the completion times of the first 48 units)."""
        if not _lib.TRACE:
            raise RuntimeError("trace records need the instrumented build (HPA_TRACE=1)")
        w = self.w
        S = w.batch * w.hkv
        W = self.last_workers
        base = (5 * W + S) * (w.hq // w.hkv) * (128 + 2) * 4     # after the partial slots
        raw = self.partial_ws[base:].cpu().numpy()
        n = (W + S) * _lib.TRACE_WAVES * _lib.TRACE_WORDS
        return raw[: n * 8].view(np.uint64).reshape(W + S, _lib.TRACE_WAVES, _lib.TRACE_WORDS)

    def output_f64(self) -> np.ndarray:
        return self.out.float().cpu().numpy().astype(np.float64)


class RouterStep:
    """A router workload (inputs.RouterWorkload) resident in HBM: activations, the
    fp32 weight, its packed split form, logits, top-k outputs and the workspace."""

    def __init__(self, rw, top_k: int = 8, device: str = "cuda"):
        import torch
        self.torch = torch
        self.rw = rw
        self.top_k = top_k
        dev = torch.device(device)
        T, E, H = rw.tokens, rw.experts, rw.hidden
        self.x = torch.from_numpy(np.ascontiguousarray(rw.x).view(np.int16)).view(torch.bfloat16).to(dev)
        self.w = torch.from_numpy(np.ascontiguousarray(rw.w, np.float32)).to(dev)
        self.packed = torch.empty(E * H * 4, dtype=torch.uint8, device=dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((T, max(top_k, 1)), dtype=torch.int32, device=dev)
        self.topk_val = torch.empty((T, max(top_k, 1)), dtype=torch.float32, device=dev)
        ws = _lib.hpa_router_workspace_size(T, E, H)
        self.workspace = torch.empty(max(ws, 16) // 4, dtype=torch.float32, device=dev)
        self.pack()

    def pack(self):
        _lib.hpa_router_pack_weights(self.w, self.packed)

    def run(self, passes: int = 2, packed=None):
        _lib.hpa_router_gemm(self.x, self.packed if packed is None else packed, self.rw.experts, passes,
                             self.logits, self.top_k, self.topk_idx[:, :self.top_k] if self.top_k else None,
                             self.topk_val[:, :self.top_k] if self.top_k else None, self.workspace)

    def results(self):
        """(logits fp64 [T, E], top-k indices int64 [T, k], top-k values fp64 [T, k])."""
        self.torch.cuda.synchronize()
        k = self.top_k
        return (self.logits.cpu().numpy().astype(np.float64),
                self.topk_idx[:, :k].cpu().numpy().astype(np.int64),
                self.topk_val[:, :k].cpu().numpy().astype(np.float64))


class MoeStep:
    """An MoE workload (inputs.MoeWorkload) resident in HBM: hidden states, routing,
    E4M3 expert weights with their scales, the output and the workspace."""

    def __init__(self, mw, device: str = "cuda"):
        import torch
        self.torch = torch
        self.mw = mw
        dev = torch.device(device)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.x = up(mw.x.view(np.int16)).view(torch.bfloat16)
        self.ids = up(mw.ids)
        self.weights = up(mw.weights)
        # the E4M3 weights row-major as drawn, then packed once into the tiled order
        self.w1_rows, self.s1 = up(mw.w1), up(mw.s1)
        self.w2_rows, self.s2 = up(mw.w2), up(mw.s2)
        self.w1 = torch.empty_like(self.w1_rows)
        self.w2 = torch.empty_like(self.w2_rows)
        _lib.hpa_moe_pack_weights(self.w1_rows, self.w1)
        _lib.hpa_moe_pack_weights(self.w2_rows, self.w2)
        self.out = torch.empty((mw.tokens, mw.hidden), dtype=torch.bfloat16, device=dev)
        ws = _lib.hpa_moe_workspace_size(mw.tokens, mw.top_k, mw.hidden, mw.inter)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(self, stream=None):
        mw = self.mw
        _lib.hpa_moe_fused(self.x, self.ids, self.weights, self.w1, self.s1, self.w2, self.s2, mw.experts, mw.inter,
                           self.out, self.workspace, self.err, stream)
        return self.out

    def output_f64(self) -> np.ndarray:
        return self.out.float().cpu().numpy().astype(np.float64)

    def activations(self) -> np.ndarray:
        """The fp32 SwiGLU outputs [T, K, I] the last call left in the workspace (after
        the token codes and scales and the routing index, each array 256-byte aligned)."""
        mw = self.mw
        al = lambda x: (x + 255) // 256 * 256
        T, K, H, I = mw.tokens, mw.top_k, mw.hidden, mw.inter
        P = T * K
        off = al(T * H) + al(T * 4) + al(P * 4) + al(3 * P * 4) + al(4)
        raw = self.workspace.cpu().numpy()
        return raw[off: off + P * I * 4].view(np.float32).reshape(T, K, I)

    def routing(self):
        """The routing index the routing pass left in the workspace (calls of more than 16
        pairs): the pair list [P], the pair-block table (expert, first list index, count)
        as three arrays of the block count's length."""
        mw = self.mw
        al = lambda x: (x + 255) // 256 * 256
        T, K, H = mw.tokens, mw.top_k, mw.hidden
        P = T * K
        raw = self.workspace.cpu().numpy()
        o = al(T * H) + al(T * 4)
        lst = raw[o: o + P * 4].view(np.int32).copy()
        o += al(P * 4)
        blk = raw[o: o + 3 * P * 4].view(np.int32).reshape(3, P)
        o += al(3 * P * 4)
        n = int(raw[o: o + 4].view(np.int32)[0])
        return lst, blk[0, :n].copy(), blk[1, :n].copy(), blk[2, :n].copy()

    def token_codes(self):
        """The tokens' E4M3 codes [T, H] and fp32 scales [T] at the start of the workspace
        (written by the routing pass; calls of at most 16 pairs quantise inside Gate-Up and
        leave them unwritten)."""
        mw = self.mw
        al = lambda x: (x + 255) // 256 * 256
        T, H = mw.tokens, mw.hidden
        raw = self.workspace.cpu().numpy()
        return raw[:T * H].reshape(T, H).copy(), raw[al(T * H): al(T * H) + T * 4].view(np.float32).copy()

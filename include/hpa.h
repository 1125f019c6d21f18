/*
 * hpa.h -- C ABI of libhpa: load-balanced split-KV decode attention over a
 * paged KV cache, for MI355X (gfx950).
 *
 * The method (xiaodao.ai, "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
 * "为什么 batch 越大，数字越漂亮"; bitbyai.com, "vLLM × HPC-Ops: High-Performance
 * Attention and MoE Backends from Tencent Hunyuan", section "Breaking Down the
 * Kernels"): each decode step, cut every request's live KV into 64-token
 * tiles, spread the global tile list evenly over persistent workers, let each
 * worker produce softmax partials (acc, m, l) for the ranges it owns and merge
 * split sequences with a log-sum-exp combine. A static split-KV schedule is
 * provided for comparison, and a fused prologue (q/k RMSNorm, RoPE, paged KV
 * append) that runs ahead of attention.
 *
 * Conventions for every call:
 *  - Tensors are caller-owned device memory; the library allocates nothing.
 *    Workspace sizes come from the *_workspace_size queries.
 *  - Calls are asynchronous on the given stream and never synchronise, except
 *    hpa_read_device_error and hpa_default_num_workers (device query, cached).
 *  - Host-side validation failures return a non-OK status and launch nothing.
 *  - Device-side data errors (a length < 0 or beyond the page table, a page id
 *    outside [0, num_pages)) OR a bit into the sticky error word held in the
 *    plan workspace; the offending work is skipped (its output is undefined).
 *  - No C++ exception crosses this boundary. All entry points are thread-safe.
 *
 * Layouts (row-major, innermost last):
 *  q, q_out        [B, Hq, 128]                    bf16
 *  out             [B, Hq, 128]                    bf16
 *  k_cache         [num_pages, Hkv, 8192]          bf16 or OCP E4M3 codes, tiled page blocks
 *  v_cache         [num_pages, Hkv, 8192]          bf16 or OCP E4M3 codes, tiled page blocks
 *                  (the row-major page [num_pages, Hkv, 64, 128] in another element
 *                  order; hpa_kv_pack_pages converts row-major pages to it)
 *  k_scale,v_scale [Hkv]                           fp32 (E4M3 caches only; value = code * scale)
 *  seq_lens        [B]                             int32, live KV length per request
 *  page_table      [B, max_pages_per_seq]          int32 physical page of each 64-token tile
 * Query head h reads KV head h / (Hq / Hkv). Sequence s = b * Hkv + g.
 *
 * Tiled page blocks: block (p, g) holds the 64 tokens x 128 dims of page p for
 * KV head g, element (token t, dim d) at index
 *   bf16 K:  t%32 = 8a + 4b + q, d = 32c + 8j + e:  4096 (t/32) + 512 (4b + c) + 8 (16j + 4a + q) + e
 *   bf16 V:  t%32 = 8j + e,      d = 16n + m:       4096 (t/32) + 512 n + 8 (16j + m) + e
 *   E4M3 K:  t = 16a + 4b + q,   d = 64p + 16j + e: 1024 (2b + p) + 16 (16j + 4a + q) + e
 *   E4M3 V:  t = 16j + e,        d = 16n + m:       1024 n + 16 (16j + m) + e
 * (all digits non-negative and below their radix). Every 1 KB of a block is what
 * one wave of the attention kernel loads in one 16-byte-per-lane instruction and
 * feeds to a 16x16x32 matrix-core product, so K and V stream as whole cache lines.
 * hpa_decode_prologue writes new tokens in this order.
 */
#ifndef HPA_H
#define HPA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HPA_OK = 0,
  HPA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, Hq % Hkv != 0, ... */
  HPA_ERR_UNSUPPORTED = 2,  /* head_dim != 128, page_size != 64, Hq/Hkv > 16 */
  HPA_ERR_WORKSPACE = 3,    /* workspace smaller than the size query returns */
  HPA_ERR_DEVICE = 4,       /* a HIP runtime call failed */
  HPA_ERR_LAUNCH = 5        /* a kernel launch failed */
} hpa_status;

typedef enum { HPA_KV_BF16 = 0, HPA_KV_FP8_E4M3 = 1 } hpa_kv_dtype;

typedef enum {
  HPA_SCHED_BALANCED = 0,      /* work list from hpa_plan (persistent workers) */
  HPA_SCHED_STATIC_SPLITS = 1, /* fixed number of splits per sequence          */
  HPA_SCHED_STATIC_CHUNK = 2,  /* fixed split size, grid sized for the longest */
  HPA_SCHED_BALANCED_FUSED = 3, /* the same balanced work list, computed inside the
                                   persistent kernel from seq_lens (no hpa_plan call,
                                   one launch less); above 2048 sequences (B x Hkv)
                                   the planner kernel runs first, into plan_ws */
  HPA_SCHED_BALANCED_SINGLE = 4 /* as FUSED, and split sequences are merged inside the
                                   same kernel by the workgroup that completes them
                                   (one launch per step); refused (HPA_ERR_UNSUPPORTED)
                                   when the partial workspace reaches 4 GiB */
} hpa_sched;

/* Sticky device error bits (hpa_read_device_error). */
enum {
  HPA_DEVERR_SEQ_LEN = 1,      /* seq_len < 0 or > max_pages_per_seq * 64 */
  HPA_DEVERR_PAGE_ID = 2,      /* page id outside [0, num_pages) */
  HPA_DEVERR_PROLOGUE = 4,     /* append position outside the page table */
  HPA_DEVERR_PLAN = 8,         /* attention launched with another worker count, batch or KV-head
                                  count than the plan was made for, or a plan workspace that is
                                  not a plan (nothing of that plan is read) */
  HPA_DEVERR_MOE_EXPERT = 16   /* an MoE routing id outside [0, experts) (that slot adds nothing) */
};

typedef struct {
  int32_t batch;               /* B  >= 0 */
  int32_t num_q_heads;         /* Hq >= 1 */
  int32_t num_kv_heads;        /* Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= 16 */
  int32_t head_dim;            /* must be 128 */
  int32_t page_size;           /* must be 64 (one page = one tile) */
  int32_t max_pages_per_seq;   /* page_table row length, >= 1 */
  int32_t num_pages;           /* physical pages in each cache pool */
  hpa_kv_dtype kv_dtype;
  float sm_scale;              /* softmax scale, e.g. 1/sqrt(128) */
} hpa_attn_desc;

/* Byte offsets of the arrays inside a plan workspace (for inspection and tests).
 * All arrays are int32. header[0..15]: 0 W' (active workers), 1 N (tiles),
 * 2 S (sequences), 3 n_items, 4 n_merge, 5 n_partials, 6 sticky error word,
 * 7 W (workers the plan was made for), 8 D (tail chunks), 9 Ws (workers with a
 * static range), 10 B and 11 Hkv (the batch and KV-head count it was made
 * for). worker_off has Ws + D + 1 entries: the items of static worker v < Ws,
 * then those of tail chunk c (virtual worker Ws + c). */
typedef struct {
  size_t header, C, worker_off, item_s, item_t0, item_t1, item_split, item_slot,
         num_splits, partial_base, merge_list, total_bytes;
  int32_t max_items;           /* 5 W + S: at most 4 W tail chunks */
} hpa_plan_layout;

/* Row-major pages -> tiled page blocks (openai-hub.com "腾讯混元HPC-Ops升级：五大算子
 * 直击推理痛点", section "五大算子覆盖了哪些场景": the attention call reads a paged
 * KV cache; the pages fix no in-page order). k_rows, v_rows: device,
 * [count, Hkv, 64, 128] row-major pages (token-major, dims innermost) of bf16
 * values or OCP E4M3 codes (desc->kv_dtype), 16-byte aligned. For i < count,
 * block (pages[i], g) of k_cache / v_cache ([num_pages, Hkv, 8192], the tiled
 * order above) receives page i of head g, element by element (no arithmetic:
 * the bytes move). pages: device int32 [count], or NULL for the whole pool
 * (count == num_pages, page i -> block i); with NULL the source may be the
 * cache itself (conversion in place: every block is read whole before it is
 * written). A page id outside [0, num_pages) is skipped and sets
 * HPA_DEVERR_PAGE_ID in device_error (device int32, may be NULL). Only
 * desc->num_kv_heads, num_pages, head_dim, page_size and kv_dtype are read.
 * One launch on `stream`; nothing allocated. */
hpa_status hpa_kv_pack_pages(const hpa_attn_desc* desc, const void* k_rows, const void* v_rows,
                             const int32_t* pages, int32_t count, void* k_cache, void* v_cache,
                             int32_t* device_error, hipStream_t stream);

/* Default worker count of a schedule on a device: compute units x workgroups of
 * that schedule's attention kernel that fit on one CU at once (cached per device).
 * For the balanced schedules it is the persistent grid; for the static ones, the
 * W their split count is derived from. num_workers = 0 in the calls below means
 * this default for the schedule concerned (for the workspace size queries: the
 * largest default over all schedules). */
hpa_status hpa_default_num_workers(int device, hpa_sched sched, int32_t* num_workers);

/* Size and layout of the plan workspace for up to num_workers workers (0 = default). */
hpa_status hpa_plan_workspace_size(const hpa_attn_desc* desc, int32_t num_workers, size_t* bytes);
hpa_status hpa_plan_workspace_layout(const hpa_attn_desc* desc, int32_t num_workers,
                                     hpa_plan_layout* layout);

/* Size of the partial-result workspace: (5 W + S) slots of Hq/Hkv x 128 fp32
 * accumulators plus a max and a sum per head. Enough for every schedule. */
hpa_status hpa_partial_workspace_size(const hpa_attn_desc* desc, int32_t num_workers, size_t* bytes);

/* Balanced planner (one workgroup; xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必
 * 快一半", section "为什么 batch 越大，数字越漂亮"): tile counts n_s = ceil(L/64)
 * per sequence and their prefix sum C. Starting an item is charged item_cost
 * tiles (bitbyai.com "vLLM × HPC-Ops …", "Breaking Down the Kernels": the
 * scheduler weighs work by progress): every non-empty sequence s occupies
 * positions [P[s], P[s+1]) of the global list, P[s] = C[s] + item_cost * (non-empty
 * sequences before s), its real tiles last. With N' = P[S] positions, W' =
 * min(W, max(1, N' / min_tiles_per_worker)) workers (0 when there is no tile);
 * worker w owns positions [w*N'/W', (w+1)*N'/W') and its items are the real
 * tiles among them, cut at sequence boundaries (a worker may get none); then
 * split ranks, partial slots and the list of sequences to merge. item_cost 0 is
 * the plain even split of the tiles. 0 <= item_cost <= 64.
 * Dynamic tail (same section: the scheduler evaluates progress as it runs;
 * tail_den > 0): the last T = N' / tail_den positions are not assigned ahead of
 * time but cut into D = min(ceil(T / tail_chunk), 4 W) chunks that the persistent
 * workers claim on a device counter whenever they run out of work; the first
 * A = N' - T positions are split as above over Ws = min(W', A) workers. Items,
 * split ranks and slots follow the virtual workers (Ws static ranges, then the
 * chunks) in order, so results do not depend on who claims which chunk.
 * tail_den = 0: no tail (Ws = W', D = 0). tail_den >= 0, tail_chunk >= 1.
 * Item order (same section: the scheduler prioritizes nearly-finished short
 * requests): item_order 0 lists each worker's items in list order; 1 lists the
 * sequences a worker holds whole (the short requests it finishes alone) first,
 * then its pieces of split sequences; 2 the pieces first, then the whole ones
 * (their partial results are complete sooner). Each class stays in list order;
 * split ranks, partial slots and so the output bits are the same in every order.
 * The planner also returns the claim counters to zero.
 * seq_lens stays on the device (no host synchronisation). The plan workspace
 * must be zero-filled before its first use (it holds the sticky error word,
 * which hpa_plan never clears). */
hpa_status hpa_plan(const hpa_attn_desc* desc, const int32_t* seq_lens, int32_t num_workers,
                    int32_t min_tiles_per_worker, int32_t item_cost, int32_t tail_den,
                    int32_t tail_chunk, int32_t item_order, void* plan_ws, size_t plan_ws_bytes,
                    hipStream_t stream);

/* The item cost, minimum tiles per worker and dynamic tail the fused schedules
 * plan with; an hpa_plan call with these values (and item_order 0) gives their
 * items exactly. */
#define HPA_FUSED_ITEM_COST 4
#define HPA_FUSED_MIN_TILES 2
#define HPA_FUSED_TAIL_DEN 0
#define HPA_FUSED_TAIL_CHUNK 1

/* Flags of hpa_decode_attn. The default (0) runs both launches. */
enum {
  HPA_ATTN_NO_MERGE = 1,    /* launch only the attention kernel (partials + unsplit rows) */
  HPA_ATTN_MERGE_ONLY = 2,  /* launch only the merge of an earlier HPA_ATTN_NO_MERGE call */
  HPA_ATTN_MERGE_IN_KERNEL = 4  /* HPA_SCHED_BALANCED only: the planned kernel merges split
                                   sequences itself, as HPA_SCHED_BALANCED_SINGLE does (one
                                   launch); not with the two flags above */
};

/* Decode attention over the paged cache (openai-hub.com "腾讯混元HPC-Ops升级：五大算子
 * 直击推理痛点", section "五大算子覆盖了哪些场景": variable-length attention reading a
 * paged KV cache; xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
 * "为什么 batch 越大，数字越漂亮": the balanced split-KV schedule and the two static
 * ones it is compared with; bitbyai.com "vLLM × HPC-Ops …", section "Breaking
 * Down the Kernels": persistent, load-balanced decode attention):
 * out[b, h] = softmax(sm_scale * q K^T) V over the first
 * seq_lens[b] tokens of request b (a zero row when seq_lens[b] == 0).
 * Arguments: desc as above; q, k_cache, v_cache, seq_lens, page_table, out in the
 * layouts at the top of this file (device memory, caller-owned, never freed or
 * kept); num_workers 0 = the schedule's default; plan_ws / partial_ws: device
 * workspaces of at least the sizes the queries return. A plan whose header names
 * another worker count, batch or KV-head count than this call is refused on the
 * device (HPA_DEVERR_PLAN; no output row of the balanced schedule is written).
 * HPA_SCHED_BALANCED runs the persistent kernel over the plan made by hpa_plan
 * with the same num_workers, then the merge kernel. HPA_SCHED_BALANCED_FUSED
 * needs no hpa_plan call: the persistent kernel evaluates the planner's closed
 * forms itself (same items and slots as hpa_plan with HPA_FUSED_MIN_TILES and
 * HPA_FUSED_ITEM_COST) and records
 * each split sequence's split count and slot base in plan_ws for the merge
 * kernel. HPA_SCHED_BALANCED_SINGLE merges inside the persistent kernel: a
 * split's partial is written with device-coherent stores, then its workgroup
 * counts itself in on an atomic counter of its group of 16 consecutive splits;
 * the workgroup completing a group reduces it (and the one completing the last
 * group reduces the group results) in the merge kernel's order; no workgroup
 * waits on another, and the counters in plan_ws return to zero. All balanced
 * schedules produce identical bits. Their persistent workers claim the tail
 * chunks of the plan (hpa_plan's dynamic tail; HPA_FUSED_TAIL_DEN for the fused
 * schedules) on a counter in plan_ws that the last workgroup to finish returns
 * to zero, so calls sharing one plan_ws must not overlap. The static schedules
 * ignore the plan (plan_ws may still be given to receive device errors; NULL
 * otherwise) and size their grid from num_workers. k_scale/v_scale are
 * required for E4M3 caches and ignored for bf16. partial_ws must hold
 * hpa_partial_workspace_size bytes. Two kernel launches (attention, then merge;
 * one for HPA_SCHED_BALANCED_SINGLE, which ignores flags); flags may split them
 * into two calls with identical arguments, so a caller can time or overlap them
 * separately. */
hpa_status hpa_decode_attn(const hpa_attn_desc* desc, hpa_sched sched, const void* q,
                           const void* k_cache, const void* v_cache, const float* k_scale,
                           const float* v_scale, const int32_t* seq_lens,
                           const int32_t* page_table, int32_t num_workers, void* plan_ws,
                           size_t plan_ws_bytes, void* partial_ws, size_t partial_ws_bytes,
                           void* out, int32_t flags, hipStream_t stream);

/* Allocation-free hpa_decode_attn, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The plan and partial workspaces are taken from a device array of
 * 32 MiB that the library holds on every GPU it runs on until the process ends;
 * the call itself allocates nothing. Same arguments and results as
 * hpa_decode_attn without plan_ws / partial_ws / flags, for the schedules that
 * need no hpa_plan call: HPA_SCHED_BALANCED_FUSED, HPA_SCHED_BALANCED_SINGLE,
 * HPA_SCHED_STATIC_SPLITS, HPA_SCHED_STATIC_CHUNK (others: HPA_ERR_INVALID_ARG).
 * Limits: at most 4096 workers and 2048 sequences (batch x KV heads), and both
 * workspaces together within the array (e.g. 256 workers, 2048 sequences, 16
 * query heads per KV head fit); beyond them HPA_ERR_UNSUPPORTED, nothing
 * launched. device_error (device int32, may be NULL) receives the sticky
 * HPA_DEVERR_* bits instead of a plan workspace. The first call on a device looks
 * up the array's device address and clears its counters on `stream`. Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must not be issued. */
hpa_status hpa_decode_attn_noalloc(const hpa_attn_desc* desc, hpa_sched sched, const void* q,
                                   const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* seq_lens, const int32_t* page_table,
                                   int32_t num_workers, void* out, int32_t* device_error, hipStream_t stream);

/* Fused decode prologue (bitbyai.com "vLLM × HPC-Ops …", "Breaking Down the
 * Kernels"): for each request b at position pos = positions[b]:
 *   q_out[b,h] = RoPE(RMSNorm(q_in[b,h]; q_norm_w, eps), pos)     (bf16)
 *   k          = RoPE(RMSNorm(k_in[b,g]; k_norm_w, eps), pos)
 *   K row pos%64 of block (page_table[b, pos/64], g) = encode(k / k_scale[g])
 *   V row pos%64 of block (page_table[b, pos/64], g) = encode(v_in[b,g] / v_scale[g])
 *   seq_lens_out[b] = pos + 1
 * RMSNorm is over the 128 dims of a head row with one weight vector per
 * projection; RoPE rotates the pairs (i, i+64) by pos * rope_theta^(-i/64).
 * encode is round-to-nearest-even bf16, or saturating round-to-nearest-even
 * OCP E4M3 (scales required). positions and seq_lens_out must not alias.
 * plan_ws (may be NULL) receives HPA_DEVERR_PROLOGUE. One kernel launch. */
hpa_status hpa_decode_prologue(const hpa_attn_desc* desc, const void* q_in, const void* k_in,
                               const void* v_in, const float* q_norm_w, const float* k_norm_w,
                               float eps, double rope_theta, const int32_t* positions,
                               const int32_t* page_table, void* k_cache, void* v_cache,
                               const float* k_scale, const float* v_scale, void* q_out,
                               int32_t* seq_lens_out, void* plan_ws, hipStream_t stream);

/* Prologue and planner in one launch (bitbyai.com "vLLM × HPC-Ops …",
 * "Breaking Down the Kernels": the prologue is fused to save launches, and the
 * scheduler runs every step): everything hpa_decode_prologue does, plus the work
 * list hpa_plan would make over seq_lens_out with the same parameters -- bit for
 * bit, including for requests whose append fails (their length stays what
 * seq_lens_out held). One extra workgroup plans from positions + 1 while the
 * others append, so no launch waits for another; batches of more than 3072
 * sequences plan in a second launch after the appends. Then run
 * hpa_decode_attn(HPA_SCHED_BALANCED) with the same num_workers. Argument rules
 * are those of the two calls; plan_ws is required and receives
 * HPA_DEVERR_PROLOGUE and HPA_DEVERR_SEQ_LEN. */
hpa_status hpa_decode_prologue_plan(const hpa_attn_desc* desc, const void* q_in, const void* k_in,
                                    const void* v_in, const float* q_norm_w, const float* k_norm_w,
                                    float eps, double rope_theta, const int32_t* positions,
                                    const int32_t* page_table, void* k_cache, void* v_cache,
                                    const float* k_scale, const float* v_scale, void* q_out,
                                    int32_t* seq_lens_out, int32_t num_workers,
                                    int32_t min_tiles_per_worker, int32_t item_cost, int32_t tail_den,
                                    int32_t tail_chunk, int32_t item_order, void* plan_ws,
                                    size_t plan_ws_bytes, hipStream_t stream);

/* Synchronises the stream, then reads (and, if clear != 0, zeroes) the sticky
 * device error word of a plan workspace. */
hpa_status hpa_read_device_error(void* plan_ws, int32_t* code, int32_t clear, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Split-precision router GEMM (xiaodao.ai, "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半",
 * section "从实验表走到 SLA，还差一轮负载测试": the router keeps its top-k expert
 * choice by splitting its fp32 weight into a bf16 high part and a bf16 residual
 * and summing two tensor-core products).
 *
 * logits[t][e] = sum_k x[t][k] * (hi[e][k] + lo[e][k]), hi = bf16 nearest to W
 * (ties to even), lo = bf16 nearest to W - hi; every product is exact in fp32 and
 * the sums are fp32 accumulations (MFMA), so |logit - x.W| stays within
 * sum_k |x_k||W_k - hi_k - lo_k| + gamma_n sum_k |x_k|(|hi_k| + |lo_k|), n = 2H + 64,
 * gamma_n = n 2^-24 / (1 - n 2^-24). One pass (hi only) is the plain bf16 router.
 * The top-k experts of a token are its k largest logits, equal logits ordered by
 * the lower expert index, listed from the largest down. Inputs must be finite.
 *
 * Shapes: tokens T in [0, 2^20], experts E a multiple of 16 in [16, 1024],
 * hidden H a multiple of 32 in [32, 65536], top_k in [0, min(32, E)].
 * ------------------------------------------------------------------------- */

/* Splits and lays out the router weight once: w (device, fp32 [E][H] row-major,
 * 16-byte aligned) -> packed (device, E * H * 4 bytes, 16-byte aligned): for each
 * 16-expert x 32-dim tile, the hi half then the lo half, each in the order the
 * GEMM's 16-byte loads read (tile = (e/16)(H/32) + k/32, lane = 16((k%32)/8) + e%16;
 * hi at byte 2048 tile + 16 lane + 2 (k%8), lo 1024 bytes after it). Caller-owned
 * memory; asynchronous on `stream`. */
hpa_status hpa_router_pack_weights(const float* w, int32_t num_experts, int32_t hidden, void* packed,
                                   hipStream_t stream);

/* Bytes of device workspace hpa_router_gemm needs for this shape (fp32 partial
 * sums of the split K ranges; 0 when tokens == 0). */
hpa_status hpa_router_workspace_size(int32_t tokens, int32_t num_experts, int32_t hidden, size_t* bytes);

/* x (device, bf16 [T][H] row-major, 16-byte aligned), packed (from
 * hpa_router_pack_weights) -> logits (device, fp32 [T][E]) and, if top_k > 0,
 * topk_idx (device, int32 [T][top_k]) and topk_val (device, fp32 [T][top_k]).
 * passes = 2 for the split weight, 1 for its high part alone. workspace: device,
 * 16-byte aligned, at least hpa_router_workspace_size bytes. Results are
 * deterministic (fixed summation order). Host-side validation returns a non-OK
 * status and launches nothing; asynchronous on `stream`. */
hpa_status hpa_router_gemm(const void* x, const void* packed, int32_t tokens, int32_t num_experts,
                           int32_t hidden, int32_t passes, float* logits, int32_t top_k, int32_t* topk_idx,
                           float* topk_val, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Fused FP8 MoE layer for decode batches (xiaodao.ai, "HPC-Ops 把 TPOT 降 48.8%，
 * 用户未必快一半", section "为什么 batch 越大，数字越漂亮", the MoE paragraph: the
 * routing index, Gate-Up, activation with requantisation, Down GEMM and the top-k
 * merge as one chain with no standalone gather; bitbyai.com "vLLM × HPC-Ops …",
 * section "Breaking Down the Kernels", MoE backend: FP8 expert GEMMs with the token
 * rearrangement, activation and result gathering fused).
 *
 * For token t and slot k, e = topk_ids[t][k], w = topk_weights[t][k]:
 *   x8, sx = E4M3 codes and scale of x[t]: sx = max|x[t]| / 448, x8 = E4M3(x[t] / sx)
 *   g[j]   = sx * s1[e][j] * sum_h x8[h] W1[e][j][h]           (j < 2I; gate j < I, up I + i)
 *   a[i]   = silu(g[i]) * g[I + i]
 *   a8, sa = E4M3 codes and scale of a (sa = max|a| / 448)
 *   y[n]   = sa * s2[e][n] * sum_i a8[i] W2[e][n][i]
 *   out[t] = bf16( sum over k, in k order, of w * y )
 * (E4M3: OCP, nearest value, ties to even, saturating; fp32 arithmetic, fp32
 * accumulation of exact products; zero rows give zero scales and codes). A slot
 * whose expert id is outside [0, experts) adds nothing and sets
 * HPA_DEVERR_MOE_EXPERT in device_error (device int32, may be NULL).
 * Layouts (device, 16-byte aligned): x, out [T][H] bf16; topk_ids [T][K] int32;
 * topk_weights [T][K] fp32; w1 = W1 [E][2I][H] E4M3 codes (gate rows, then up rows)
 * and w2 = W2 [E][H][I] as packed by hpa_moe_pack_weights; s1 [E][2I], s2 [E][H]
 * fp32 (row-major). Shapes: tokens
 * 0 .. 1024, experts 1 .. 1024, top_k 1 .. 16, hidden and inter multiples of 128 up
 * to 4096, tokens x top_k <= 16384 (others: HPA_ERR_UNSUPPORTED, nothing launched).
 * workspace: at least hpa_moe_workspace_size bytes (token codes, the routing
 * index, the fp32 activations and their codes, the weighted per-slot results).
 * Five launches on `stream` (quantise + routing index, Gate-Up, requantise, Down,
 * merge); two when tokens x top_k <= 16 (each pair its own block: Gate-Up quantises
 * the tokens, Down requantises and merges; only the activations and their slice
 * maxima are written to the workspace). Nothing allocated; results are
 * deterministic and the same either way. */
/* Packs row-major E4M3 expert weights w [E][rows][cols] (device, 16-byte aligned)
 * into the tiled order hpa_moe_fused reads (packed: device, E * rows * cols bytes,
 * 16-byte aligned, another buffer): tile (e, rb, c) holds rows 16 rb .. + 16 and
 * cols 128 c .. + 128 at byte ((e rows/16 + rb) cols/128 + c) * 2048; inside it, for
 * row m and col 32 q + j (q < 4, j < 32) of the tile, lane l = m + 16 q: byte 16 l + j
 * for j < 16, 1024 + 16 l + j - 16 otherwise -- so every 16-byte-per-lane load of a
 * wave reads one contiguous 1 KB. rows a multiple of 16 up to 8192 (W1: 2I, W2: H),
 * cols a multiple of 128 up to 4096 (W1: H, W2: I). Once per weight; one launch. */
hpa_status hpa_moe_pack_weights(const void* w, int32_t experts, int32_t rows, int32_t cols, void* packed,
                                hipStream_t stream);
hpa_status hpa_moe_workspace_size(int32_t tokens, int32_t top_k, int32_t hidden, int32_t inter, size_t* bytes);
hpa_status hpa_moe_fused(const void* x, const int32_t* topk_ids, const float* topk_weights, const void* w1,
                         const float* s1, const void* w2, const float* s2, int32_t tokens, int32_t experts,
                         int32_t top_k, int32_t hidden, int32_t inter, void* out, void* workspace,
                         size_t workspace_bytes, int32_t* device_error, hipStream_t stream);

/* Measurement aid (not part of the attention path): reads `bytes` of device
 * memory at `buf` once and computes nothing from it, so its duration gives the
 * plain streaming-read bandwidth of this GPU, the practical ceiling for the
 * HBM-bound attention kernel. `bytes` must be a positive multiple of 16 and
 * `buf` 16-byte aligned. Each of `workgroups` workgroups (0: four per compute
 * unit of the current device) of 256 threads reads one contiguous slice with
 * 16-byte non-temporal loads, 8 in flight per lane. `sink` (device, at least
 * `workgroups` int32) receives a word only if a slice's XOR equals a fixed
 * constant, which keeps the loads without writing in practice. Asynchronous on
 * `stream`. */
hpa_status hpa_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups, int32_t* sink,
                                 hipStream_t stream);

const char* hpa_status_string(hpa_status status);
/* Message of the last non-OK status returned on the calling thread. */
const char* hpa_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* HPA_H */

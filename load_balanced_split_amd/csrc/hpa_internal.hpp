// Internal declarations shared by the host library and the HIP kernels of libhpa.
// gfx950 (CDNA4) only: wave64, MFMA 16x16x32 bf16, OCP E4M3 converts.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>
#include <algorithm>

#include "hpa.h"

namespace hpa {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;          // tokens per page == tokens per tile
constexpr int kMaxGroup = 16;      // query heads per KV head (MFMA N width)
constexpr int kWaves = 4;          // waves per attention workgroup (one worker)
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kAttnBlocksPerCu = 1;  // one worker per CU: the full register file for the K/V pipeline
constexpr int kPlanThreads = 1024;
constexpr int kHeaderInts = 16;

// In-page layout of the KV pools. Each (page, KV head) block holds 64 tokens x
// 128 dims (16 KB bf16, 8 KB E4M3), ordered so that every 16-byte-per-lane load
// the attention kernel issues reads one contiguous 1 KB: lane l of load i reads
// block bytes [i*1024 + 16 l, +16) of its unit (bf16: units of 32 tokens at byte
// 8192 * (t / 32); E4M3: one unit per block). The element index of (token t,
// dim d) inside a block:
//   bf16 K:  t%32 = 8a + 4b + q, d = 32c + 8j + e  ->  4096 (t/32) + 512 (4b + c) + 8 (16j + 4a + q) + e
//   bf16 V:  t%32 = 8j + e,      d = 16n + m       ->  4096 (t/32) + 512 n + 8 (16j + m) + e
//   E4M3 K:  t = 16a + 4b + q,   d = 64p + 16j + e ->  1024 (2b + p) + 16 (16j + 4a + q) + e
//   E4M3 V:  t = 16j + e,        d = 16n + m       ->  1024 n + 16 (16j + m) + e
// so that lane l = 16j + m of load i holds MFMA operand row m and k-slice j of
// the 16x16x32 products the kernel forms (scores from K, output from V).
constexpr int kBlockElems = kPage * kHeadDim;
__host__ __device__ inline int k_block_index(int t, int d, bool fp8) {
  if (!fp8) {
    const int r = t & 31;
    return 4096 * (t >> 5) + 512 * (4 * ((r >> 2) & 1) + (d >> 5)) +
           8 * (16 * ((d >> 3) & 3) + 4 * (r >> 3) + (r & 3)) + (d & 7);
  }
  return 1024 * (2 * ((t >> 2) & 3) + (d >> 6)) + 16 * (16 * ((d >> 4) & 3) + 4 * (t >> 4) + (t & 3)) + (d & 15);
}
__host__ __device__ inline int v_block_index(int t, int d, bool fp8) {
  if (!fp8) {
    const int r = t & 31;
    return 4096 * (t >> 5) + 512 * (d >> 4) + 8 * (16 * (r >> 3) + (d & 15)) + (r & 7);
  }
  return 1024 * (d >> 4) + 16 * (16 * (t >> 4) + (d & 15)) + (t & 15);
}

// Header slots of the plan workspace (int32).
enum : int {
  H_WP = 0, H_N = 1, H_S = 2, H_NITEMS = 3, H_NMERGE = 4, H_NPART = 5, H_ERR = 6, H_W = 7, H_ND = 8, H_WS = 9,
  H_B = 10, H_HKV = 11
};

// Offsets of the plan arrays, in int32 elements.
// Offsets are int32 (kernel arguments are read at launch, so they are kept small):
// with at most kMaxSeqs sequences and kMaxWorkers workers the plan stays far below
// 2^31 ints.
constexpr int64_t kMaxSeqs = int64_t(1) << 24;      // batch x KV heads
constexpr int64_t kMaxWorkers = int64_t(1) << 20;
struct PlanOffsets {
  int32_t header, C, worker_off, item_s, item_t0, item_t1, item_split, item_slot,
          num_splits, partial_base, merge_list, ne, gctr, sctr, qctr, total;
  int32_t max_items;
};

// A dynamic tail has at most this many chunks per worker, so a plan for W
// workers has at most (1 + kTailChunksPerWorker) W virtual workers.
constexpr int kTailChunksPerWorker = 4;

inline PlanOffsets plan_offsets(int64_t S, int64_t W) {
  PlanOffsets o{};
  auto al = [](int64_t x) { return (x + 63) & ~int64_t(63); };   // 256-byte aligned arrays
  const int64_t V = (1 + kTailChunksPerWorker) * W;                // virtual workers, at most
  const int64_t mi = V + S;
  int64_t p = 0;   // every value below fits in int32 for S <= kMaxSeqs, W <= kMaxWorkers
  o.header = static_cast<int32_t>(p);       p += al(kHeaderInts);
  o.C = static_cast<int32_t>(p);            p += al(S + 1);
  o.worker_off = static_cast<int32_t>(p);   p += al(V + 1);
  o.item_s = static_cast<int32_t>(p);       p += al(mi);
  o.item_t0 = static_cast<int32_t>(p);      p += al(mi);
  o.item_t1 = static_cast<int32_t>(p);      p += al(mi);
  o.item_split = static_cast<int32_t>(p);   p += al(mi);
  o.item_slot = static_cast<int32_t>(p);    p += al(mi);
  o.num_splits = static_cast<int32_t>(p);   p += al(S);
  o.partial_base = static_cast<int32_t>(p); p += al(S);
  o.merge_list = static_cast<int32_t>(p);   p += al(S);
  o.ne = static_cast<int32_t>(p);           p += al(S + 1);
  // arrival counters of the in-kernel merge (fused schedule): one per split group,
  // indexed by the group's first partial slot, and one per sequence; each is
  // returned to 0 by the workgroup that sees the last arrival
  o.gctr = static_cast<int32_t>(p);         p += al(mi);
  o.sctr = static_cast<int32_t>(p);         p += al(S);
  // dynamic tail: chunks claimed so far, workgroups finished; the last workgroup to
  // finish returns both to 0 (the planner clears them too)
  o.qctr = static_cast<int32_t>(p);         p += al(2);
  o.total = static_cast<int32_t>(p);
  o.max_items = static_cast<int32_t>(mi);
  return o;
}

// Partial-result workspace: acc [slots][G][128] fp32, then m [slots][G], l [slots][G].
struct PartialLayout {
  int64_t slots, acc, m, l, total_bytes;
};

inline PartialLayout partial_layout(int64_t slots, int64_t G) {
  PartialLayout p{};
  p.slots = slots;
  p.acc = 0;
  p.m = slots * G * kHeadDim * 4;
  p.l = p.m + slots * G * 4;
  p.total_bytes = p.l + slots * G * 4;
  return p;
}

// Partial slots a launch may need: one per item, and a plan has at most one item
// per (virtual worker, sequence boundary): (1 + kTailChunksPerWorker) W + S.
inline int64_t max_slots(int64_t W, int64_t S) { return (1 + kTailChunksPerWorker) * W + S; }

// Split results of one sequence are combined in a fixed order, in three levels:
// contiguous groups of kMergeGroup splits, each reduced max-first (the group's
// largest running max, then every split's weight 2^(m - max), then the weighted l
// and acc summed in split order); contiguous blocks of kMergeBlock group results,
// reduced the same way in group order; the block results folded in block order
// with a running max, starting from the empty state.
constexpr int kMergeGroup = 16;
constexpr int kMergeBlock = 16;

// Everything an attention kernel needs, passed by value.
struct AttnArgs {
  const uint16_t* q;           // [B, Hq, 128] bf16
  const uint8_t* k_cache;      // [P, Hkv, 8192] x elem, tiled page blocks
  const uint8_t* v_cache;      // [P, Hkv, 8192] x elem, tiled page blocks
  const float* k_scale;
  const float* v_scale;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t* plan;               // plan workspace (may be null for static schedules)
  int32_t* err;                // sticky device error word (may be null: errors are dropped)
  int32_t* gctr;               // in-kernel merge arrival counters (fused schedule), in plan
  int32_t* sctr;
  int32_t* qctr;               // dynamic tail counters [claimed, finished], in plan
  float* part_acc;
  float* part_m;
  float* part_l;
  uint16_t* out;               // [B, Hq, 128] bf16
  PlanOffsets po;
  int batch, hq, hkv, group, max_pages, num_pages;
  int workers;                 // W the kernels were launched for (plan header must agree)
  int64_t slots;               // partial slots available (max_slots(W, S))
  float sm_scale;
  // static schedules
  int static_splits;           // S_split
  int static_chunk;            // fixed chunk (flavour "chunk"), 0 for flavour "splits"
  int min_tiles;               // fused schedule: minimum tiles per active worker
  int item_cost;               // fused schedule: virtual tiles charged per item
  int tail_den, tail_chunk;    // fused schedule: dynamic tail (last 1/tail_den of the positions)
  // instrumented builds only: per-wave records [block][wave][kTraceWords]
  uint64_t* trace;
};

// Instrumented builds (HPA_TRACE) append a per-wave record area to the partial
// workspace: for each workgroup (up to W + S of them) and wave, 16 words:
// start and end of the wave on the 100 MHz realtime counter, the hardware
// wave/CU id register with the XCC id in the upper half, the units computed,
// four start-up times (each after waiting for all of the wave's loads so far:
// work range known, first item known, its length known, its q and page ids
// known), then for each of the wave's first kTraceItems items three times: its
// first unit issued, its last unit computed, its combine done; then the
// completion times of the wave's first kTraceUnits units.
constexpr int kTraceItems = 4;
constexpr int kTraceStart = 4;
constexpr int kTraceUnits = 48;
constexpr int kTraceWords = 4 + kTraceStart + 3 * kTraceItems + kTraceUnits;
#ifdef HPA_TRACE
constexpr bool kTraceBuild = true;
#else
constexpr bool kTraceBuild = false;
#endif
inline int64_t trace_bytes(int64_t blocks) { return kTraceBuild ? blocks * kWaves * kTraceWords * 8 : 0; }

// Comparison builds (HPA_VALU_PRODUCTS) compute both products of the attention
// kernels, Q.K^T and P.V, with VALU bf16 dot products instead of MFMA, from the
// same registers and the same cache layout, for up to kValuMaxGroup query heads
// per KV head. Such a library exists to measure the MFMA choice; it is otherwise
// identical.
#ifdef HPA_VALU_PRODUCTS
constexpr bool kValuProducts = true;
#else
constexpr bool kValuProducts = false;
#endif
constexpr int kValuMaxGroup = 8;

// Closed forms of the balanced partition, shared by the planner kernel and the
// in-kernel planning of the fused schedule. Worker w owns global positions
// [w*N/W', (w+1)*N/W'); the owner of position t is floor(((t+1)*W' - 1)/N)
// (N counts tiles, plus the virtual per-item tiles when items carry a cost).
// `small` (both products below 2^31) selects exact 32-bit arithmetic.
__device__ inline int owner_of_tile(int t, int Wp, int N, bool small) {
  if (small) return static_cast<int>((static_cast<uint32_t>(t + 1) * Wp - 1) / static_cast<uint32_t>(N));
  return static_cast<int>(((int64_t(t) + 1) * Wp - 1) / N);
}

__device__ inline int range_begin(int w, int Wp, int N, bool small) {
  // a power-of-two worker count (one worker per CU: 256 on MI355X) divides by a shift
  if ((Wp & (Wp - 1)) == 0) {
    const int sh = __builtin_ctz(static_cast<uint32_t>(Wp));
    if (small) return static_cast<int>((static_cast<uint32_t>(w) * N) >> sh);
    return static_cast<int>((int64_t(w) * N) >> sh);
  }
  if (small) return static_cast<int>(static_cast<uint32_t>(w) * N / static_cast<uint32_t>(Wp));
  return static_cast<int>(int64_t(w) * N / Wp);
}

__device__ inline bool small_products(int N, int Wp) {
  return (int64_t(N) + 1) * (int64_t(Wp) + 1) < (int64_t(1) << 31);
}

// The balanced partition of Np positions (N real tiles) with a dynamic tail: the
// last T = Np / tail_den positions (none without a tail) are cut into D chunks
// claimed at run time, the first A = Np - T are split evenly over Ws = min(Wp, A)
// static workers (Wp active workers), so every virtual worker owns at least one
// position. Virtual worker v < Ws is static worker v, virtual worker Ws + c is chunk c.
struct Partition {
  int Np, Wp, Ws, A, T, D;
  bool small_a, small_t;      // exact 32-bit products

  __device__ static Partition make(int N, int Np, int W, int min_tiles, int tail_den, int tail_chunk) {
    Partition p;
    p.Np = Np;
    p.Wp = N == 0 ? 0 : min(W, max(1, Np / min_tiles));
    p.T = (tail_den > 0 && N > 0) ? Np / tail_den : 0;
    p.A = Np - p.T;
    p.Ws = min(p.Wp, p.A);
    p.D = p.T > 0 ? min((p.T + tail_chunk - 1) / tail_chunk, kTailChunksPerWorker * W) : 0;
    p.small_a = small_products(p.A, p.Ws);
    p.small_t = small_products(p.T, p.D);
    return p;
  }
  __device__ int V() const { return Ws + D; }
  // first position of virtual worker v, 0 <= v <= V (begin(V) = Np)
  __device__ int begin(int v) const {
    if (v < Ws) return range_begin(v, Ws, A, small_a);
    return A + (v == Ws ? 0 : range_begin(v - Ws, D, T, small_t));
  }
  // virtual worker owning position p, 0 <= p < Np
  __device__ int owner(int p) const {
    if (p < A) return owner_of_tile(p, Ws, A, small_a);
    return Ws + owner_of_tile(p - A, D, T, small_t);
  }
};

// Largest s in [0, S) with C[s] <= t, for 0 <= t < C[S].
__device__ inline int seq_of_tile(const int32_t* C, int S, int t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (C[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline int tiles_of(int L) { return (L + kPage - 1) / kPage; }

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves: shifts
// by 1, 2, 4, 8 within each row of 16 lanes (lanes whose source falls outside
// the row add 0), then lane 15 of rows 0 and 2 is added to rows 1 and 3, and
// lane 31 to rows 2 and 3. Every lane must be active.
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Launch wrappers (defined in the .hip files). Return hipSuccess or the launch error.
hipError_t launch_plan(const int32_t* seq_lens, int batch, int hkv, int max_pages, int num_workers,
                       int min_tiles, int item_cost, int tail_den, int tail_chunk, int order, int32_t* plan,
                       const PlanOffsets& po, hipStream_t stream);
hipError_t launch_attn_balanced(const AttnArgs& a, bool fp8, bool merge_in_kernel, int num_workers,
                                hipStream_t stream);
hipError_t launch_attn_static(const AttnArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_attn_fused(const AttnArgs& a, bool fp8, bool merge_in_kernel, int num_workers, hipStream_t stream);
// merge modes: which schedule produced the partials
enum MergeMode : int { MERGE_PLAN = 0, MERGE_STATIC = 1, MERGE_FUSED = 2 };
hipError_t launch_merge(const AttnArgs& a, MergeMode mode, hipStream_t stream);
constexpr int kFusedMaxSeqs = 2048;  // sequences (B x Hkv) the fused schedules plan in LDS; larger
                                     // batches plan in the workspace first (one launch more)
constexpr int kRegPlanSeqs = 256;    // up to this many, every wave plans in registers instead
// The planner's arguments when the prologue launch also plans (hpa_decode_prologue_plan).
struct PlanArgs {
  int32_t* ws;
  PlanOffsets po;
  int workers, min_tiles, item_cost, tail_den, tail_chunk, order;
};
hipError_t launch_prologue(const hpa_attn_desc& d, const uint16_t* q_in, const uint16_t* k_in,
                           const uint16_t* v_in, const float* q_norm_w, const float* k_norm_w,
                           float eps, double rope_theta, const int32_t* positions,
                           const int32_t* page_table, uint8_t* k_cache, uint8_t* v_cache,
                           const float* k_scale, const float* v_scale, uint16_t* q_out,
                           int32_t* seq_lens_out, int32_t* err_word, const PlanArgs* plan, hipStream_t stream);
hipError_t launch_clear_word(int32_t* word, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, int32_t* sink, hipStream_t stream);

// Where the allocation-free entry point puts what normally lives in the plan
// workspace at shape-dependent offsets: the error word and the in-kernel merge's
// arrival counters (which must be zero at every launch, so they stay at one place).
struct AttnRedirect {
  int32_t* err;
  int32_t* gctr;
  int32_t* sctr;
};
// hpa_decode_attn's body (host.cpp); redirect may be null.
hpa_status decode_attn(const hpa_attn_desc* desc, hpa_sched sched, const void* q, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                       const int32_t* page_table, int32_t num_workers, void* plan_ws, size_t plan_ws_bytes,
                       void* partial_ws, size_t partial_ws_bytes, void* out, int32_t flags,
                       const AttnRedirect* redirect, hipStream_t stream);
// Validates desc, resolves num_workers (0: the schedule's default) and returns the
// plan and partial workspace bytes hpa_decode_attn needs for that worker count.
hpa_status attn_workspace_bytes(const hpa_attn_desc* desc, hpa_sched sched, int32_t num_workers, int32_t* workers,
                                size_t* plan_bytes, size_t* partial_bytes);

// Records a message for hpa_last_error_message() on this thread and returns st
// (defined in host.cpp; for the entry points of other source files).
hpa_status report_status(hpa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

int attn_blocks_per_cu(bool fp8);         // persistent attention kernels
int attn_static_blocks_per_cu(bool fp8);  // static split-KV attention kernel

}  // namespace hpa

// The balanced planner as a device function of one workgroup, shared by the
// planner kernel and the prologue kernel's planning workgroup.
//
// xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section "为什么 batch 越大，
// 数字越漂亮": live KV is cut into 64-token tiles and the global tile list is
// spread as evenly as possible over persistent workers; bitbyai.com "vLLM ×
// HPC-Ops …", section "Breaking Down the Kernels": recomputed every decode step.
//
// Output (all int32, see PlanOffsets): prefix sum C over per-sequence tile
// counts, W' active workers, items (s, t0, t1, split, slot) cut at sequence
// boundaries, num_splits, partial_base and the list of sequences to merge
// (num_splits != 1).
// Item cost c (bitbyai.com, same section: the scheduler weighs work by
// progress): starting an item costs as much as c tiles, so c virtual tiles stand
// in front of every non-empty sequence of the global list. Sequence s then
// occupies positions [P[s], P[s+1]) with P[s] = C[s] + c * NE[s] (NE: non-empty
// sequences before s), its real tiles at [P[s] + c, P[s+1]); N' = P[S]. Worker w
// owns positions [w*N'/W', (w+1)*N'/W'), W' = min(W, max(1, N'/min_tiles)), and
// its items are the real tiles it owns; c = 0 is the plain even split.
// Dynamic tail (same section: the scheduler evaluates progress as it goes): the
// last T = N' / tail_den positions are cut into D chunks that workers claim at run
// time; the first A = N' - T are split over Ws = min(W', A) static workers. The
// plan lists virtual workers v < Ws + D (static ranges, then chunks) in order, so
// it does not depend on who claims which chunk. tail_den 0: no tail, Ws = W'.
// Every quantity is closed-form (Partition), so no thread walks another worker's
// range: the first virtual worker of sequence s owns position P[s] + c, the last
// owns P[s+1] - 1, and all those between hold part of s.
#pragma once
#include "hpa_internal.hpp"

namespace hpa {

// Exclusive scans of two ints per thread over the whole block (one set of
// barriers for both); also returns the two totals.
template <int NT>
__device__ void block_exclusive_scan2(int va, int vb, int2* tmp /* NT/64 + 1 */, int& ra, int& rb, int& ta,
                                      int& tb) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int nw = NT / 64;
  const int xa = wave_incl_scan(va), xb = wave_incl_scan(vb);
  if (lane == 63) tmp[wid] = make_int2(xa, xb);
  __syncthreads();
  if (wid == 0) {
    const int2 t = lane < nw ? tmp[lane] : make_int2(0, 0);
    const int ua = wave_incl_scan(t.x), ub = wave_incl_scan(t.y);
    if (lane < nw) tmp[lane] = make_int2(ua - t.x, ub - t.y);
    if (lane == nw - 1) tmp[nw] = make_int2(ua, ub);
  }
  __syncthreads();
  ra = xa - va + tmp[wid].x;
  rb = xb - vb + tmp[wid].y;
  ta = tmp[nw].x;
  tb = tmp[nw].y;
  __syncthreads();
}

// Batches up to this many sequences keep the planner's arrays in LDS; larger ones
// work on the copies in the workspace.
constexpr int kPlanLdsSeqs = 3072;

// Largest s in [0, S) with P[s] = C[s] + c * NE[s] <= t, for 0 <= t < P[S].
__device__ inline int seq_of_pos(const int32_t* C, const int32_t* NE, int c, int S, int t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (C[mid] + c * NE[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The planner over one workgroup of NT threads. lens(b) gives request b's live
// length (plan_kernel: seq_lens[b]; the prologue's planner: the length after its
// append); everything else as in hpa_plan.
template <int NT, bool LDS, class Lens>
__device__ void plan_block(const Lens& lens, int B, int Hkv, int max_pages, int W, int min_tiles, int cost,
                           int tail_den, int tail_chunk, int order, int32_t* __restrict__ ws, const PlanOffsets& po) {
  __shared__ int2 tmp[NT / 64 + 1];
  __shared__ int sh_bad;
  __shared__ int sC[LDS ? kPlanLdsSeqs + 1 : 1];
  __shared__ int sNE[LDS ? kPlanLdsSeqs + 1 : 1];
  __shared__ int sNS[LDS ? kPlanLdsSeqs : 1];
  __shared__ int sPB[LDS ? kPlanLdsSeqs : 1];
  const int tid = threadIdx.x;
  const int S = B * Hkv;
  int32_t* hdr = ws + po.header;
  int32_t* C = LDS ? sC : ws + po.C;
  int32_t* NE = LDS ? sNE : ws + po.ne;
  if (tid == 0) sh_bad = 0;
  __syncthreads();

  // 1. tile counts, their prefix sum C, and the prefix count NE of non-empty sequences
  int carry = 0, carry_ne = 0;
  for (int base = 0; base < S; base += NT) {
    const int s = base + tid;
    int n = 0;
    if (s < S) {
      int L = lens(s / Hkv);
      if (L < 0 || L > max_pages * kPage) {
        sh_bad = 1;
        L = 0;
      }
      n = tiles_of(L);
    }
    int ex, ex_ne, tot, tot_ne;
    block_exclusive_scan2<NT>(n, n > 0 ? 1 : 0, tmp, ex, ex_ne, tot, tot_ne);
    if (s < S) {
      C[s] = carry + ex;
      NE[s] = carry_ne + ex_ne;
    }
    carry += tot;
    carry_ne += tot_ne;
  }
  if (tid == 0) {
    C[S] = carry;
    NE[S] = carry_ne;
  }
  __syncthreads();
  const int N = carry;
  const int Np = N + cost * carry_ne;               // positions: real plus virtual tiles
  const Partition part = Partition::make(N, Np, W, min_tiles, tail_den, tail_chunk);
  const int V = part.V();
  auto P = [&](int s) { return C[s] + cost * NE[s]; };

  // 2. splits per sequence, partial slot bases, merge list
  int32_t* num_splits = LDS ? sNS : ws + po.num_splits;
  int32_t* pbase = LDS ? sPB : ws + po.partial_base;
  int32_t* mlist = ws + po.merge_list;
  int carry_p = 0, carry_m = 0;
  for (int base = 0; base < S; base += NT) {
    const int s = base + tid;
    int ns = 0;
    if (s < S) {
      if (C[s + 1] > C[s])
        ns = part.owner(P(s + 1) - 1) - part.owner(P(s) + cost) + 1;
      num_splits[s] = ns;
    }
    int ex_p, ex_m, tot_p, tot_m;
    block_exclusive_scan2<NT>((s < S && ns > 1) ? ns : 0, (s < S && ns != 1) ? 1 : 0, tmp, ex_p, ex_m, tot_p, tot_m);
    if (s < S) {
      pbase[s] = carry_p + ex_p;
      if (ns != 1) mlist[carry_m + ex_m] = s;
    }
    carry_p += tot_p;
    carry_m += tot_m;
  }

  // 3. items per virtual worker and their CSR offsets
  int32_t* woff = ws + po.worker_off;
  int carry_i = 0;
  int my_off = 0;                     // worker tid's first item (kept when one pass covers all workers)
  for (int base = 0; base < V; base += NT) {
    const int w = base + tid;
    int cnt = 0;
    if (w < V) {
      const int a = part.begin(w), e = part.begin(w + 1);
      // sf / sl hold positions a / e - 1 (both non-empty); the sequences between them
      // lie inside [a, e); sf and sl count when their real tiles start before e
      const int sf = seq_of_pos(C, NE, cost, S, a), sl = seq_of_pos(C, NE, cost, S, e - 1);
      cnt = NE[sl] - NE[sf] + 1 - (P(sf) + cost >= e ? 1 : 0) - (sl != sf && P(sl) + cost >= e ? 1 : 0);
    }
    int ex, unused, tot, unused_t;
    block_exclusive_scan2<NT>(cnt, 0, tmp, ex, unused, tot, unused_t);
    if (w < V) woff[w] = my_off = carry_i + ex;
    carry_i += tot;
  }
  if (tid == 0) woff[V] = carry_i;
  __syncthreads();

  // 4. emit items, worker by worker, in sequence order -- or (order 1 / 2) in two passes:
  // the sequences a worker holds whole, then the pieces of split ones (1), or the
  // reverse (2); each pass in sequence order. Ranks and slots do not depend on it.
  int32_t* is = ws + po.item_s;
  int32_t* it0 = ws + po.item_t0;
  int32_t* it1 = ws + po.item_t1;
  int32_t* isp = ws + po.item_split;
  int32_t* isl = ws + po.item_slot;
  for (int w = tid; w < V; w += NT) {
    const int a = part.begin(w), e = part.begin(w + 1);
    const int s_first = seq_of_pos(C, NE, cost, S, a);
    int pos = V <= NT ? my_off : woff[w];
    for (int pass = 0; pass < (order ? 2 : 1); ++pass) {
      const bool want_whole = (order == 1) == (pass == 0);
      for (int s = s_first; s < S && P(s) < e; ++s) {
        if (C[s + 1] == C[s]) continue;
        if (order && (num_splits[s] == 1) != want_whole) continue;
        const int r0 = P(s) + cost, r1 = P(s + 1);      // the real tiles of s
        const int lo = max(a, r0), hi = min(e, r1);
        if (lo >= hi) continue;
        const int split = w - part.owner(r0);
        is[pos] = s;
        it0[pos] = lo - r0;
        it1[pos] = hi - r0;
        isp[pos] = split;
        isl[pos] = num_splits[s] > 1 ? pbase[s] + split : -1;
        ++pos;
      }
    }
  }
  if (LDS) {
    // publish the per-sequence arrays
    for (int s = tid; s <= S; s += NT) {
      ws[po.C + s] = C[s];
      if (s < S) {
        ws[po.num_splits + s] = num_splits[s];
        ws[po.partial_base + s] = pbase[s];
      }
    }
  }
  if (tid == 0) {
    hdr[H_WP] = part.Wp;
    hdr[H_WS] = part.Ws;
    hdr[H_ND] = part.D;
    ws[po.qctr] = 0;
    ws[po.qctr + 1] = 0;
    hdr[H_N] = N;
    hdr[H_S] = S;
    hdr[H_B] = B;
    hdr[H_HKV] = Hkv;
    hdr[H_NITEMS] = carry_i;
    hdr[H_NMERGE] = carry_m;
    hdr[H_NPART] = carry_p;
    hdr[H_W] = W;
    if (sh_bad) atomicOr(&hdr[H_ERR], HPA_DEVERR_SEQ_LEN);
  }
}

}  // namespace hpa

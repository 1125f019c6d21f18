// Balanced split-KV planner: one workgroup turns live lengths into a work list.
//
// xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section "为什么 batch 越大，
// 数字越漂亮": live KV is cut into 64-token tiles and the global tile list is
// spread as evenly as possible over persistent workers; bitbyai.com "vLLM ×
// HPC-Ops …", section "Breaking Down the Kernels": recomputed every decode step.
//
// Output (all int32, see PlanOffsets): prefix sum C over per-sequence tile
// counts, W' active workers, worker w owning global tiles [w*N/W', (w+1)*N/W'),
// items (s, t0, t1, split, slot) cut at sequence boundaries, num_splits,
// partial_base and the list of sequences to merge (num_splits != 1).
// Every quantity is closed-form, so no thread walks another worker's range:
//   worker owning tile t      = floor(((t+1) * W' - 1) / N)
//   first worker of sequence s = owner of tile C[s], last = owner of C[s+1]-1.
#include "hpa_internal.hpp"

namespace hpa {
namespace {

// Exclusive scan of one int per thread over the whole block; also returns the total.
__device__ int block_exclusive_scan(int v, int* tmp /* kPlanThreads/64 + 1 */, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int nw = kPlanThreads / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int t = lane < nw ? tmp[lane] : 0;
    int u = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(u, o, 64);
      if (lane >= o) u += y;
    }
    if (lane < nw) tmp[lane] = u - t;
    if (lane == nw - 1) tmp[nw] = u;
  }
  __syncthreads();
  int r = x - v + tmp[wid];
  total = tmp[nw];
  __syncthreads();
  return r;
}

__device__ inline int tiles_of(int L) { return (L + kPage - 1) / kPage; }

// Largest s in [0, S) with C[s] <= t, for 0 <= t < C[S].
__device__ inline int seq_of_tile(const int32_t* C, int S, int t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (C[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline int owner_of_tile(int64_t t, int64_t Wp, int64_t N) {
  return static_cast<int>(((t + 1) * Wp - 1) / N);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int B, int Hkv, int max_pages, int W, int min_tiles,
    int32_t* __restrict__ ws, PlanOffsets po) {
  __shared__ int tmp[kPlanThreads / 64 + 1];
  __shared__ int sh_bad;
  const int tid = threadIdx.x;
  const int S = B * Hkv;
  int32_t* hdr = ws + po.header;
  int32_t* C = ws + po.C;
  int32_t* NE = ws + po.ne;
  if (tid == 0) sh_bad = 0;
  __syncthreads();

  // 1. tile counts, their prefix sum C, and the prefix count NE of non-empty sequences
  int carry = 0, carry_ne = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int n = 0;
    if (s < S) {
      int L = seq_lens[s / Hkv];
      if (L < 0 || L > max_pages * kPage) {
        sh_bad = 1;
        L = 0;
      }
      n = tiles_of(L);
    }
    int tot, tot_ne;
    int ex = block_exclusive_scan(n, tmp, tot);
    int ex_ne = block_exclusive_scan(n > 0 ? 1 : 0, tmp, tot_ne);
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
  const int Wp = N == 0 ? 0 : min(W, max(1, N / min_tiles));

  // 2. splits per sequence, partial slot bases, merge list
  int32_t* num_splits = ws + po.num_splits;
  int32_t* pbase = ws + po.partial_base;
  int32_t* mlist = ws + po.merge_list;
  int carry_p = 0, carry_m = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int ns = 0;
    if (s < S) {
      const int c0 = C[s], c1 = C[s + 1];
      if (c1 > c0) ns = owner_of_tile(c1 - 1, Wp, N) - owner_of_tile(c0, Wp, N) + 1;
      num_splits[s] = ns;
    }
    int tot_p, tot_m;
    int ex_p = block_exclusive_scan((s < S && ns > 1) ? ns : 0, tmp, tot_p);
    int ex_m = block_exclusive_scan((s < S && ns != 1) ? 1 : 0, tmp, tot_m);
    if (s < S) {
      pbase[s] = carry_p + ex_p;
      if (ns != 1) mlist[carry_m + ex_m] = s;
    }
    carry_p += tot_p;
    carry_m += tot_m;
  }

  // 3. items per worker and their CSR offsets
  int32_t* woff = ws + po.worker_off;
  int carry_i = 0;
  for (int base = 0; base < Wp; base += kPlanThreads) {
    const int w = base + tid;
    int cnt = 0;
    if (w < Wp) {
      const int a = static_cast<int>(int64_t(w) * N / Wp);
      const int e = static_cast<int>(int64_t(w + 1) * N / Wp);
      const int sf = seq_of_tile(C, S, a), sl = seq_of_tile(C, S, e - 1);
      cnt = NE[sl] - NE[sf] + 1;
    }
    int tot;
    int ex = block_exclusive_scan(cnt, tmp, tot);
    if (w < Wp) woff[w] = carry_i + ex;
    carry_i += tot;
  }
  if (tid == 0) woff[Wp] = carry_i;
  __syncthreads();

  // 4. emit items, worker by worker, in sequence order
  int32_t* is = ws + po.item_s;
  int32_t* it0 = ws + po.item_t0;
  int32_t* it1 = ws + po.item_t1;
  int32_t* isp = ws + po.item_split;
  int32_t* isl = ws + po.item_slot;
  for (int w = tid; w < Wp; w += kPlanThreads) {
    int a = static_cast<int>(int64_t(w) * N / Wp);
    const int e = static_cast<int>(int64_t(w + 1) * N / Wp);
    int s = seq_of_tile(C, S, a);
    int pos = woff[w];
    while (a < e) {
      const int c0 = C[s], c1 = C[s + 1];
      if (c1 > c0) {
        const int t1 = min(e, c1);
        const int split = w - owner_of_tile(c0, Wp, N);
        is[pos] = s;
        it0[pos] = a - c0;
        it1[pos] = t1 - c0;
        isp[pos] = split;
        isl[pos] = num_splits[s] > 1 ? pbase[s] + split : -1;
        ++pos;
        a = t1;
      }
      ++s;
    }
  }
  if (tid == 0) {
    hdr[H_WP] = Wp;
    hdr[H_N] = N;
    hdr[H_S] = S;
    hdr[H_NITEMS] = carry_i;
    hdr[H_NMERGE] = carry_m;
    hdr[H_NPART] = carry_p;
    hdr[H_W] = W;
    if (sh_bad) atomicOr(&hdr[H_ERR], HPA_DEVERR_SEQ_LEN);
  }
}

__global__ void clear_word_kernel(int32_t* w) { *w = 0; }

}  // namespace

hipError_t launch_plan(const int32_t* seq_lens, int batch, int hkv, int max_pages, int num_workers,
                       int min_tiles, int32_t* plan, const PlanOffsets& po, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch, hkv,
                     max_pages, num_workers, min_tiles, plan, po);
  return hipGetLastError();
}

hipError_t launch_clear_word(int32_t* word, hipStream_t stream) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, word);
  return hipGetLastError();
}

}  // namespace hpa

// Balanced split-KV planner kernel: one workgroup turns live lengths into a work
// list (the planner itself, with its sources and closed forms, is plan_block.hpp).
#include "plan_block.hpp"

namespace hpa {
namespace {

struct SeqLens {
  const int32_t* p;
  __device__ int operator()(int b) const { return p[b]; }
};

template <bool LDS>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int B, int Hkv, int max_pages, int W, int min_tiles,
    int cost, int tail_den, int tail_chunk, int order, int32_t* __restrict__ ws, PlanOffsets po) {
  plan_block<kPlanThreads, LDS>(SeqLens{seq_lens}, B, Hkv, max_pages, W, min_tiles, cost, tail_den, tail_chunk,
                                order, ws, po);
}

__global__ void clear_word_kernel(int32_t* w) { *w = 0; }

}  // namespace

hipError_t launch_plan(const int32_t* seq_lens, int batch, int hkv, int max_pages, int num_workers,
                       int min_tiles, int item_cost, int tail_den, int tail_chunk, int order, int32_t* plan,
                       const PlanOffsets& po, hipStream_t stream) {
  if (int64_t(batch) * hkv <= kPlanLdsSeqs)
    hipLaunchKernelGGL(plan_kernel<true>, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch, hkv,
                       max_pages, num_workers, min_tiles, item_cost, tail_den, tail_chunk, order, plan, po);
  else
    hipLaunchKernelGGL(plan_kernel<false>, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch, hkv,
                       max_pages, num_workers, min_tiles, item_cost, tail_den, tail_chunk, order, plan, po);
  return hipGetLastError();
}

hipError_t launch_clear_word(int32_t* word, hipStream_t stream) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, word);
  return hipGetLastError();
}

}  // namespace hpa

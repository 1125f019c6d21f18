// Balanced split-KV planner kernel: one workgroup turns live lengths into a work
// list (the planner itself, with its sources and closed forms, is plan_block.hpp).
#include "plan_block.hpp"

namespace hpa {
namespace {

struct SeqLens {
  const int32_t* p;
  __device__ int operator()(int b) const { return p[b]; }
};

// NT threads: kPlanThreads, or kPlanThreadsSmall when the sequences and the virtual
// workers each fit one pass of them (fewer waves meet at each of the planner's
// barriers: 5.9 -> 5.5 us for 32 sequences and 256 workers)
template <int NT, bool LDS>
__global__ __launch_bounds__(NT) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int B, int Hkv, int max_pages, int W, int min_tiles,
    int cost, int tail_den, int tail_chunk, int order, int32_t* __restrict__ ws, PlanOffsets po) {
  plan_block<NT, LDS>(SeqLens{seq_lens}, B, Hkv, max_pages, W, min_tiles, cost, tail_den, tail_chunk, order, ws,
                      po);
}
constexpr int kPlanThreadsSmall = 256;

__global__ void clear_word_kernel(int32_t* w) { *w = 0; }

}  // namespace

hipError_t launch_plan(const int32_t* seq_lens, int batch, int hkv, int max_pages, int num_workers,
                       int min_tiles, int item_cost, int tail_den, int tail_chunk, int order, int32_t* plan,
                       const PlanOffsets& po, hipStream_t stream) {
  const int64_t S = int64_t(batch) * hkv;
  // virtual workers: the static ones plus at most kTailChunksPerWorker tail chunks each
  const int64_t V = tail_den > 0 ? (1 + kTailChunksPerWorker) * int64_t(num_workers) : num_workers;
  if (S <= kPlanThreadsSmall && V <= kPlanThreadsSmall)
    hipLaunchKernelGGL((plan_kernel<kPlanThreadsSmall, true>), dim3(1), dim3(kPlanThreadsSmall), 0, stream, seq_lens,
                       batch, hkv, max_pages, num_workers, min_tiles, item_cost, tail_den, tail_chunk, order, plan, po);
  else if (S <= kPlanLdsSeqs)
    hipLaunchKernelGGL((plan_kernel<kPlanThreads, true>), dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch,
                       hkv, max_pages, num_workers, min_tiles, item_cost, tail_den, tail_chunk, order, plan, po);
  else
    hipLaunchKernelGGL((plan_kernel<kPlanThreads, false>), dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch,
                       hkv, max_pages, num_workers, min_tiles, item_cost, tail_den, tail_chunk, order, plan, po);
  return hipGetLastError();
}

hipError_t launch_clear_word(int32_t* word, hipStream_t stream) {
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, word);
  return hipGetLastError();
}

}  // namespace hpa

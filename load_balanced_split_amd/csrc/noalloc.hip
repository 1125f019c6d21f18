// Allocation-free decode attention: hpa_decode_attn with its two workspaces carved
// out of one statically sized device array instead of taking them from the caller.
//
// The array (`scratch`) is a file-scope device variable, so every GPU the library
// runs on holds its own copy from module load until the process ends; nothing is
// allocated or freed here. In host code `scratch` names a host-side stand-in, not
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is ever handed to kernels.
//
// Layout of the array: [error word, pad to 256 B][arrival counters][plan | partials].
// The plan and partial areas move with the batch shape, but the in-kernel merge's
// arrival counters must read zero at every launch, so they have a fixed place of
// their own (zero at load, cleared once more at set-up, and returned to zero by the
// kernels that use them).
#include "hpa_internal.hpp"

#include <mutex>
#include <vector>

namespace hpa {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
// The fused schedules plan without a dynamic tail, so the tail's claim counters (in
// the plan area, which moves with the shape) are never touched here.
static_assert(HPA_FUSED_TAIL_DEN == 0, "the allocation-free call keeps no tail counters");
constexpr int kNoAllocMaxWorkers = 4096;
constexpr int64_t kCounterInts = (1 + kTailChunksPerWorker) * int64_t(kNoAllocMaxWorkers) + kFusedMaxSeqs + kFusedMaxSeqs;
constexpr size_t kHeadBytes = 256;                                   // error word, padded
constexpr size_t kCounterBytes = ((size_t(kCounterInts) * 4 + 255) / 256) * 256;
constexpr size_t kAreaOffset = kHeadBytes + kCounterBytes;           // plan, then partials

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void clear_ints_kernel(int32_t* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0;
}

std::mutex g_mu;
std::vector<unsigned char*> g_ptr;   // device address of `scratch`, per device (null: not set up)

// The device address of this device's copy of `scratch`; the first call on a device
// looks it up (with that device current) and clears the error word and counters on
// `stream`.
hpa_status scratch_of(int device, hipStream_t stream, unsigned char** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (static_cast<size_t>(device) >= g_ptr.size()) g_ptr.resize(device + 1, nullptr);
  if (!g_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return report_status(HPA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d", device);
    const int64_t n = static_cast<int64_t>(kAreaOffset / 4);
    hipLaunchKernelGGL(clear_ints_kernel, dim3(64), dim3(256), 0, stream, static_cast<int32_t*>(p), n);
    if (hipGetLastError() != hipSuccess) return report_status(HPA_ERR_LAUNCH, "scratch clear launch failed");
    g_ptr[device] = static_cast<unsigned char*>(p);
  }
  *out = g_ptr[device];
  return HPA_OK;
}

}  // namespace
}  // namespace hpa

extern "C" hpa_status hpa_decode_attn_noalloc(const hpa_attn_desc* desc, hpa_sched sched, const void* q,
                                              const void* k_cache, const void* v_cache, const float* k_scale,
                                              const float* v_scale, const int32_t* seq_lens,
                                              const int32_t* page_table, int32_t num_workers, void* out,
                                              int32_t* device_error, hipStream_t stream) {
  using namespace hpa;
  if (sched != HPA_SCHED_BALANCED_FUSED && sched != HPA_SCHED_BALANCED_SINGLE && sched != HPA_SCHED_STATIC_SPLITS &&
      sched != HPA_SCHED_STATIC_CHUNK)
    return report_status(HPA_ERR_INVALID_ARG, "sched %d: the allocation-free call runs the fused, single-launch "
                         "and static schedules (they need no hpa_plan call)", static_cast<int>(sched));
  if (num_workers > kNoAllocMaxWorkers)
    return report_status(HPA_ERR_UNSUPPORTED, "num_workers %d > %d (allocation-free call)", num_workers,
                         kNoAllocMaxWorkers);
  int32_t W = 0;
  size_t plan_bytes = 0, partial_bytes = 0;
  hpa_status st = attn_workspace_bytes(desc, sched, num_workers, &W, &plan_bytes, &partial_bytes);
  if (st != HPA_OK) return st;
  if (W > kNoAllocMaxWorkers)
    return report_status(HPA_ERR_UNSUPPORTED, "%d workers > %d (allocation-free call)", W, kNoAllocMaxWorkers);
  if (int64_t(desc->batch) * desc->num_kv_heads > kFusedMaxSeqs)
    return report_status(HPA_ERR_UNSUPPORTED, "batch x kv heads %lld > %d (allocation-free call)",
                         (long long)(int64_t(desc->batch) * desc->num_kv_heads), kFusedMaxSeqs);
  const size_t plan_al = (plan_bytes + 255) / 256 * 256;
  if (kAreaOffset + plan_al + partial_bytes > kScratchBytes)
    return report_status(HPA_ERR_UNSUPPORTED, "workspaces of %zu bytes exceed the %zu-byte scratch array",
                         plan_al + partial_bytes, kScratchBytes - kAreaOffset);
  if (desc->batch == 0) return HPA_OK;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return report_status(HPA_ERR_DEVICE, "hipGetDevice failed");
  unsigned char* base = nullptr;
  if ((st = scratch_of(device, stream, &base)) != HPA_OK) return st;
  int32_t* ctr = reinterpret_cast<int32_t*>(base + kHeadBytes);
  AttnRedirect r{device_error ? device_error : reinterpret_cast<int32_t*>(base), ctr,
                 ctr + (1 + kTailChunksPerWorker) * int64_t(kNoAllocMaxWorkers) + kFusedMaxSeqs};
  return decode_attn(desc, sched, q, k_cache, v_cache, k_scale, v_scale, seq_lens, page_table, W,
                     base + kAreaOffset, plan_bytes, base + kAreaOffset + plan_al, partial_bytes, out, 0, &r, stream);
}

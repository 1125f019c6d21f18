// Row-major KV pages -> the library's tiled page blocks.
//
// The pages say only that the cache is paged (openai-hub.com "腾讯混元HPC-Ops升级：
// 五大算子直击推理痛点", section "五大算子覆盖了哪些场景"); the common row-major page
// [num_pages, Hkv, 64 tokens, 128 dims] is what a caller's prefill or cache
// manager usually holds. hpa_kv_pack_pages turns such pages into the tiled
// blocks the attention kernel streams (k_block_index / v_block_index), so a
// caller can keep that layout upstream and pay one pass per page at write time.
//
// One workgroup per (page, KV head, K or V): 256 threads read the 64 x 128 block
// with 16-byte loads (row-major, so consecutive threads read consecutive bytes),
// scatter each element to its tiled position in LDS, and after one barrier write
// the block out with 16-byte stores. The whole block is in LDS before the first
// store, so a block may be converted in place.
#include "hpa_internal.hpp"

namespace hpa {
namespace {

constexpr int kPackThreads = 256;

typedef __attribute__((address_space(1))) int32_t gint32_t;

template <bool FP8>
__global__ __launch_bounds__(kPackThreads) void pack_pages_kernel(const uint8_t* k_rows, const uint8_t* v_rows,
                                                                  const int32_t* pages, int num_pages, int hkv,
                                                                  uint8_t* k_cache, uint8_t* v_cache,
                                                                  int32_t* err) {
  constexpr int EB = FP8 ? 1 : 2;                    // bytes per element
  constexpr int kBlockBytes = kBlockElems * EB;
  constexpr int kChunks = kBlockBytes / 16;          // 16-byte pieces of a block
  constexpr int kPer = kChunks / kPackThreads;       // per thread
  constexpr int kElemsPerChunk = 16 / EB;
  __shared__ __align__(16) uint8_t blk[kBlockBytes];
  const int64_t unit = blockIdx.x;                   // (i * hkv + g) * 2 + kv
  const bool is_v = unit & 1;
  const int64_t ig = unit >> 1;                      // i * hkv + g
  const int64_t i = ig / hkv;
  const int g = static_cast<int>(ig - i * hkv);
  const int p = pages ? pages[i] : static_cast<int>(i);
  if (p < 0 || p >= num_pages) {
    if (threadIdx.x == 0 && err)
      __hip_atomic_fetch_or((gint32_t*)err, HPA_DEVERR_PAGE_ID, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const uint8_t* src = (is_v ? v_rows : k_rows) + ig * kBlockBytes;
  uint8_t* dst = (is_v ? v_cache : k_cache) + (int64_t(p) * hkv + g) * kBlockBytes;
  uint4 in[kPer];
#pragma unroll
  for (int c = 0; c < kPer; ++c) in[c] = reinterpret_cast<const uint4*>(src)[c * kPackThreads + threadIdx.x];
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const int e0 = (c * kPackThreads + threadIdx.x) * kElemsPerChunk;   // first element, row-major
    const int t = e0 / kHeadDim, d0 = e0 % kHeadDim;
    const uint32_t w[4] = {in[c].x, in[c].y, in[c].z, in[c].w};
#pragma unroll
    for (int k = 0; k < kElemsPerChunk; ++k) {
      const int idx = is_v ? v_block_index(t, d0 + k, FP8) : k_block_index(t, d0 + k, FP8);
      if constexpr (FP8)
        blk[idx] = static_cast<uint8_t>(w[k / 4] >> (8 * (k % 4)));
      else
        reinterpret_cast<uint16_t*>(blk)[idx] = static_cast<uint16_t>(w[k / 2] >> (16 * (k % 2)));
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kPer; ++c)
    reinterpret_cast<uint4*>(dst)[c * kPackThreads + threadIdx.x] =
        reinterpret_cast<const uint4*>(blk)[c * kPackThreads + threadIdx.x];
}

}  // namespace
}  // namespace hpa

extern "C" hpa_status hpa_kv_pack_pages(const hpa_attn_desc* desc, const void* k_rows, const void* v_rows,
                                        const int32_t* pages, int32_t count, void* k_cache, void* v_cache,
                                        int32_t* device_error, hipStream_t stream) {
  using namespace hpa;
  if (!desc) return report_status(HPA_ERR_INVALID_ARG, "desc is NULL");
  if (desc->head_dim != kHeadDim || desc->page_size != kPage)
    return report_status(HPA_ERR_UNSUPPORTED, "head_dim %d / page_size %d (only 128 / 64)", desc->head_dim,
                         desc->page_size);
  if (desc->num_kv_heads < 1 || desc->num_pages < 0)
    return report_status(HPA_ERR_INVALID_ARG, "num_kv_heads %d, num_pages %d", desc->num_kv_heads, desc->num_pages);
  if (desc->kv_dtype != HPA_KV_BF16 && desc->kv_dtype != HPA_KV_FP8_E4M3)
    return report_status(HPA_ERR_INVALID_ARG, "kv_dtype %d", static_cast<int>(desc->kv_dtype));
  if (count < 0) return report_status(HPA_ERR_INVALID_ARG, "count %d < 0", count);
  if (!pages && count != desc->num_pages)
    return report_status(HPA_ERR_INVALID_ARG, "without a page list count (%d) must equal num_pages (%d)", count,
                         desc->num_pages);
  if (int64_t(count) * desc->num_kv_heads * 2 > INT32_MAX)
    return report_status(HPA_ERR_INVALID_ARG, "count x num_kv_heads too large");
  if (count == 0) return HPA_OK;
  if (!k_rows || !v_rows || !k_cache || !v_cache) return report_status(HPA_ERR_INVALID_ARG, "a pointer is NULL");
  for (const void* ptr : {k_rows, v_rows, static_cast<const void*>(k_cache), static_cast<const void*>(v_cache)})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return report_status(HPA_ERR_INVALID_ARG, "pointer not 16-byte aligned");
  if (pages && (k_rows == k_cache || v_rows == v_cache))
    return report_status(HPA_ERR_INVALID_ARG, "in-place packing needs pages == NULL (whole pool)");
  const dim3 grid(static_cast<unsigned>(int64_t(count) * desc->num_kv_heads * 2));
  const auto* kr = static_cast<const uint8_t*>(k_rows);
  const auto* vr = static_cast<const uint8_t*>(v_rows);
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  if (desc->kv_dtype == HPA_KV_FP8_E4M3)
    hipLaunchKernelGGL(pack_pages_kernel<true>, grid, dim3(kPackThreads), 0, stream, kr, vr, pages, desc->num_pages,
                       desc->num_kv_heads, kc, vc, device_error);
  else
    hipLaunchKernelGGL(pack_pages_kernel<false>, grid, dim3(kPackThreads), 0, stream, kr, vr, pages,
                       desc->num_pages, desc->num_kv_heads, kc, vc, device_error);
  if (hipGetLastError() != hipSuccess) return report_status(HPA_ERR_LAUNCH, "pack launch failed");
  return HPA_OK;
}

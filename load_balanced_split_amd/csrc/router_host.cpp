// C-ABI entry points of the split-precision router GEMM: validation, workspace
// size, launches (kernels in router.hip).
#include <cstdint>

#include "hpa_internal.hpp"      // hpa::report_status
#include "router_internal.hpp"

namespace {

hpa_status check_router_shape(int32_t tokens, int32_t experts, int32_t hidden) {
  if (tokens < 0 || tokens > hpa::kRouterMaxTokens)
    return hpa::report_status(HPA_ERR_INVALID_ARG, "tokens %d", tokens);
  if (experts < 16 || experts > hpa::kRouterMaxExperts || experts % 16 != 0)
    return hpa::report_status(HPA_ERR_UNSUPPORTED, "num_experts %d (a multiple of 16 up to %d)", experts,
                              hpa::kRouterMaxExperts);
  if (hidden < 32 || hidden > hpa::kRouterMaxHidden || hidden % 32 != 0)
    return hpa::report_status(HPA_ERR_UNSUPPORTED, "hidden %d (a multiple of 32 up to %d)", hidden,
                              hpa::kRouterMaxHidden);
  return HPA_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

extern "C" {

hpa_status hpa_router_pack_weights(const float* w, int32_t num_experts, int32_t hidden, void* packed,
                                   hipStream_t stream) {
  if (hpa_status st = check_router_shape(0, num_experts, hidden); st != HPA_OK) return st;
  if (!w || !packed) return hpa::report_status(HPA_ERR_INVALID_ARG, "w or packed is NULL");
  if (!aligned16(w) || !aligned16(packed))
    return hpa::report_status(HPA_ERR_INVALID_ARG, "w and packed must be 16-byte aligned");
  if (hpa::launch_router_pack(w, num_experts, hidden, static_cast<uint8_t*>(packed), stream) != hipSuccess)
    return hpa::report_status(HPA_ERR_LAUNCH, "router pack launch failed");
  return HPA_OK;
}

hpa_status hpa_router_workspace_size(int32_t tokens, int32_t num_experts, int32_t hidden, size_t* bytes) {
  if (!bytes) return hpa::report_status(HPA_ERR_INVALID_ARG, "bytes is NULL");
  if (hpa_status st = check_router_shape(tokens, num_experts, hidden); st != HPA_OK) return st;
  const hpa::RouterPlan p = hpa::RouterPlan::make(tokens, num_experts, hidden);
  *bytes = size_t(p.partial_slots) * size_t(tokens) * size_t(num_experts) * sizeof(float);
  return HPA_OK;
}

hpa_status hpa_router_gemm(const void* x, const void* packed, int32_t tokens, int32_t num_experts,
                           int32_t hidden, int32_t passes, float* logits, int32_t top_k, int32_t* topk_idx,
                           float* topk_val, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (hpa_status st = check_router_shape(tokens, num_experts, hidden); st != HPA_OK) return st;
  if (passes != 1 && passes != 2) return hpa::report_status(HPA_ERR_INVALID_ARG, "passes %d (1 or 2)", passes);
  if (top_k < 0 || top_k > std::min(hpa::kRouterMaxTopK, num_experts))
    return hpa::report_status(HPA_ERR_INVALID_ARG, "top_k %d (0 .. min(32, num_experts))", top_k);
  if (tokens == 0) return HPA_OK;
  if (!x || !packed || !logits || !workspace)
    return hpa::report_status(HPA_ERR_INVALID_ARG, "x, packed, logits or workspace is NULL");
  if (top_k > 0 && (!topk_idx || !topk_val))
    return hpa::report_status(HPA_ERR_INVALID_ARG, "topk_idx or topk_val is NULL");
  if (!aligned16(x) || !aligned16(packed) || !aligned16(workspace))
    return hpa::report_status(HPA_ERR_INVALID_ARG, "x, packed and workspace must be 16-byte aligned");
  size_t need = 0;
  hpa_router_workspace_size(tokens, num_experts, hidden, &need);
  if (workspace_bytes < need)
    return hpa::report_status(HPA_ERR_WORKSPACE, "router workspace %zu < %zu bytes", workspace_bytes, need);
  hpa::RouterArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.packed = static_cast<const uint8_t*>(packed);
  a.part = static_cast<float*>(workspace);
  a.logits = logits;
  a.topk_idx = topk_idx;
  a.topk_val = topk_val;
  a.T = tokens;
  a.E = num_experts;
  a.H = hidden;
  a.passes = passes;
  a.top_k = top_k;
  a.p = hpa::RouterPlan::make(tokens, num_experts, hidden);
  if (hpa::launch_router(a, stream) != hipSuccess) return hpa::report_status(HPA_ERR_LAUNCH, "router launch failed");
  return HPA_OK;
}

}  // extern "C"

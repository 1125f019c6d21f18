// Host side of libhpa: argument validation, workspace sizing, launches.
// Nothing here allocates device memory or synchronises (except the two
// documented calls); every launch goes to the caller's stream.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hpa_internal.hpp"

namespace {

thread_local std::string g_last_error;

hpa_status vfail(hpa_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_last_error = buf;
  return st;
}

hpa_status fail(hpa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hpa_status fail(hpa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  st = vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

hpa_status check_desc(const hpa_attn_desc* d) {
  if (!d) return fail(HPA_ERR_INVALID_ARG, "desc is NULL");
  if (d->head_dim != hpa::kHeadDim) return fail(HPA_ERR_UNSUPPORTED, "head_dim %d (only 128)", d->head_dim);
  if (d->page_size != hpa::kPage) return fail(HPA_ERR_UNSUPPORTED, "page_size %d (only 64)", d->page_size);
  if (d->batch < 0) return fail(HPA_ERR_INVALID_ARG, "batch %d < 0", d->batch);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(HPA_ERR_INVALID_ARG, "heads %d:%d", d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(HPA_ERR_INVALID_ARG, "num_q_heads %d not a multiple of num_kv_heads %d", d->num_q_heads,
                d->num_kv_heads);
  if (d->num_q_heads / d->num_kv_heads > hpa::kMaxGroup)
    return fail(HPA_ERR_UNSUPPORTED, "group size %d > 16", d->num_q_heads / d->num_kv_heads);
  if (hpa::kValuProducts && d->num_q_heads / d->num_kv_heads > hpa::kValuMaxGroup)
    return fail(HPA_ERR_UNSUPPORTED, "group size %d > %d (VALU-product build)", d->num_q_heads / d->num_kv_heads,
                hpa::kValuMaxGroup);
  if (d->max_pages_per_seq < 1) return fail(HPA_ERR_INVALID_ARG, "max_pages_per_seq %d < 1", d->max_pages_per_seq);
  if (int64_t(d->max_pages_per_seq) * hpa::kPage > INT32_MAX / 2)
    return fail(HPA_ERR_INVALID_ARG, "max_pages_per_seq %d too large", d->max_pages_per_seq);
  if (d->num_pages < 0) return fail(HPA_ERR_INVALID_ARG, "num_pages %d < 0", d->num_pages);
  if (int64_t(d->batch) * d->num_kv_heads > hpa::kMaxSeqs)
    return fail(HPA_ERR_INVALID_ARG, "batch x num_kv_heads %lld > %lld", (long long)(int64_t(d->batch) * d->num_kv_heads),
                (long long)hpa::kMaxSeqs);
  if (d->kv_dtype != HPA_KV_BF16 && d->kv_dtype != HPA_KV_FP8_E4M3)
    return fail(HPA_ERR_INVALID_ARG, "kv_dtype %d", static_cast<int>(d->kv_dtype));
  if (!(d->sm_scale > 0.f)) return fail(HPA_ERR_INVALID_ARG, "sm_scale must be > 0");
  return HPA_OK;
}

struct DeviceInfo {
  bool ready = false;
  int cus = 0;
  int per_cu = 0;          // persistent (balanced) attention workgroups per CU
  int per_cu_static = 0;   // static split-KV attention workgroups per CU
};
std::mutex g_dev_mu;
std::vector<DeviceInfo> g_dev;

bool is_static(hpa_sched s) { return s == HPA_SCHED_STATIC_SPLITS || s == HPA_SCHED_STATIC_CHUNK; }

// num_workers as given, or (0) the default of the schedule; sched < 0: the
// largest default over all schedules (workspace sizing).
hpa_status resolve_workers(int32_t requested, int sched, int32_t* out) {
  if (requested < 0) return fail(HPA_ERR_INVALID_ARG, "num_workers %d < 0", requested);
  if (requested > hpa::kMaxWorkers)
    return fail(HPA_ERR_INVALID_ARG, "num_workers %d > %lld", requested, (long long)hpa::kMaxWorkers);
  if (requested > 0) {
    *out = requested;
    return HPA_OK;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(HPA_ERR_DEVICE, "hipGetDevice failed");
  if (sched >= 0) return hpa_default_num_workers(dev, static_cast<hpa_sched>(sched), out);
  int32_t a = 0, b = 0;
  hpa_status st = hpa_default_num_workers(dev, HPA_SCHED_BALANCED, &a);
  if (st == HPA_OK) st = hpa_default_num_workers(dev, HPA_SCHED_STATIC_SPLITS, &b);
  *out = std::max(a, b);
  return st;
}

}  // namespace

namespace hpa {
hpa_status report_status(hpa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  st = vfail(st, fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace hpa

extern "C" {

const char* hpa_status_string(hpa_status s) {
  switch (s) {
    case HPA_OK: return "ok";
    case HPA_ERR_INVALID_ARG: return "invalid argument";
    case HPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case HPA_ERR_WORKSPACE: return "workspace too small";
    case HPA_ERR_DEVICE: return "HIP runtime error";
    case HPA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* hpa_last_error_message(void) { return g_last_error.c_str(); }

hpa_status hpa_default_num_workers(int device, hpa_sched sched, int32_t* num_workers) {
  if (!num_workers) return fail(HPA_ERR_INVALID_ARG, "num_workers is NULL");
  if (sched != HPA_SCHED_BALANCED && sched != HPA_SCHED_STATIC_SPLITS && sched != HPA_SCHED_STATIC_CHUNK &&
      sched != HPA_SCHED_BALANCED_FUSED && sched != HPA_SCHED_BALANCED_SINGLE)
    return fail(HPA_ERR_INVALID_ARG, "sched %d", static_cast<int>(sched));
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (device < 0) return fail(HPA_ERR_INVALID_ARG, "device %d", device);
  if (static_cast<size_t>(device) >= g_dev.size()) g_dev.resize(device + 1);
  DeviceInfo& di = g_dev[device];
  if (!di.ready) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(HPA_ERR_DEVICE, "hipGetDevice failed");
    if (hipSetDevice(device) != hipSuccess) return fail(HPA_ERR_DEVICE, "hipSetDevice(%d) failed", device);
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    const int per_cu = std::min(hpa::attn_blocks_per_cu(false), hpa::attn_blocks_per_cu(true));
    const int per_cu_static = std::min(hpa::attn_static_blocks_per_cu(false), hpa::attn_static_blocks_per_cu(true));
    (void)hipSetDevice(cur);
    if (e != hipSuccess || cus <= 0) return fail(HPA_ERR_DEVICE, "cannot read the CU count of device %d", device);
    di.cus = cus;
    di.per_cu = per_cu;
    di.per_cu_static = per_cu_static;
    di.ready = true;
  }
  *num_workers = di.cus * (is_static(sched) ? di.per_cu_static : di.per_cu);
  return HPA_OK;
}

hpa_status hpa_plan_workspace_layout(const hpa_attn_desc* desc, int32_t num_workers, hpa_plan_layout* layout) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  if (!layout) return fail(HPA_ERR_INVALID_ARG, "layout is NULL");
  int32_t W = 0;
  if ((st = resolve_workers(num_workers, -1, &W)) != HPA_OK) return st;
  const hpa::PlanOffsets o = hpa::plan_offsets(int64_t(desc->batch) * desc->num_kv_heads, W);
  layout->header = size_t(o.header) * 4;
  layout->C = size_t(o.C) * 4;
  layout->worker_off = size_t(o.worker_off) * 4;
  layout->item_s = size_t(o.item_s) * 4;
  layout->item_t0 = size_t(o.item_t0) * 4;
  layout->item_t1 = size_t(o.item_t1) * 4;
  layout->item_split = size_t(o.item_split) * 4;
  layout->item_slot = size_t(o.item_slot) * 4;
  layout->num_splits = size_t(o.num_splits) * 4;
  layout->partial_base = size_t(o.partial_base) * 4;
  layout->merge_list = size_t(o.merge_list) * 4;
  layout->total_bytes = size_t(o.total) * 4;
  layout->max_items = o.max_items;
  return HPA_OK;
}

hpa_status hpa_plan_workspace_size(const hpa_attn_desc* desc, int32_t num_workers, size_t* bytes) {
  if (!bytes) return fail(HPA_ERR_INVALID_ARG, "bytes is NULL");
  hpa_plan_layout l;
  hpa_status st = hpa_plan_workspace_layout(desc, num_workers, &l);
  if (st != HPA_OK) return st;
  *bytes = l.total_bytes;
  return HPA_OK;
}

hpa_status hpa_partial_workspace_size(const hpa_attn_desc* desc, int32_t num_workers, size_t* bytes) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  if (!bytes) return fail(HPA_ERR_INVALID_ARG, "bytes is NULL");
  int32_t W = 0;
  if ((st = resolve_workers(num_workers, -1, &W)) != HPA_OK) return st;
  const int64_t S = int64_t(desc->batch) * desc->num_kv_heads;
  *bytes = static_cast<size_t>(hpa::partial_layout(hpa::max_slots(W, S), desc->num_q_heads / desc->num_kv_heads).total_bytes +
                               hpa::trace_bytes(W + S));
  return HPA_OK;
}

hpa_status hpa_plan(const hpa_attn_desc* desc, const int32_t* seq_lens, int32_t num_workers,
                    int32_t min_tiles_per_worker, int32_t item_cost, int32_t tail_den, int32_t tail_chunk,
                    int32_t item_order, void* plan_ws, size_t plan_ws_bytes, hipStream_t stream) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  if (min_tiles_per_worker < 1) return fail(HPA_ERR_INVALID_ARG, "min_tiles_per_worker %d < 1", min_tiles_per_worker);
  if (item_cost < 0 || item_cost > 64) return fail(HPA_ERR_INVALID_ARG, "item_cost %d outside [0, 64]", item_cost);
  if (tail_den < 0) return fail(HPA_ERR_INVALID_ARG, "tail_den %d < 0", tail_den);
  if (tail_chunk < 1) return fail(HPA_ERR_INVALID_ARG, "tail_chunk %d < 1", tail_chunk);
  if (item_order < 0 || item_order > 2) return fail(HPA_ERR_INVALID_ARG, "item_order %d outside [0, 2]", item_order);
  if (!plan_ws) return fail(HPA_ERR_INVALID_ARG, "plan_ws is NULL");
  if (desc->batch > 0 && !seq_lens) return fail(HPA_ERR_INVALID_ARG, "seq_lens is NULL");
  int32_t W = 0;
  if ((st = resolve_workers(num_workers, HPA_SCHED_BALANCED, &W)) != HPA_OK) return st;
  const hpa::PlanOffsets o = hpa::plan_offsets(int64_t(desc->batch) * desc->num_kv_heads, W);
  if (plan_ws_bytes < size_t(o.total) * 4)
    return fail(HPA_ERR_WORKSPACE, "plan workspace %zu bytes < %lld", plan_ws_bytes, (long long)o.total * 4);
  if (hpa::launch_plan(seq_lens, desc->batch, desc->num_kv_heads, desc->max_pages_per_seq, W,
                       min_tiles_per_worker, item_cost, tail_den, tail_chunk, item_order,
                       static_cast<int32_t*>(plan_ws), o, stream) != hipSuccess)
    return fail(HPA_ERR_LAUNCH, "planner launch failed");
  return HPA_OK;
}

hpa_status hpa_decode_attn(const hpa_attn_desc* desc, hpa_sched sched, const void* q, const void* k_cache,
                           const void* v_cache, const float* k_scale, const float* v_scale,
                           const int32_t* seq_lens, const int32_t* page_table, int32_t num_workers,
                           void* plan_ws, size_t plan_ws_bytes, void* partial_ws, size_t partial_ws_bytes,
                           void* out, int32_t flags, hipStream_t stream) {
  return hpa::decode_attn(desc, sched, q, k_cache, v_cache, k_scale, v_scale, seq_lens, page_table, num_workers,
                          plan_ws, plan_ws_bytes, partial_ws, partial_ws_bytes, out, flags, nullptr, stream);
}

}  // extern "C"

namespace hpa {

hpa_status attn_workspace_bytes(const hpa_attn_desc* desc, hpa_sched sched, int32_t num_workers, int32_t* workers,
                                size_t* plan_bytes, size_t* partial_bytes) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  int32_t W = 0;
  if ((st = resolve_workers(num_workers, static_cast<int>(sched), &W)) != HPA_OK) return st;
  const int64_t S = int64_t(desc->batch) * desc->num_kv_heads;
  const int G = desc->num_q_heads / desc->num_kv_heads;
  *workers = W;
  *plan_bytes = size_t(plan_offsets(S, W).total) * 4;
  *partial_bytes = static_cast<size_t>(partial_layout(max_slots(W, S), G).total_bytes + trace_bytes(W + S));
  return HPA_OK;
}

hpa_status decode_attn(const hpa_attn_desc* desc, hpa_sched sched, const void* q, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                       const int32_t* page_table, int32_t num_workers, void* plan_ws, size_t plan_ws_bytes,
                       void* partial_ws, size_t partial_ws_bytes, void* out, int32_t flags,
                       const AttnRedirect* redirect, hipStream_t stream) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  if (sched != HPA_SCHED_BALANCED && sched != HPA_SCHED_STATIC_SPLITS && sched != HPA_SCHED_STATIC_CHUNK &&
      sched != HPA_SCHED_BALANCED_FUSED && sched != HPA_SCHED_BALANCED_SINGLE)
    return fail(HPA_ERR_INVALID_ARG, "sched %d", static_cast<int>(sched));

  if (flags & ~(HPA_ATTN_NO_MERGE | HPA_ATTN_MERGE_ONLY | HPA_ATTN_MERGE_IN_KERNEL) ||
      (flags & (HPA_ATTN_NO_MERGE | HPA_ATTN_MERGE_ONLY)) == (HPA_ATTN_NO_MERGE | HPA_ATTN_MERGE_ONLY) ||
      ((flags & HPA_ATTN_MERGE_IN_KERNEL) &&
       (sched != HPA_SCHED_BALANCED || (flags & (HPA_ATTN_NO_MERGE | HPA_ATTN_MERGE_ONLY)))))
    return fail(HPA_ERR_INVALID_ARG, "flags %d", flags);
  const bool in_kernel_merge = sched == HPA_SCHED_BALANCED_SINGLE || (flags & HPA_ATTN_MERGE_IN_KERNEL);
  if (desc->batch == 0) return HPA_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !page_table || !out || !partial_ws)
    return fail(HPA_ERR_INVALID_ARG, "a required pointer is NULL");
  const bool fp8 = desc->kv_dtype == HPA_KV_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return fail(HPA_ERR_INVALID_ARG, "E4M3 cache needs k_scale and v_scale");
  int32_t W = 0;
  if ((st = resolve_workers(num_workers, static_cast<int>(sched), &W)) != HPA_OK) return st;
  const int64_t S = int64_t(desc->batch) * desc->num_kv_heads;
  const int G = desc->num_q_heads / desc->num_kv_heads;
  const hpa::PartialLayout pl = hpa::partial_layout(hpa::max_slots(W, S), G);
  const int64_t need = pl.total_bytes + hpa::trace_bytes(W + S);
  if (partial_ws_bytes < static_cast<size_t>(need))
    return fail(HPA_ERR_WORKSPACE, "partial workspace %zu bytes < %lld", partial_ws_bytes, (long long)need);
  // the in-kernel merge addresses the partials through buffer resources with 32-bit
  // byte offsets
  if (in_kernel_merge && pl.l + hpa::max_slots(W, S) * G * 4 > int64_t(UINT32_MAX))
    return fail(HPA_ERR_UNSUPPORTED, "single-launch schedule: partial workspace of %lld bytes needs 32-bit offsets",
                (long long)pl.total_bytes);
  const hpa::PlanOffsets po = hpa::plan_offsets(S, W);
  if (sched == HPA_SCHED_BALANCED || sched == HPA_SCHED_BALANCED_FUSED || sched == HPA_SCHED_BALANCED_SINGLE) {
    if (!plan_ws) return fail(HPA_ERR_INVALID_ARG, "balanced schedules need plan_ws");
    if (plan_ws_bytes < size_t(po.total) * 4)
      return fail(HPA_ERR_WORKSPACE, "plan workspace %zu bytes < %lld", plan_ws_bytes, (long long)po.total * 4);
  } else if (plan_ws && plan_ws_bytes < size_t(po.total) * 4) {
    return fail(HPA_ERR_WORKSPACE, "plan workspace %zu bytes < %lld", plan_ws_bytes, (long long)po.total * 4);
  }

  hpa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint8_t*>(k_cache);
  a.v_cache = static_cast<const uint8_t*>(v_cache);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.plan = static_cast<int32_t*>(plan_ws);
  a.err = a.plan ? a.plan + po.header + hpa::H_ERR : nullptr;
  a.gctr = a.plan ? a.plan + po.gctr : nullptr;
  a.sctr = a.plan ? a.plan + po.sctr : nullptr;
  a.qctr = a.plan ? a.plan + po.qctr : nullptr;
  if (redirect) {
    a.err = redirect->err;
    a.gctr = redirect->gctr;
    a.sctr = redirect->sctr;
  }
  char* pw = static_cast<char*>(partial_ws);
  a.part_acc = reinterpret_cast<float*>(pw + pl.acc);
  a.part_m = reinterpret_cast<float*>(pw + pl.m);
  a.part_l = reinterpret_cast<float*>(pw + pl.l);
  a.trace = hpa::kTraceBuild ? reinterpret_cast<uint64_t*>(pw + pl.total_bytes) : nullptr;
  a.out = static_cast<uint16_t*>(out);
  a.po = po;
  a.batch = desc->batch;
  a.hq = desc->num_q_heads;
  a.hkv = desc->num_kv_heads;
  a.group = G;
  a.max_pages = desc->max_pages_per_seq;
  a.num_pages = desc->num_pages;
  a.sm_scale = desc->sm_scale;
  a.workers = W;
  a.slots = static_cast<int>(hpa::max_slots(W, S));

  const bool do_attn = !(flags & HPA_ATTN_MERGE_ONLY), do_merge = !(flags & HPA_ATTN_NO_MERGE);
  a.min_tiles = HPA_FUSED_MIN_TILES;
  a.item_cost = HPA_FUSED_ITEM_COST;
  a.tail_den = HPA_FUSED_TAIL_DEN;
  a.tail_chunk = HPA_FUSED_TAIL_CHUNK;
  if (sched == HPA_SCHED_BALANCED || sched == HPA_SCHED_BALANCED_FUSED || sched == HPA_SCHED_BALANCED_SINGLE) {
    // Batches of more than kFusedMaxSeqs sequences do not fit the fused kernels' LDS
    // plan: the planner kernel writes the same work list (the fused parameters) to
    // plan_ws first and the planned kernels run over it -- identical items, slots and
    // output bits, one launch more.
    const bool via_plan = sched != HPA_SCHED_BALANCED && S > hpa::kFusedMaxSeqs;
    if (via_plan && (sched == HPA_SCHED_BALANCED_SINGLE || do_attn) &&
        hpa::launch_plan(seq_lens, desc->batch, desc->num_kv_heads, desc->max_pages_per_seq, W, a.min_tiles,
                         a.item_cost, a.tail_den, a.tail_chunk, 0, a.plan, po, stream) != hipSuccess)
      return fail(HPA_ERR_LAUNCH, "planner launch failed");
    if (sched == HPA_SCHED_BALANCED_SINGLE) {
      // one launch (two above kFusedMaxSeqs): plan, attend and merge (flags have no effect)
      if ((via_plan ? hpa::launch_attn_balanced(a, fp8, true, W, stream)
                    : hpa::launch_attn_fused(a, fp8, true, W, stream)) != hipSuccess)
        return fail(HPA_ERR_LAUNCH, "attention launch failed");
      return HPA_OK;
    }
    if (sched == HPA_SCHED_BALANCED && in_kernel_merge) {   // the plan from hpa_plan, merged in-kernel
      if (hpa::launch_attn_balanced(a, fp8, true, W, stream) != hipSuccess)
        return fail(HPA_ERR_LAUNCH, "attention launch failed");
      return HPA_OK;
    }
    const bool fused = sched == HPA_SCHED_BALANCED_FUSED && !via_plan;
    if (do_attn && (fused ? hpa::launch_attn_fused(a, fp8, false, W, stream)
                          : hpa::launch_attn_balanced(a, fp8, false, W, stream)) != hipSuccess)
      return fail(HPA_ERR_LAUNCH, "attention launch failed");
    if (do_merge && hpa::launch_merge(a, fused ? hpa::MERGE_FUSED : hpa::MERGE_PLAN, stream) != hipSuccess)
      return fail(HPA_ERR_LAUNCH, "merge launch failed");
    return HPA_OK;
  }
  // static split-KV: S_split = clamp(ceil(W / S), 1, max_pages)
  const int64_t ss = std::max<int64_t>(1, std::min<int64_t>((W + S - 1) / S, desc->max_pages_per_seq));
  a.static_splits = static_cast<int>(ss);
  a.static_chunk = sched == HPA_SCHED_STATIC_CHUNK
                       ? static_cast<int>((desc->max_pages_per_seq + ss - 1) / ss) : 0;
  if (do_attn && hpa::launch_attn_static(a, fp8, stream) != hipSuccess)
    return fail(HPA_ERR_LAUNCH, "attention launch failed");
  if (do_merge && hpa::launch_merge(a, hpa::MERGE_STATIC, stream) != hipSuccess)
    return fail(HPA_ERR_LAUNCH, "merge launch failed");
  return HPA_OK;
}

}  // namespace hpa

extern "C" {

hpa_status hpa_decode_prologue(const hpa_attn_desc* desc, const void* q_in, const void* k_in, const void* v_in,
                               const float* q_norm_w, const float* k_norm_w, float eps, double rope_theta,
                               const int32_t* positions, const int32_t* page_table, void* k_cache,
                               void* v_cache, const float* k_scale, const float* v_scale, void* q_out,
                               int32_t* seq_lens_out, void* plan_ws, hipStream_t stream) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  if (desc->batch == 0) return HPA_OK;
  if (!q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !positions || !page_table || !k_cache || !v_cache ||
      !q_out || !seq_lens_out)
    return fail(HPA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (desc->kv_dtype == HPA_KV_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(HPA_ERR_INVALID_ARG, "E4M3 cache needs k_scale and v_scale");
  if (static_cast<const void*>(positions) == static_cast<const void*>(seq_lens_out))
    return fail(HPA_ERR_INVALID_ARG, "positions and seq_lens_out must not alias");
  if (!(eps >= 0.f) || !(rope_theta > 0.0)) return fail(HPA_ERR_INVALID_ARG, "eps < 0 or rope_theta <= 0");
  int32_t* err = plan_ws ? static_cast<int32_t*>(plan_ws) + hpa::H_ERR : nullptr;
  if (hpa::launch_prologue(*desc, static_cast<const uint16_t*>(q_in), static_cast<const uint16_t*>(k_in),
                           static_cast<const uint16_t*>(v_in), q_norm_w, k_norm_w, eps, rope_theta, positions,
                           page_table, static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale,
                           v_scale, static_cast<uint16_t*>(q_out), seq_lens_out, err, nullptr, stream) != hipSuccess)
    return fail(HPA_ERR_LAUNCH, "prologue launch failed");
  return HPA_OK;
}

hpa_status hpa_decode_prologue_plan(const hpa_attn_desc* desc, const void* q_in, const void* k_in,
                                    const void* v_in, const float* q_norm_w, const float* k_norm_w, float eps,
                                    double rope_theta, const int32_t* positions, const int32_t* page_table,
                                    void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                                    void* q_out, int32_t* seq_lens_out, int32_t num_workers,
                                    int32_t min_tiles_per_worker, int32_t item_cost, int32_t tail_den,
                                    int32_t tail_chunk, int32_t item_order, void* plan_ws, size_t plan_ws_bytes,
                                    hipStream_t stream) {
  hpa_status st = check_desc(desc);
  if (st != HPA_OK) return st;
  if (min_tiles_per_worker < 1) return fail(HPA_ERR_INVALID_ARG, "min_tiles_per_worker %d < 1", min_tiles_per_worker);
  if (item_cost < 0 || item_cost > 64) return fail(HPA_ERR_INVALID_ARG, "item_cost %d outside [0, 64]", item_cost);
  if (tail_den < 0) return fail(HPA_ERR_INVALID_ARG, "tail_den %d < 0", tail_den);
  if (tail_chunk < 1) return fail(HPA_ERR_INVALID_ARG, "tail_chunk %d < 1", tail_chunk);
  if (item_order < 0 || item_order > 2) return fail(HPA_ERR_INVALID_ARG, "item_order %d outside [0, 2]", item_order);
  if (!plan_ws) return fail(HPA_ERR_INVALID_ARG, "plan_ws is NULL");
  if (desc->batch == 0) return HPA_OK;
  if (!q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !positions || !page_table || !k_cache || !v_cache ||
      !q_out || !seq_lens_out)
    return fail(HPA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (desc->kv_dtype == HPA_KV_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(HPA_ERR_INVALID_ARG, "E4M3 cache needs k_scale and v_scale");
  if (static_cast<const void*>(positions) == static_cast<const void*>(seq_lens_out))
    return fail(HPA_ERR_INVALID_ARG, "positions and seq_lens_out must not alias");
  if (!(eps >= 0.f) || !(rope_theta > 0.0)) return fail(HPA_ERR_INVALID_ARG, "eps < 0 or rope_theta <= 0");
  int32_t W = 0;
  if ((st = resolve_workers(num_workers, HPA_SCHED_BALANCED, &W)) != HPA_OK) return st;
  const hpa::PlanOffsets o = hpa::plan_offsets(int64_t(desc->batch) * desc->num_kv_heads, W);
  if (plan_ws_bytes < size_t(o.total) * 4)
    return fail(HPA_ERR_WORKSPACE, "plan workspace %zu bytes < %lld", plan_ws_bytes, (long long)o.total * 4);
  int32_t* ws = static_cast<int32_t*>(plan_ws);
  const hpa::PlanArgs pa{ws, o, W, min_tiles_per_worker, item_cost, tail_den, tail_chunk, item_order};
  if (hpa::launch_prologue(*desc, static_cast<const uint16_t*>(q_in), static_cast<const uint16_t*>(k_in),
                           static_cast<const uint16_t*>(v_in), q_norm_w, k_norm_w, eps, rope_theta, positions,
                           page_table, static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale,
                           v_scale, static_cast<uint16_t*>(q_out), seq_lens_out, ws + o.header + hpa::H_ERR, &pa,
                           stream) != hipSuccess)
    return fail(HPA_ERR_LAUNCH, "prologue launch failed");
  return HPA_OK;
}

hpa_status hpa_read_device_error(void* plan_ws, int32_t* code, int32_t clear, hipStream_t stream) {
  if (!plan_ws || !code) return fail(HPA_ERR_INVALID_ARG, "plan_ws or code is NULL");
  int32_t* word = static_cast<int32_t*>(plan_ws) + hpa::H_ERR;
  if (hipMemcpyAsync(code, word, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return fail(HPA_ERR_DEVICE, "reading the error word failed");
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(HPA_ERR_DEVICE, "stream synchronise failed");
  if (clear) {
    if (hpa::launch_clear_word(word, stream) != hipSuccess) return fail(HPA_ERR_LAUNCH, "clear launch failed");
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(HPA_ERR_DEVICE, "stream synchronise failed");
  }
  return HPA_OK;
}

hpa_status hpa_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups, int32_t* sink,
                                 hipStream_t stream) {
  if (!buf || !sink) return fail(HPA_ERR_INVALID_ARG, "buf or sink is NULL");
  if (bytes == 0 || bytes % 16 != 0) return fail(HPA_ERR_INVALID_ARG, "bytes %zu not a positive multiple of 16", bytes);
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(HPA_ERR_INVALID_ARG, "buf not 16-byte aligned");
  if (workgroups < 0 || workgroups > (1 << 20)) return fail(HPA_ERR_INVALID_ARG, "workgroups %d", workgroups);
  if (workgroups == 0) {
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      return fail(HPA_ERR_DEVICE, "compute unit count query failed");
    workgroups = 4 * cus;
  }
  if (hpa::launch_stream_read(buf, bytes, workgroups, sink, stream) != hipSuccess)
    return fail(HPA_ERR_LAUNCH, "stream-read probe launch failed");
  return HPA_OK;
}

}  // extern "C"

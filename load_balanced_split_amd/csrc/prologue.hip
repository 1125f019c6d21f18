// Fused decode prologue: q/k RMSNorm, rotate-half RoPE, KV quantise and paged append.
//
// bitbyai.com "vLLM × HPC-Ops: High-Performance Attention and MoE Backends from
// Tencent Hunyuan", section "Breaking Down the Kernels": RoPE, query-key
// normalisation and the KV write run as one prologue ahead of attention, to
// save launches and HBM round trips.
//
// One workgroup per request; each wave takes whole head rows (Hq query rows,
// Hkv key rows, Hkv value rows). Lane i owns the rotation pair (i, i + 64).
// With PLAN, workgroup 0 runs the balanced planner (plan_block.hpp) over the
// lengths after this launch's appends while workgroups 1..B append; it starts
// first because it runs longest.
// RMSNorm (Zhang & Sennrich 2019): y = x / sqrt(mean(x^2) + eps) * w, fp32.
// RoPE (Su et al. 2021, rotate-half form): angle_i = pos * theta^(-i/64) is
// formed and reduced modulo 2*pi in fp64 (positions reach 131072, where an fp32
// angle would be off by ~0.016 rad); sine, cosine and the rotation are fp32.
#include "plan_block.hpp"

#include <cmath>

namespace hpa {
namespace {

constexpr int kProThreads = 256;

__device__ inline float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// fp32 -> OCP E4M3, round to nearest even, saturating at 448, NaN -> 0x7f.
__device__ inline uint8_t f32_to_e4m3(float x) {
  if (x != x) return 0x7f;
  const uint8_t sign = __builtin_signbit(x) ? 0x80 : 0x00;
  float a = fminf(fabsf(x), 448.0f);
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9 (codes 0..8)
    const int q = static_cast<int>(rintf(a * 512.0f));
    return sign | static_cast<uint8_t>(q);
  }
  int e;
  frexpf(a, &e);                             // a = f * 2^e, f in [0.5, 1)
  int E = e - 1;                             // a in [2^E, 2^(E+1))
  int qm = static_cast<int>(rintf(ldexpf(a, 3 - E)));   // in [8, 16]
  if (qm == 16) {
    qm = 8;
    ++E;
  }
  return sign | static_cast<uint8_t>(((E + 7) << 3) | (qm - 8));
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Rows of one request a wave handles per pass (loads of a pass are issued before
// any of its arithmetic, so a pass costs one memory round trip).
constexpr int kProRowsPerPass = 4;

// Request b's live length once this launch's append is done: position + 1 when
// the append is valid (the prologue writes exactly that to seq_lens_out), else the
// unchanged seq_lens_out[b] (no workgroup writes it then) -- so the plan equals
// hpa_plan over seq_lens_out bit for bit.
struct LensAfterAppend {
  const int32_t* positions;
  const int32_t* page_table;
  const int32_t* seq_lens_out;
  int max_pages, num_pages;
  __device__ int operator()(int b) const {
    const int pos = positions[b];
    int pid = -1;
    if (pos >= 0 && pos < max_pages * kPage) pid = page_table[int64_t(b) * max_pages + pos / kPage];
    return (pid >= 0 && pid < num_pages) ? pos + 1 : seq_lens_out[b];
  }
};

template <bool PLAN>
__global__ __launch_bounds__(kProThreads) void prologue_kernel(
    const uint16_t* __restrict__ q_in, const uint16_t* __restrict__ k_in,
    const uint16_t* __restrict__ v_in, const float* __restrict__ q_norm_w,
    const float* __restrict__ k_norm_w, float eps, double rope_theta,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ page_table,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, uint16_t* __restrict__ q_out, int32_t* __restrict__ seq_lens_out,
    int32_t* err_word, int hq, int hkv, int max_pages, int num_pages, int fp8, PlanArgs pa) {
  if constexpr (PLAN) {
    if (blockIdx.x == 0) {
      plan_block<kProThreads, true>(LensAfterAppend{positions, page_table, seq_lens_out, max_pages, num_pages},
                                    static_cast<int>(gridDim.x) - 1, hkv, max_pages, pa.workers, pa.min_tiles,
                                    pa.item_cost, pa.tail_den, pa.tail_chunk, pa.order, pa.ws, pa.po);
      return;
    }
  }
  const int b = static_cast<int>(blockIdx.x) - (PLAN ? 1 : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kProWaves = kProThreads / 64;
  const int rows = hq + 2 * hkv;
  // rows base + wave + kProWaves * i of a pass, zero past the last row
  auto load_pass = [&](int base, float (&x0)[kProRowsPerPass], float (&x1)[kProRowsPerPass]) {
#pragma unroll
    for (int i = 0; i < kProRowsPerPass; ++i) {
      const int r = base + wave + kProWaves * i;
      x0[i] = x1[i] = 0.f;
      if (r < rows) {
        const uint16_t* src = r < hq ? q_in + (int64_t(b) * hq + r) * kHeadDim
                            : r < hq + hkv ? k_in + (int64_t(b) * hkv + (r - hq)) * kHeadDim
                                           : v_in + (int64_t(b) * hkv + (r - hq - hkv)) * kHeadDim;
        x0[i] = bf16_to_f32(src[lane]);
        x1[i] = bf16_to_f32(src[lane + 64]);
      }
    }
  };
  // everything that does not depend on the position goes out first
  const int pos = positions[b];
  const float wq0 = q_norm_w[lane], wq1 = q_norm_w[lane + 64];
  const float wk0 = k_norm_w[lane], wk1 = k_norm_w[lane + 64];
  float x0[kProRowsPerPass], x1[kProRowsPerPass];
  load_pass(0, x0, x1);
  int pid = -1;
  if (pos >= 0 && pos < max_pages * kPage) pid = page_table[int64_t(b) * max_pages + pos / kPage];
  if (pid < 0 || pid >= num_pages) {
    if (threadIdx.x == 0 && err_word) atomicOr(err_word, HPA_DEVERR_PROLOGUE);
    return;
  }
  if (threadIdx.x == 0) seq_lens_out[b] = pos + 1;
  const int slot = pos % kPage;

  // rotation of pair (lane, lane + 64): the angle is formed and reduced mod 2 pi in
  // fp64; its sine and cosine are then taken in fp32 on the reduced angle
  const double two_pi = 6.283185307179586476925286766559;
  const double ang = static_cast<double>(pos) * pow(rope_theta, -static_cast<double>(lane) / 64.0);
  const float red = static_cast<float>(ang - two_pi * rint(ang / two_pi));
  float sn, cs;
  sincosf(red, &sn, &cs);

  for (int base = 0; base < rows; base += kProWaves * kProRowsPerPass) {
    if (base > 0) load_pass(base, x0, x1);
#pragma unroll
    for (int i = 0; i < kProRowsPerPass; ++i) {
      const int r = base + wave + kProWaves * i;
      if (r >= rows) break;                   // uniform per wave
      if (r < hq + hkv) {
        const bool is_q = r < hq;
        const float ms = wave_sum(x0[i] * x0[i] + x1[i] * x1[i]) * (1.0f / kHeadDim);
        const float inv = 1.0f / sqrtf(ms + eps);
        const float y0 = x0[i] * inv * (is_q ? wq0 : wk0), y1 = x1[i] * inv * (is_q ? wq1 : wk1);
        const float o0 = y0 * cs - y1 * sn, o1 = y1 * cs + y0 * sn;
        if (is_q) {
          uint16_t* dst = q_out + (int64_t(b) * hq + r) * kHeadDim;
          dst[lane] = f32_to_bf16(o0);
          dst[lane + 64] = f32_to_bf16(o1);
        } else {
          const int g = r - hq;
          const int64_t blk = (int64_t(pid) * hkv + g) * kBlockElems;
          const int64_t i0 = blk + k_block_index(slot, lane, fp8), i1 = blk + k_block_index(slot, lane + 64, fp8);
          if (fp8) {
            const float sc = k_scale[g];
            k_cache[i0] = f32_to_e4m3(o0 / sc);
            k_cache[i1] = f32_to_e4m3(o1 / sc);
          } else {
            uint16_t* kc = reinterpret_cast<uint16_t*>(k_cache);
            kc[i0] = f32_to_bf16(o0);
            kc[i1] = f32_to_bf16(o1);
          }
        }
      } else {
        const int g = r - hq - hkv;
        const int64_t blk = (int64_t(pid) * hkv + g) * kBlockElems;
        const int64_t i0 = blk + v_block_index(slot, lane, fp8), i1 = blk + v_block_index(slot, lane + 64, fp8);
        if (fp8) {
          const float sc = v_scale[g];
          v_cache[i0] = f32_to_e4m3(x0[i] / sc);
          v_cache[i1] = f32_to_e4m3(x1[i] / sc);
        } else {
          uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache);
          vc[i0] = f32_to_bf16(x0[i]);
          vc[i1] = f32_to_bf16(x1[i]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_prologue(const hpa_attn_desc& d, const uint16_t* q_in, const uint16_t* k_in,
                           const uint16_t* v_in, const float* q_norm_w, const float* k_norm_w,
                           float eps, double rope_theta, const int32_t* positions,
                           const int32_t* page_table, uint8_t* k_cache, uint8_t* v_cache,
                           const float* k_scale, const float* v_scale, uint16_t* q_out,
                           int32_t* seq_lens_out, int32_t* err_word, const PlanArgs* plan, hipStream_t stream) {
  if (d.batch == 0) return hipSuccess;
  const int fp8 = d.kv_dtype == HPA_KV_FP8_E4M3 ? 1 : 0;
  const bool together = plan && int64_t(d.batch) * d.num_kv_heads <= kPlanLdsSeqs;
  if (together) {
    hipLaunchKernelGGL(prologue_kernel<true>, dim3(d.batch + 1), dim3(kProThreads), 0, stream, q_in, k_in, v_in,
                       q_norm_w, k_norm_w, eps, rope_theta, positions, page_table, k_cache, v_cache, k_scale,
                       v_scale, q_out, seq_lens_out, err_word, d.num_q_heads, d.num_kv_heads, d.max_pages_per_seq,
                       d.num_pages, fp8, *plan);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(prologue_kernel<false>, dim3(d.batch), dim3(kProThreads), 0, stream, q_in, k_in, v_in,
                     q_norm_w, k_norm_w, eps, rope_theta, positions, page_table, k_cache, v_cache, k_scale,
                     v_scale, q_out, seq_lens_out, err_word, d.num_q_heads, d.num_kv_heads, d.max_pages_per_seq,
                     d.num_pages, fp8, PlanArgs{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !plan) return e;
  // batches too large for the planner's LDS arrays: plan after the appends instead
  return launch_plan(seq_lens_out, d.batch, d.num_kv_heads, d.max_pages_per_seq, plan->workers, plan->min_tiles,
                     plan->item_cost, plan->tail_den, plan->tail_chunk, plan->order, plan->ws, plan->po, stream);
}

}  // namespace hpa

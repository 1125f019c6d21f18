// Fused FP8 mixture-of-experts layer for decode batches, gfx950.
//
// xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section "为什么 batch 越大，
// 数字越漂亮" (the MoE paragraph): at small decode batches each expert gets few
// tokens, so routing, token movement, intermediate tensors and launches cost more
// than the matrix products; the routing index, Gate-Up, activation with
// requantisation, Down GEMM and the top-k merge run as one chain with no
// standalone gather. bitbyai.com "vLLM × HPC-Ops …", section "Breaking Down the
// Kernels" (MoE backend): token rearrangement, FP8 expert GEMMs, activation and
// result gathering fused to avoid intermediate HBM round trips and launches.
//
// Three launches, no gather, no sort:
//  moe_gate_up_kernel  workgroup (expert e, block of 16 of its pairs, 64 of I): finds
//      its pairs by scanning the routing ids (pairs p = t K + k with ids[p] == e, in
//      p order), reads the tokens' bf16 rows by index and quantises them to E4M3 in
//      LDS (scale amax / 448 per token), multiplies with 64 gate and 64 up rows of W1
//      on v_mfma_f32_16x16x128_f8f6f4, and in the epilogue applies the per-channel
//      scales and SwiGLU; it writes the fp32 activation slice and the slice's amax.
//  moe_down_kernel     workgroup (expert e, block of 16 pairs, 64 of H): requantises
//      its pairs' activations to E4M3 as they come into LDS (scale = the row amax /
//      448, the amax taken over the slices' maxima), multiplies with 64 rows of W2
//      and writes y * scale * routing weight per pair.
//  moe_merge_kernel    out[t] = sum over k, in k order, of the pair results -> bf16.
//
// Both products: A = weight rows (16 per wave), B = quantised activations of 16
// pairs (LDS); per 128-wide k chunk a lane holds 32 consecutive bytes of its row
// (16-byte loads, whole 128-byte lines of each weight row) and one MFMA consumes
// them. A and B use the same lane -> k assignment, so the product is the plain
// sum over k. Weight bytes are read once per (expert, pair block) from HBM with
// the streaming policy.
#include "hpa_internal.hpp"
#include "moe_internal.hpp"

#include <cmath>

namespace hpa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kMoeThreads = 256;
constexpr int kPairsPerBlock = 16;
constexpr int kLdsPad = 16;          // bytes after every LDS row: 16-byte reads of 16 rows hit distinct banks
constexpr int kBufDword3 = 0x00020000;
constexpr int kPolicyStream = 2;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kBufDword3);
}

__device__ inline u32x4 wload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), kPolicyStream);
}

// fp32 -> OCP E4M3 code: nearest value, ties to even mantissa, saturating at 448.
__device__ inline uint32_t e4m3_code(float x) {
  const uint32_t sign = __builtin_signbit(x) ? 0x80u : 0u;
  const float a = fminf(fabsf(x), 448.0f);
  if (a < 0.015625f) return sign | static_cast<uint32_t>(rintf(a * 512.0f));   // subnormals, 2^-9 steps
  int e;
  frexpf(a, &e);                               // a = f 2^e, f in [0.5, 1)
  int E = e - 1;
  int qm = static_cast<int>(rintf(ldexpf(a, 3 - E)));   // 8 .. 16
  if (qm == 16) {
    qm = 8;
    ++E;
  }
  return sign | static_cast<uint32_t>(((E + 7) << 3) | (qm - 8));
}

// 32 bytes of E4M3 codes (two 16-byte pieces) as one operand of the 16x16x128 product:
// format 0 (E4M3) for both operands, no block scale (scale operands 0: the unscaled
// instruction).
__device__ inline i32x8 operand(u32x4 lo, u32x4 hi) {
  return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// The pairs of expert e with rank [16 pb, 16 pb + 16) among its pairs (in pair order),
// found by wave 0 scanning the routing ids; returns how many (<= 0: none).
__device__ int find_pairs(const MoeArgs& a, int e, int pb, int* pairs, int* count) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const int lo = kPairsPerBlock * pb, hi = lo + kPairsPerBlock;
    int found = 0;
    for (int base = 0; base < a.P && found < hi; base += 64 * 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = base + 64 * j + lane;
        v[j] = p < a.P ? a.ids[p] : -1;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool hit = v[j] == e;
        const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
        const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
        const int idx = found + below;
        if (hit && idx >= lo && idx < hi) pairs[idx - lo] = base + 64 * j + lane;
        found += __builtin_popcountll(m);
      }
    }
    if (lane == 0) *count = min(kPairsPerBlock, found - lo);
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*count);
}

// Gate-Up + SwiGLU. Grid: experts x pair blocks x I / 64.
__global__ __launch_bounds__(kMoeThreads) void moe_gate_up_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // [16][H + pad] E4M3 codes
  __shared__ int pairs[kPairsPerBlock];
  __shared__ int count;
  __shared__ float sx[kPairsPerBlock];
  __shared__ float wmax[4][kPairsPerBlock];
  const int it = blockIdx.x % a.IT, rest = blockIdx.x / a.IT;
  const int pb0 = rest % a.PB, e = rest / a.PB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int rs = a.H + kLdsPad;
  // pair chunks pb0, pb0 + PB, ...: with distinct experts per token an expert has at
  // most T pairs and the first chunk is the only one; repeated ids take more turns
  for (int pb = pb0;; pb += a.PB) {
    const int n = find_pairs(a, e, pb, pairs, &count);
    if (n <= 0) return;
    // the tokens' rows, quantised: wave w takes rows w, w + 4, ...; lane l holds 16-byte
    // pieces l, l + 64, ... of the row (8 bf16 each)
    const int pieces = a.H / 8;
    for (int r = wave; r < kPairsPerBlock; r += 4) {
      uint8_t* dst = xs + r * rs;
      if (r >= n) {                                   // padding rows multiply as zeros
        for (int c = lane; c < pieces; c += 64) *reinterpret_cast<uint2*>(dst + 8 * c) = make_uint2(0, 0);
        if (lane == 0) sx[r] = 0.f;
        continue;
      }
      const int t = pairs[r] / a.K;
      const uint16_t* row = a.x + int64_t(t) * a.H;
      u32x4 v[kMoeMaxHidden / 512];
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < kMoeMaxHidden / 512; ++j)
        if (j * 64 + lane < pieces) v[j] = *reinterpret_cast<const u32x4*>(row + 8 * (j * 64 + lane));
#pragma unroll
      for (int j = 0; j < kMoeMaxHidden / 512; ++j) {
        if (j * 64 + lane >= pieces) continue;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v[j][d] << 16)));
          amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v[j][d] & 0xffff0000u)));
        }
      }
      amax = wave_max(amax);
      const float s = amax / 448.0f;
      if (lane == 0) sx[r] = s;
#pragma unroll
      for (int j = 0; j < kMoeMaxHidden / 512; ++j) {
        if (j * 64 + lane >= pieces) continue;
        uint32_t w[2] = {0, 0};
        if (s > 0.f) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float lo = __builtin_bit_cast(float, v[j][d] << 16);
            const float hi = __builtin_bit_cast(float, v[j][d] & 0xffff0000u);
            w[d / 2] |= (e4m3_code(lo / s) | (e4m3_code(hi / s) << 8)) << (16 * (d % 2));
          }
        }
        *reinterpret_cast<uint2*>(dst + 8 * (j * 64 + lane)) = make_uint2(w[0], w[1]);
      }
    }
    __syncthreads();
    // 16 gate rows and the matching 16 up rows per wave; lane (m, q) holds row m's bytes
    // [128 c + 32 q, + 32) of every chunk c
    const int m16 = lane & 15, q = lane >> 4;
    const int g0 = it * 64 + 16 * wave;                      // first gate row of this wave (< I)
    const int nch = a.H / 128;
    const uint8_t* w1e = a.w1 + int64_t(e) * 2 * a.I * a.H;
    const rsrc_t rw = make_rsrc(w1e, static_cast<uint32_t>(int64_t(2) * a.I * a.H));
    const uint32_t og = static_cast<uint32_t>((g0 + m16) * a.H + 32 * q);
    const uint32_t ou = static_cast<uint32_t>((a.I + g0 + m16) * a.H + 32 * q);
    f32x4 accg = f32x4{0.f, 0.f, 0.f, 0.f}, accu = accg;
    constexpr int kDepth = 4;
    u32x4 ag[kDepth][2], au[kDepth][2];
    auto load = [&](int slot, int c) {
      const uint32_t sc = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(128 * c));
      ag[slot][0] = wload16(rw, og, sc);
      ag[slot][1] = wload16(rw, og + 16, sc);
      au[slot][0] = wload16(rw, ou, sc);
      au[slot][1] = wload16(rw, ou + 16, sc);
    };
    // chunk c lives in ring slot c % kDepth; slots are compile-time (the loop is unrolled
    // by kDepth), and the loads of chunk c + kDepth - 1 go out before chunk c is used
    auto mul = [&](int slot, int c) {
      const uint8_t* brow = xs + m16 * rs + 128 * c + 32 * q;
      const i32x8 B = operand(*reinterpret_cast<const u32x4*>(brow), *reinterpret_cast<const u32x4*>(brow + 16));
      accg = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(ag[slot][0], ag[slot][1]), B, accg,
                                                              0, 0, 0, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(au[slot][0], au[slot][1]), B, accu,
                                                              0, 0, 0, 0, 0, 0);
    };
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) load(d, min(d, nch - 1));
    int c = 0;
    for (; c + kDepth <= nch; c += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load((d + kDepth - 1) % kDepth, min(c + d + kDepth - 1, nch - 1));
        mul(d, c + d);
      }
    }
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      if (c + d < nch) mul(d, c + d);
    // epilogue: lane (m16, q) holds gate / up rows g0 + 4 q + i (i < 4) of pair slot m16
    const float* s1e = a.s1 + int64_t(e) * 2 * a.I;
    const f32x4 sg = *reinterpret_cast<const f32x4*>(s1e + g0 + 4 * q);
    const f32x4 su = *reinterpret_cast<const f32x4*>(s1e + a.I + g0 + 4 * q);
    const float sxm = sx[m16];
    f32x4 act;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = accg[i] * sxm * sg[i];
      const float u = accu[i] * sxm * su[i];
      act[i] = g / (1.0f + expf(-g)) * u;
      amax = fmaxf(amax, fabsf(act[i]));
    }
    const bool valid = m16 < n;
    const int p = valid ? pairs[m16] : 0;
    if (valid) *reinterpret_cast<f32x4*>(a.act + int64_t(p) * a.I + g0 + 4 * q) = act;
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (q == 0) wmax[wave][m16] = amax;
    __syncthreads();
    if (threadIdx.x < n) {
      const int r = threadIdx.x;
      const float mx = fmaxf(fmaxf(wmax[0][r], wmax[1][r]), fmaxf(wmax[2][r], wmax[3][r]));
      a.amax[int64_t(pairs[r]) * a.IT + it] = mx;
    }
    __syncthreads();                  // pairs, sx, wmax and the LDS rows are rewritten next turn
  }
}

// Down + scales + routing weight. Grid: experts x pair blocks x H / 64.
__global__ __launch_bounds__(kMoeThreads) void moe_down_kernel(MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t as8[];   // [16][I + pad] E4M3 codes
  __shared__ int pairs[kPairsPerBlock];
  __shared__ int count;
  __shared__ float sa[kPairsPerBlock];
  const int ht = blockIdx.x % a.HT, rest = blockIdx.x / a.HT;
  const int pb0 = rest % a.PB, e = rest / a.PB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int rs = a.I + kLdsPad;
  for (int pb = pb0;; pb += a.PB) {   // pair chunks as in the Gate-Up kernel
    const int n = find_pairs(a, e, pb, pairs, &count);
    if (n <= 0) return;
    // activation rows, requantised: lane l holds 4-float pieces l, l + 64, ...
    const int pieces = a.I / 4;
    for (int r = wave; r < kPairsPerBlock; r += 4) {
      uint8_t* dst = as8 + r * rs;
      if (r >= n) {
        for (int c = lane; c < pieces; c += 64) *reinterpret_cast<uint32_t*>(dst + 4 * c) = 0;
        continue;
      }
      const int p = pairs[r];
      float amax = 0.f;
      for (int j = lane; j < a.IT; j += 64) amax = fmaxf(amax, a.amax[int64_t(p) * a.IT + j]);
      amax = wave_max(amax);
      const float s = amax / 448.0f;
      if (lane == 0) sa[r] = s;
      const float* row = a.act + int64_t(p) * a.I;
      f32x4 v[kMoeMaxInter / 256];
#pragma unroll
      for (int j = 0; j < kMoeMaxInter / 256; ++j)
        if (j * 64 + lane < pieces) v[j] = *reinterpret_cast<const f32x4*>(row + 4 * (j * 64 + lane));
#pragma unroll
      for (int j = 0; j < kMoeMaxInter / 256; ++j) {
        if (j * 64 + lane >= pieces) continue;
        uint32_t w = 0;
        if (s > 0.f) {
#pragma unroll
          for (int d = 0; d < 4; ++d) w |= e4m3_code(v[j][d] / s) << (8 * d);
        }
        *reinterpret_cast<uint32_t*>(dst + 4 * (j * 64 + lane)) = w;
      }
    }
    __syncthreads();
    const int m16 = lane & 15, q = lane >> 4;
    const int n0 = ht * 64 + 16 * wave;                       // first output row of this wave (< H)
    const int nch = a.I / 128;
    const uint8_t* w2e = a.w2 + int64_t(e) * a.H * a.I;
    const rsrc_t rw = make_rsrc(w2e, static_cast<uint32_t>(int64_t(a.H) * a.I));
    const uint32_t ow = static_cast<uint32_t>((n0 + m16) * a.I + 32 * q);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kDepth = 4;
    u32x4 aw[kDepth][2];
    auto load = [&](int slot, int c) {
      const uint32_t sc = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(128 * c));
      aw[slot][0] = wload16(rw, ow, sc);
      aw[slot][1] = wload16(rw, ow + 16, sc);
    };
    auto mul = [&](int slot, int c) {
      const uint8_t* brow = as8 + m16 * rs + 128 * c + 32 * q;
      const i32x8 B = operand(*reinterpret_cast<const u32x4*>(brow), *reinterpret_cast<const u32x4*>(brow + 16));
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(aw[slot][0], aw[slot][1]), B, acc,
                                                             0, 0, 0, 0, 0, 0);
    };
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) load(d, min(d, nch - 1));
    int c = 0;
    for (; c + kDepth <= nch; c += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load((d + kDepth - 1) % kDepth, min(c + d + kDepth - 1, nch - 1));
        mul(d, c + d);
      }
    }
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      if (c + d < nch) mul(d, c + d);
    if (m16 < n) {
      const int p = pairs[m16];
      const f32x4 s2 = *reinterpret_cast<const f32x4*>(a.s2 + int64_t(e) * a.H + n0 + 4 * q);
      const float f = sa[m16] * a.wts[p];
      f32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = acc[i] * f * s2[i];
      *reinterpret_cast<f32x4*>(a.ybuf + int64_t(p) * a.H + n0 + 4 * q) = y;
    }
    __syncthreads();                  // pairs, sa and the LDS rows are rewritten next turn
  }
}

// out[t][n .. n + 3] = bf16 of the sum over k (in k order) of the pair results; pairs
// whose expert id is outside [0, E) add nothing (and report an error).
__global__ __launch_bounds__(kMoeThreads) void moe_merge_kernel(MoeArgs a) {
  const int t = blockIdx.y;
  const int nq = blockIdx.x * kMoeThreads + threadIdx.x;     // 4-dim piece
  if (4 * nq >= a.H) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int k = 0; k < a.K; ++k) {
    const int p = t * a.K + k;
    const int e = a.ids[p];
    if (e < 0 || e >= a.E) {
      bad = true;
      continue;
    }
    s += *reinterpret_cast<const f32x4*>(a.ybuf + int64_t(p) * a.H + 4 * nq);
  }
  uint2 o;
  o.x = f32_to_bf16(s[0]) | (uint32_t(f32_to_bf16(s[1])) << 16);
  o.y = f32_to_bf16(s[2]) | (uint32_t(f32_to_bf16(s[3])) << 16);
  *reinterpret_cast<uint2*>(a.out + int64_t(t) * a.H + 4 * nq) = o;
  if (bad && nq == 0 && a.err)
    __hip_atomic_fetch_or(a.err, HPA_DEVERR_MOE_EXPERT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hpa_status moe_check_shape(int32_t tokens, int32_t experts, int32_t top_k, int32_t hidden, int32_t inter) {
  if (tokens < 0 || tokens > kMoeMaxTokens) return report_status(HPA_ERR_UNSUPPORTED, "tokens %d (0 .. %d)", tokens,
                                                                kMoeMaxTokens);
  if (experts < 1 || experts > kMoeMaxExperts)
    return report_status(HPA_ERR_UNSUPPORTED, "experts %d (1 .. %d)", experts, kMoeMaxExperts);
  if (top_k < 1 || top_k > kMoeMaxTopK) return report_status(HPA_ERR_UNSUPPORTED, "top_k %d (1 .. %d)", top_k,
                                                              kMoeMaxTopK);
  if (hidden < 128 || hidden > kMoeMaxHidden || hidden % 128 != 0)
    return report_status(HPA_ERR_UNSUPPORTED, "hidden %d (a multiple of 128 up to %d)", hidden, kMoeMaxHidden);
  if (inter < 128 || inter > kMoeMaxInter || inter % 128 != 0)
    return report_status(HPA_ERR_UNSUPPORTED, "inter %d (a multiple of 128 up to %d)", inter, kMoeMaxInter);
  if (int64_t(tokens) * top_k > kMoeMaxPairs)
    return report_status(HPA_ERR_UNSUPPORTED, "tokens x top_k %lld > %d", (long long)(int64_t(tokens) * top_k),
                         kMoeMaxPairs);
  return HPA_OK;
}

hipError_t launch_moe(const MoeArgs& a, hipStream_t stream) {
  const size_t lds1 = size_t(kPairsPerBlock) * (a.H + kLdsPad);
  const size_t lds2 = size_t(kPairsPerBlock) * (a.I + kLdsPad);
  // rows of up to 4096 bytes take just over 64 KB of LDS: raise the kernels' limit once
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_gate_up_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_down_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(moe_gate_up_kernel, dim3(static_cast<unsigned>(int64_t(a.E) * a.PB * a.IT)), dim3(kMoeThreads),
                     lds1, stream, a);
  hipLaunchKernelGGL(moe_down_kernel, dim3(static_cast<unsigned>(int64_t(a.E) * a.PB * a.HT)), dim3(kMoeThreads), lds2,
                     stream, a);
  hipLaunchKernelGGL(moe_merge_kernel, dim3((a.H / 4 + kMoeThreads - 1) / kMoeThreads, a.T), dim3(kMoeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace hpa

extern "C" hpa_status hpa_moe_workspace_size(int32_t tokens, int32_t top_k, int32_t hidden, int32_t inter,
                                             size_t* bytes) {
  using namespace hpa;
  if (!bytes) return report_status(HPA_ERR_INVALID_ARG, "bytes is NULL");
  if (hpa_status st = moe_check_shape(tokens, 1, top_k, hidden, inter); st != HPA_OK) return st;
  *bytes = moe_workspace(tokens, top_k, hidden, inter).total;
  return HPA_OK;
}

extern "C" hpa_status hpa_moe_fused(const void* x, const int32_t* topk_ids, const float* topk_weights, const void* w1,
                                    const float* s1, const void* w2, const float* s2, int32_t tokens, int32_t experts,
                                    int32_t top_k, int32_t hidden, int32_t inter, void* out, void* workspace,
                                    size_t workspace_bytes, int32_t* device_error, hipStream_t stream) {
  using namespace hpa;
  if (hpa_status st = moe_check_shape(tokens, experts, top_k, hidden, inter); st != HPA_OK) return st;
  if (tokens == 0) return HPA_OK;
  if (!x || !topk_ids || !topk_weights || !w1 || !s1 || !w2 || !s2 || !out || !workspace)
    return report_status(HPA_ERR_INVALID_ARG, "a required pointer is NULL");
  for (const void* p : {x, static_cast<const void*>(w1), static_cast<const void*>(w2), static_cast<const void*>(s1),
                        static_cast<const void*>(s2), static_cast<const void*>(out), static_cast<const void*>(workspace)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return report_status(HPA_ERR_INVALID_ARG, "pointer not 16-byte aligned");
  const MoeWorkspace ws = moe_workspace(tokens, top_k, hidden, inter);
  if (workspace_bytes < ws.total)
    return report_status(HPA_ERR_WORKSPACE, "MoE workspace %zu bytes < %zu", workspace_bytes, ws.total);
  MoeArgs a{};
  char* wb = static_cast<char*>(workspace);
  a.x = static_cast<const uint16_t*>(x);
  a.ids = topk_ids;
  a.wts = topk_weights;
  a.w1 = static_cast<const uint8_t*>(w1);
  a.s1 = s1;
  a.w2 = static_cast<const uint8_t*>(w2);
  a.s2 = s2;
  a.act = reinterpret_cast<float*>(wb + ws.act);
  a.amax = reinterpret_cast<float*>(wb + ws.amax);
  a.ybuf = reinterpret_cast<float*>(wb + ws.ybuf);
  a.out = static_cast<uint16_t*>(out);
  a.err = device_error;
  a.T = tokens;
  a.E = experts;
  a.K = top_k;
  a.H = hidden;
  a.I = inter;
  a.P = tokens * top_k;
  a.PB = (tokens + 15) / 16;
  a.IT = inter / 64;
  a.HT = hidden / 64;
  if (launch_moe(a, stream) != hipSuccess) return report_status(HPA_ERR_LAUNCH, "MoE launch failed");
  return HPA_OK;
}

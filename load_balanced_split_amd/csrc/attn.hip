// Split-KV decode attention over a paged KV cache, for gfx950.
//
// Balanced schedule (xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
// "为什么 batch 越大，数字越漂亮"): persistent workgroups walk the work list the
// planner made from 64-token tiles of the live lengths. Static schedule (same
// section: a fixed split count, or a fixed split size sized for the longest
// request): one workgroup per (sequence, split). Both share the per-item code,
// so a comparison isolates scheduling. Split sequences are combined by the
// merge kernel with a log-sum-exp rescale (the only exact way to combine
// softmax over disjoint token ranges).
//
// Per workgroup: 4 waves on one item; wave w takes the item's units w, w+4, ...
// A unit is 32 tokens for bf16 KV and 64 tokens (a whole page) for E4M3 KV, i.e.
// 16 KB of K+V either way, loaded straight into the registers MFMA reads
// (16-byte loads, one unit prefetched while the previous one is computed).
//   scores  S^T[tok x head] = K[tok x 32 dims] * Q^T[32 dims x head]  (16x16x32, 4 k-chunks)
//   output  O^T[dim x head] += V^T[dim x 32 tok] * P^T[32 tok x head] (16x16x32)
// The 8 query heads of a KV head fill half of the 16-wide N side. The V page is
// stored dim-major so the MFMA A operand (8 consecutive tokens of one dim) is a
// single 16-byte load. Rows of K are assigned to MFMA rows so that the score
// registers a lane holds after Q*K^T are exactly the tokens it feeds into P*V.
#include "hpa_internal.hpp"

#include <cmath>

namespace hpa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kORow = kHeadDim + 4;     // padded LDS row of the combine buffers

template <bool FP8>
struct Cfg {
  static constexpr int UNIT = FP8 ? 64 : 32;   // tokens per unit
  static constexpr int UPT = kPage / UNIT;      // units per tile
  static constexpr int NBLK = UNIT / 16;        // 16-token MFMA row blocks
  static constexpr int KSTEPS = UNIT / 32;      // 32-token PV k-steps
  static constexpr int TS = UNIT / 4;           // tokens per lane group
  static constexpr int EB = FP8 ? 1 : 2;        // bytes per element
};

// Token (within the unit) held by MFMA row m of score block b.
template <bool FP8>
__device__ inline int row_token(int b, int m) {
  return Cfg<FP8>::TS * (m >> 2) + 8 * (b >> 1) + 4 * (b & 1) + (m & 3);
}

// First of the 8 head dims lane group j feeds into k-chunk c of Q*K^T.
template <bool FP8>
__device__ inline int chunk_dim(int c, int j) {
  return FP8 ? 64 * (c >> 1) + 16 * j + 8 * (c & 1) : 32 * c + 8 * j;
}

__device__ inline u32x4 load16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Uniform base + 32-bit lane offset (lets the compiler use the SGPR-base form).
__device__ inline u32x4 load16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact: every E4M3 value is a bf16 value).
__device__ inline bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

struct UnitBuf {
  u32x4 k[8];
  u32x4 v[8];
};

struct Item {
  int s, t0, t1, slot;
};

// Shared state of the 4 waves for the end-of-item combine.
struct CombineLds {
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  float o[kWaves][kMaxGroup][kORow];
};

template <bool FP8>
struct ItemRunner {
  const AttnArgs& a;
  CombineLds& lds;
  int lane, wave, m16, j;

  __device__ ItemRunner(const AttnArgs& args, CombineLds& l)
      : a(args), lds(l), lane(threadIdx.x & 63), wave(threadIdx.x >> 6), m16(threadIdx.x & 15),
        j((threadIdx.x & 63) >> 4) {}

  // Issue the 16 loads of one unit: tokens [half * UNIT, half * UNIT + UNIT) of page
  // `pid`, KV head g. Page bases are wave-uniform; per-lane offsets are 32-bit.
  __device__ void issue(UnitBuf& buf, int pid, int g, int half) {
    using C = Cfg<FP8>;
    constexpr uint32_t page_bytes = kPage * kHeadDim * C::EB;
    const uint8_t* kp = a.k_cache + (uint64_t(pid) * a.hkv + g) * page_bytes;
    const uint8_t* vp = a.v_cache + (uint64_t(pid) * a.hkv + g) * page_bytes;
    const uint32_t tb = half * C::UNIT;
    // K rows: block b adds 4*b tokens to block 0's row (row_token), chunk c adds dims
    const uint32_t koff = ((tb + row_token<FP8>(0, m16)) * kHeadDim + chunk_dim<FP8>(0, j)) * C::EB;
    if constexpr (!FP8) {
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          buf.k[b * 4 + c] = load16(kp + (4 * b * kHeadDim + 32 * c) * 2, koff);
    } else {
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          buf.k[b * 2 + p] = load16(kp + 4 * b * kHeadDim + 64 * p, koff);
    }
    // V^T rows: dim 16n + m16, tokens tb + TS*j .. +16 bytes
    const uint32_t voff = (m16 * kPage + tb + C::TS * j) * C::EB;
#pragma unroll
    for (int n = 0; n < 8; ++n) buf.v[n] = load16(vp + 16 * n * kPage * C::EB, voff);
  }

  __device__ inline bf16x8 k_operand(const UnitBuf& buf, int b, int c) const {
    if constexpr (!FP8) {
      return as_bf16x8(buf.k[b * 4 + c]);
    } else {
      const u32x4 w = buf.k[b * 2 + (c >> 1)];
      return (c & 1) ? e4m3x8_to_bf16(w[2], w[3]) : e4m3x8_to_bf16(w[0], w[1]);
    }
  }

  __device__ inline bf16x8 v_operand(const UnitBuf& buf, int n, int ks) const {
    if constexpr (!FP8) {
      return as_bf16x8(buf.v[n]);
    } else {
      const u32x4 w = buf.v[n];
      return ks ? e4m3x8_to_bf16(w[2], w[3]) : e4m3x8_to_bf16(w[0], w[1]);
    }
  }

  // Online-softmax update with one unit: tokens [tok0, tok0 + UNIT) of the sequence.
  __device__ void compute(const UnitBuf& buf, const bf16x8 (&q)[4], int tok0, int L, float qk_scale,
                          float& m_run, float& l_part, f32x4 (&o)[8]) {
    using C = Cfg<FP8>;
    f32x4 sc[C::NBLK];
#pragma unroll
    for (int b = 0; b < C::NBLK; ++b) {
      sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(buf, b, c), q[c], sc[b], 0, 0, 0);
    }
    const bool partial = tok0 + C::UNIT > L;
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < C::NBLK; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = sc[b][i] * qk_scale;
        if (partial && tok0 + row_token<FP8>(b, 4 * j + i) >= L) s = -INFINITY;
        sc[b][i] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < C::NBLK; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[b][i] - m_new);
        sc[b][i] = p;
        psum += p;
      }
    }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] *= alpha;
    bf16x8 pk[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pk[ks][i] = static_cast<__bf16>(sc[2 * ks][i]);
        pk[ks][4 + i] = static_cast<__bf16>(sc[2 * ks + 1][i]);
      }
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        bf16x8 vop = v_operand(buf, n, ks);
        if (partial) {
          // padding rows may hold anything (NaN included): zero them, never multiply
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (tok0 + C::TS * j + 8 * ks + e >= L) vop[e] = static_cast<__bf16>(0.f);
        }
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pk[ks], o[n], 0, 0, 0);
      }
    }
  }

  __device__ int load_pid(int b, int tile) const { return a.page_table[int64_t(b) * a.max_pages + tile]; }

  __device__ bool bad_pid(int pid) const { return pid < 0 || pid >= a.num_pages; }

  // One item: all 4 waves; ends with the combine and the output / partial write.
  __device__ void run(const Item it) {
    using C = Cfg<FP8>;
    const int b = it.s / a.hkv, g = it.s - b * a.hkv;
    const int L = a.seq_lens[b];
    // units: UPT per tile, minus a trailing half-tile that starts past L
    int nu = (it.t1 - it.t0) * C::UPT;
    if (C::UPT > 1 && it.t1 * kPage - C::UNIT >= L) nu -= 1;
    const float qk_scale = a.sm_scale * kLog2e * (FP8 ? a.k_scale[g] : 1.f);

    // Q^T operand: lane holds head m16, dims chunk_dim(c, j) .. +8
    bf16x8 q[4];
    const int h = g * a.group + m16;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (m16 < a.group)
        v = load16(reinterpret_cast<const uint8_t*>(a.q + (int64_t(b) * a.hq + h) * kHeadDim +
                                                    chunk_dim<FP8>(c, j)));
      q[c] = as_bf16x8(v);
    }

    float m_run = -INFINITY, l_part = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    int u = wave;
    if (u < nu) {
      UnitBuf bufA, bufB;
      bool badA = false, badB = false, any_bad = false;
      // page id of the unit after the one being issued (tile t0 stands in past the end)
      int pid_next = load_pid(b, u + kWaves < nu ? it.t0 + (u + kWaves) / C::UPT : it.t0);
      {
        int pid = __builtin_amdgcn_readfirstlane(load_pid(b, it.t0 + u / C::UPT));
        badA = bad_pid(pid);
        any_bad |= badA;
        issue(bufA, badA ? 0 : pid, g, u % C::UPT);
      }
      for (;;) {
        // prefetch unit u+4 into B while A is consumed
        const int uB = u + kWaves;
        if (uB < nu) {
          int pid = __builtin_amdgcn_readfirstlane(pid_next);
          const int un = uB + kWaves;
          pid_next = load_pid(b, un < nu ? it.t0 + un / C::UPT : it.t0);
          badB = bad_pid(pid);
          any_bad |= badB;
          issue(bufB, badB ? 0 : pid, g, uB % C::UPT);
        }
        if (!badA) compute(bufA, q, (it.t0 + u / C::UPT) * kPage + (u % C::UPT) * C::UNIT, L, qk_scale, m_run, l_part, o);
        if (uB >= nu) break;
        const int uA = uB + kWaves;
        if (uA < nu) {
          int pid = __builtin_amdgcn_readfirstlane(pid_next);
          const int un = uA + kWaves;
          pid_next = load_pid(b, un < nu ? it.t0 + un / C::UPT : it.t0);
          badA = bad_pid(pid);
          any_bad |= badA;
          issue(bufA, badA ? 0 : pid, g, uA % C::UPT);
        }
        if (!badB) compute(bufB, q, (it.t0 + uB / C::UPT) * kPage + (uB % C::UPT) * C::UNIT, L, qk_scale, m_run, l_part, o);
        if (uA >= nu) break;
        u = uA;
      }
      if (any_bad && lane == 0 && a.plan) atomicOr(&a.plan[a.po.header + H_ERR], HPA_DEVERR_PAGE_ID);
    }

    // wave state -> LDS: l summed over the 4 lane groups
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (m16 < a.group) {
      if (j == 0) {
        lds.m[wave][m16] = m_run;
        lds.l[wave][m16] = l_tot;
      }
#pragma unroll
      for (int n = 0; n < 8; ++n)
        *reinterpret_cast<f32x4*>(&lds.o[wave][m16][16 * n + 4 * j]) = o[n];
    }
    __syncthreads();

    // combine the 4 waves; write the output row or a partial slot
    const float vscale = FP8 ? a.v_scale[g] : 1.f;
    for (int idx = threadIdx.x; idx < a.group * kHeadDim; idx += kAttnThreads) {
      const int hh = idx >> 7, d = idx & (kHeadDim - 1);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds.m[w][hh]);
      float Ls = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(lds.m[w][hh] - M);   // 0 for idle waves
        Ls += f * lds.l[w][hh];
        acc += f * lds.o[w][hh][d];
      }
      acc *= vscale;
      if (it.slot < 0) {
        a.out[(int64_t(b) * a.hq + g * a.group + hh) * kHeadDim + d] = f32_to_bf16_rne(acc / Ls);
      } else {
        const int64_t sl = it.slot;
        a.part_acc[(sl * a.group + hh) * kHeadDim + d] = acc;
        if (d == 0) {
          a.part_m[sl * a.group + hh] = M;
          a.part_l[sl * a.group + hh] = Ls;
        }
      }
    }
    __syncthreads();
  }
};

template <bool FP8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_balanced_kernel(AttnArgs a) {
  __shared__ CombineLds lds;
  const int32_t* hdr = a.plan + a.po.header;
  const int w = blockIdx.x;
  if (hdr[H_W] != static_cast<int>(gridDim.x)) {
    if (w == 0 && threadIdx.x == 0) atomicOr(&a.plan[a.po.header + H_ERR], HPA_DEVERR_PLAN);
    return;
  }
  if (w >= hdr[H_WP]) return;
  const int i0 = a.plan[a.po.worker_off + w], i1 = a.plan[a.po.worker_off + w + 1];
  ItemRunner<FP8> r(a, lds);
  const int S = a.batch * a.hkv;
  for (int i = i0; i < i1; ++i) {
    Item it{a.plan[a.po.item_s + i], a.plan[a.po.item_t0 + i], a.plan[a.po.item_t1 + i],
            a.plan[a.po.item_slot + i]};
    // a work list that does not fit this launch is reported, never followed
    if (it.s < 0 || it.s >= S || it.t0 < 0 || it.t1 <= it.t0 || it.t1 > a.max_pages || it.slot >= a.slots) {
      if (threadIdx.x == 0) atomicOr(&a.plan[a.po.header + H_ERR], HPA_DEVERR_PLAN);
      continue;
    }
    r.run(it);
  }
}

// Static split-KV: block (s, k) handles chunk k of sequence s.
template <bool FP8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_static_kernel(AttnArgs a) {
  __shared__ CombineLds lds;
  const int s = blockIdx.x / a.static_splits, k = blockIdx.x - s * a.static_splits;
  const int b = s / a.hkv;
  int L = a.seq_lens[b];
  if (L < 0 || L > a.max_pages * kPage) {
    if (k == 0 && threadIdx.x == 0 && a.plan) atomicOr(&a.plan[a.po.header + H_ERR], HPA_DEVERR_SEQ_LEN);
    return;
  }
  const int n = (L + kPage - 1) / kPage;
  if (n == 0) return;
  const int chunk = a.static_chunk > 0 ? a.static_chunk : (n + a.static_splits - 1) / a.static_splits;
  const int t0 = k * chunk, t1 = min(n, t0 + chunk);
  if (t0 >= t1) return;
  const int nchunks = (n + chunk - 1) / chunk;
  ItemRunner<FP8> r(a, lds);
  r.run(Item{s, t0, t1, nchunks > 1 ? s * a.static_splits + k : -1});
}

// Merge: block (i, h) combines head h of the i-th sequence to merge. 512 threads =
// 32 dim-quads x 16 split-groups. Empty sequences get a zero row.
constexpr int kMergeThreads = 512;
constexpr int kMergeGroups = kMergeThreads / 32;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnArgs a, int balanced) {
  __shared__ float red[kMergeThreads / 64];
  __shared__ f32x4 part[kMergeGroups][32];
  const int hh = blockIdx.y;
  int s, n, base;
  if (balanced) {
    const int32_t* hdr = a.plan + a.po.header;
    if (hdr[H_W] != a.workers || static_cast<int>(blockIdx.x) >= hdr[H_NMERGE]) return;
    s = a.plan[a.po.merge_list + blockIdx.x];
    if (s < 0 || s >= a.batch * a.hkv) return;
    n = a.plan[a.po.num_splits + s];
    base = a.plan[a.po.partial_base + s];
    if (n < 0 || base < 0 || base + n > a.slots) return;
  } else {
    s = blockIdx.x;
    const int L = a.seq_lens[s / a.hkv];
    if (L < 0 || L > a.max_pages * kPage) return;
    const int nt = (L + kPage - 1) / kPage;
    const int chunk = nt == 0 ? 1 : (a.static_chunk > 0 ? a.static_chunk : (nt + a.static_splits - 1) / a.static_splits);
    n = (nt + chunk - 1) / chunk;
    if (n == 1) return;
    base = s * a.static_splits;
  }
  const int b = s / a.hkv, g = s - b * a.hkv;
  uint16_t* orow = a.out + (int64_t(b) * a.hq + g * a.group + hh) * kHeadDim;
  const int tid = threadIdx.x, q4 = tid & 31, kg = tid >> 5;
  if (n == 0) {
    if (tid < kHeadDim) orow[tid] = 0;
    return;
  }
  // M = max_k m_k
  float mx = -INFINITY;
  for (int k = tid; k < n; k += kMergeThreads) mx = fmaxf(mx, a.part_m[int64_t(base + k) * a.group + hh]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  // Lsum = sum_k l_k 2^(m_k - M)
  float ls = 0.f;
  for (int k = tid; k < n; k += kMergeThreads) {
    const int64_t i = int64_t(base + k) * a.group + hh;
    ls += a.part_l[i] * __builtin_amdgcn_exp2f(a.part_m[i] - M);
  }
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ls;
  __syncthreads();
  float Ls = 0.f;
  for (int w = 0; w < kMergeThreads / 64; ++w) Ls += red[w];
  // acc over splits k = kg, kg + 16, ... for dims 4*q4 .. +3
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kg; k < n; k += kMergeGroups) {
    const int64_t i = int64_t(base + k) * a.group + hh;
    const float f = __builtin_amdgcn_exp2f(a.part_m[i] - M);
    acc += f * *reinterpret_cast<const f32x4*>(a.part_acc + i * kHeadDim + 4 * q4);
  }
  part[kg][q4] = acc;
  __syncthreads();
  if (kg == 0) {
    f32x4 t = part[0][q4];
    for (int k = 1; k < kMergeGroups; ++k) t += part[k][q4];
    const float inv = 1.f / Ls;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[4 * q4 + e] = f32_to_bf16_rne(t[e] * inv);
  }
}

}  // namespace

int attn_blocks_per_cu(bool fp8) {
  int nb = 0;
  hipError_t e = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_balanced_kernel<true>, kAttnThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_balanced_kernel<false>, kAttnThreads, 0);
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

hipError_t launch_attn_balanced(const AttnArgs& a, bool fp8, int num_workers, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL(attn_balanced_kernel<true>, dim3(num_workers), dim3(kAttnThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_balanced_kernel<false>, dim3(num_workers), dim3(kAttnThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_static(const AttnArgs& a, bool fp8, hipStream_t stream) {
  const int64_t grid = int64_t(a.batch) * a.hkv * a.static_splits;
  if (grid == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL(attn_static_kernel<true>, dim3(grid), dim3(kAttnThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_static_kernel<false>, dim3(grid), dim3(kAttnThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, bool balanced, hipStream_t stream) {
  const int S = a.batch * a.hkv;
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(S, a.group), dim3(kMergeThreads), 0, stream, a, balanced ? 1 : 0);
  return hipGetLastError();
}

}  // namespace hpa

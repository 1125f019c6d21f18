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

// Raw buffer resources (gfx9 dword3: 32-bit data format). A load whose offset is
// past num_records returns zeros without touching memory, which turns "no such
// unit" and "bad page" into ordinary straight-line loads.
constexpr int kBufDword3 = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufDword3);
}

__device__ inline u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

__device__ inline int bload_i32(rsrc_t r, uint32_t soff) {
  return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(r, 0, static_cast<int>(soff), 0));
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

// Per-wave record of the instrumented build, written by lane 0 when the wave ends.
struct WaveTrace {
  uint64_t* rec;
  uint64_t t0;
  uint32_t units = 0;
  __device__ explicit WaveTrace(const AttnArgs& a) {
    rec = (kTraceBuild && a.trace) ? a.trace + (uint64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * kTraceWords
                                   : nullptr;
    t0 = kTraceBuild ? __builtin_amdgcn_s_memrealtime() : 0;
  }
  __device__ ~WaveTrace() {
    if (kTraceBuild && rec && (threadIdx.x & 63) == 0) {
      const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
      const uint64_t hw = static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 4));   // HW_ID
      const uint64_t xcc = static_cast<uint32_t>(__builtin_amdgcn_s_getreg((15 << 11) | 20)); // XCC_ID
      rec[0] = t0;
      rec[1] = t1;
      rec[2] = hw | (xcc << 32);
      rec[3] = units;
    }
  }
};

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
  uint32_t units_done = 0;
  int lane, wave, m16, j;
  uint32_t koff, voff;   // per-lane byte offsets of a unit's K rows and V^T rows

  __device__ ItemRunner(const AttnArgs& args, CombineLds& l)
      : a(args), lds(l), lane(threadIdx.x & 63),
        wave(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6))),
        m16(threadIdx.x & 15), j((threadIdx.x & 63) >> 4) {
    using C = Cfg<FP8>;
    koff = (row_token<FP8>(0, m16) * kHeadDim + chunk_dim<FP8>(0, j)) * C::EB;
    voff = (m16 * kPage + C::TS * j) * C::EB;
  }

  // Issue the 16 loads of one unit: tokens [half * UNIT, half * UNIT + UNIT) of one
  // (page, KV head). rk / rv cover that page's K and V (num_records 0 when the
  // unit does not exist or its page id is bad: the loads then return zeros).
  // Lane offsets are fixed for the kernel; the unit offset goes into soffset.
  __device__ void issue(UnitBuf& buf, rsrc_t rk, rsrc_t rv, int half) const {
    using C = Cfg<FP8>;
    const uint32_t tb = half * C::UNIT;
    const uint32_t ks = tb * kHeadDim * C::EB;
    if constexpr (!FP8) {
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          buf.k[b * 4 + c] = bload16(rk, koff + (4 * b * kHeadDim + 32 * c) * 2, ks);
    } else {
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          buf.k[b * 2 + p] = bload16(rk, koff + 4 * b * kHeadDim + 64 * p, ks);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) buf.v[n] = bload16(rv, voff, (16 * n * kPage + tb) * C::EB);
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
  __device__ void compute(UnitBuf& buf, const bf16x8 (&q)[4], int tok0, int L, float qk_scale,
                          float& m_run, float& l_part, f32x4 (&o)[8]) {
    using C = Cfg<FP8>;
    if (kTraceBuild) ++units_done;
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
    if (partial) {
      // padding rows may hold anything (NaN included): zero their V bytes, never multiply.
      // Lane group j holds tokens TS*j .. TS*j + TS-1 of the unit in each V register.
      const int nvalid = L - tok0 - C::TS * j;     // tokens of this lane's run that are live
#pragma unroll
      for (int n = 0; n < 8; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dword e holds tokens [e * 4 / EB, (e + 1) * 4 / EB) of the run
          constexpr int per = 4 / C::EB;
          const int first = e * per;
          uint32_t keep = 0;
          if (nvalid >= first + per) keep = 0xffffffffu;
          else if (nvalid > first) keep = (1u << (8 * C::EB * (nvalid - first))) - 1u;
          buf.v[n][e] &= keep;
        }
      }
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_operand(buf, n, ks), pk[ks], o[n], 0, 0, 0);
    }
  }

  __device__ bool bad_pid(int pid) const { return pid < 0 || pid >= a.num_pages; }

  // One item: all 4 waves; ends with the combine and the output / partial write.
  __device__ void run(const Item it) {
    using C = Cfg<FP8>;
    constexpr uint32_t page_bytes = kPage * kHeadDim * C::EB;
    const int b = it.s / a.hkv, g = it.s - b * a.hkv;
    const int L = a.seq_lens[b];
    // units: UPT per tile, minus a trailing half-tile that starts past L
    int nu = (it.t1 - it.t0) * C::UPT;
    if (C::UPT > 1 && it.t1 * kPage - C::UNIT >= L) nu -= 1;
    const float qk_scale = a.sm_scale * kLog2e * (FP8 ? a.k_scale[g] : 1.f);

    // Q^T operand: lane holds head m16, dims chunk_dim(c, j) .. +8 (zeros for heads >= G)
    const rsrc_t rq = make_rsrc(a.q + (int64_t(b) * a.hq + g * a.group) * kHeadDim,
                                a.group * kHeadDim * 2);
    bf16x8 q[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) q[c] = as_bf16x8(bload16(rq, (m16 * kHeadDim + chunk_dim<FP8>(c, j)) * 2, 0));

    float m_run = -INFINITY, l_part = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // page ids come through a buffer resource too (vector loads, ordered with the data)
    const rsrc_t rpt = make_rsrc(a.page_table + int64_t(b) * a.max_pages, a.max_pages * 4);
    const uint8_t* kbase = a.k_cache + uint64_t(g) * page_bytes;
    const uint8_t* vbase = a.v_cache + uint64_t(g) * page_bytes;
    const uint64_t pstride = uint64_t(a.hkv) * page_bytes;
    auto tile_of = [&](int u) { return it.t0 + (u < nu ? u : 0) / C::UPT; };
    // unit u -> resources (empty when u is past the item or its page id is bad)
    auto unit_rsrc = [&](int u, int pid_raw, rsrc_t& rk, rsrc_t& rv) -> bool {
      const int pid = __builtin_amdgcn_readfirstlane(pid_raw);
      const bool ok = u < nu && !bad_pid(pid);
      const uint64_t off = ok ? uint64_t(pid) * pstride : 0;
      rk = make_rsrc(kbase + off, ok ? page_bytes : 0);
      rv = make_rsrc(vbase + off, ok ? page_bytes : 0);
      return ok;
    };

    const int u0 = wave;
    bool any_bad = false;
    if (u0 < nu) {
      UnitBuf bufA, bufB;
      rsrc_t rk, rv;
      int pidA = bload_i32(rpt, tile_of(u0) * 4);
      int pidB = bload_i32(rpt, tile_of(u0 + kWaves) * 4);
      bool okA = unit_rsrc(u0, pidA, rk, rv), okB;
      any_bad |= !okA;
      issue(bufA, rk, rv, u0 % C::UPT);
      for (int u = u0;; u += 2 * kWaves) {
        // unit u + 4 -> B (loads always issued; empty resources past the end)
        const int uB = u + kWaves, uA = uB + kWaves;
        okB = unit_rsrc(uB, pidB, rk, rv);
        any_bad |= uB < nu && !okB;
        pidA = bload_i32(rpt, tile_of(uA) * 4);
        issue(bufB, rk, rv, uB % C::UPT);
        if (okA) compute(bufA, q, (it.t0 + u / C::UPT) * kPage + (u % C::UPT) * C::UNIT, L, qk_scale, m_run, l_part, o);
        if (uB >= nu) break;
        // unit u + 8 -> A
        okA = unit_rsrc(uA, pidA, rk, rv);
        any_bad |= uA < nu && !okA;
        pidB = bload_i32(rpt, tile_of(uA + kWaves) * 4);
        issue(bufA, rk, rv, uA % C::UPT);
        if (okB) compute(bufB, q, (it.t0 + uB / C::UPT) * kPage + (uB % C::UPT) * C::UNIT, L, qk_scale, m_run, l_part, o);
        if (uA >= nu) break;
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
  WaveTrace tr(a);
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
  tr.units = r.units_done;
}

// Static split-KV: block (s, k) handles chunk k of sequence s.
template <bool FP8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_static_kernel(AttnArgs a) {
  __shared__ CombineLds lds;
  WaveTrace tr(a);
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
  tr.units = r.units_done;
}

// Merge: block (i, h, c) combines dims [32c, 32c + 32) of head h of the i-th
// sequence to merge: out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k with
// M = max_k m_k. One pass: 256 threads = 8 dim-quads x 32 split groups; each
// group folds its splits k = kg, kg + 32, ... with a running max, then the 32
// group states are combined the same way. Empty sequences get a zero row.
constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 32;
constexpr int kMergeQuads = kMergeDims / 4;
constexpr int kMergeGroups = kMergeThreads / kMergeQuads;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnArgs a, int balanced) {
  __shared__ float gm[kMergeGroups], gl[kMergeGroups];
  __shared__ f32x4 gacc[kMergeGroups][kMergeQuads];
  const int hh = blockIdx.y, d0 = blockIdx.z * kMergeDims;
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
  uint16_t* orow = a.out + (int64_t(b) * a.hq + g * a.group + hh) * kHeadDim + d0;
  const int tid = threadIdx.x;
  if (n == 0) {
    if (tid < kMergeDims) orow[tid] = 0;
    return;
  }
  const int q4 = tid % kMergeQuads, kg = tid / kMergeQuads;
  const int64_t row = int64_t(base) * a.group + hh;            // (slot, head) row of split 0
  const float* pm = a.part_m + row;
  const float* pl = a.part_l + row;
  const float* pa = a.part_acc + row * kHeadDim + d0 + 4 * q4;
  const int G = a.group;
  float M = -INFINITY, Ls = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = kg; k < n; k += kMergeGroups) {
    const float mk = pm[int64_t(k) * G], lk = pl[int64_t(k) * G];
    const f32x4 ak = *reinterpret_cast<const f32x4*>(pa + int64_t(k) * G * kHeadDim);
    const float Mn = fmaxf(M, mk);
    const float fo = __builtin_amdgcn_exp2f(M - Mn), fk = __builtin_amdgcn_exp2f(mk - Mn);
    Ls = Ls * fo + lk * fk;
    acc = acc * fo + ak * fk;
    M = Mn;
  }
  if (q4 == 0) {
    gm[kg] = M;
    gl[kg] = Ls;
  }
  gacc[kg][q4] = acc;
  __syncthreads();
  if (tid < kMergeQuads) {
    float Mt = -INFINITY;
    for (int k = 0; k < kMergeGroups; ++k) Mt = fmaxf(Mt, gm[k]);
    float Lt = 0.f;
    f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < kMergeGroups; ++k) {
      const float f = __builtin_amdgcn_exp2f(gm[k] - Mt);      // 0 for groups without splits
      Lt += f * gl[k];
      t += f * gacc[k][tid];
    }
    const float inv = 1.f / Lt;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[4 * tid + e] = f32_to_bf16_rne(t[e] * inv);
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
  hipLaunchKernelGGL(merge_kernel, dim3(S, a.group, kHeadDim / kMergeDims), dim3(kMergeThreads), 0, stream, a,
                     balanced ? 1 : 0);
  return hipGetLastError();
}

}  // namespace hpa

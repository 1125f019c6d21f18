// Split-precision router GEMM for gfx950: logits[t][e] = x[t] . W[e] with the fp32
// router weight W carried as a bf16 high part plus a bf16 residual, each multiplied
// on MFMA and accumulated in fp32, then the top-k experts of every token.
//
// Method: xiaodao.ai "HPC-Ops 把 TPOT 降 48.8%，用户未必快一半", section
// "从实验表走到 SLA，还差一轮负载测试" -- the router keeps its top-k expert choice
// by splitting its fp32 weight into a bf16 high part and a bf16 residual and
// summing two tensor-core products. hi = bf16 nearest to W, lo = bf16 nearest to
// W - hi (exact in fp32), so hi + lo carries 16 significant bits of W and every
// product with a bf16 activation is exact in fp32.
//
// Packed weight (written once by router_pack_kernel; both halves of one 16-expert
// x 32-dim tile side by side, the tile in MFMA A-operand order): for expert e and
// dim k, with tile = (e / 16) * (H / 32) + k / 32 and lane = 16 * ((k % 32) / 8) + e % 16,
//   hi at byte 2048 * tile + 16 * lane + 2 * (k % 8), lo 1024 bytes further.
// A wave's 16-byte load of one tile half is one contiguous 1 KB.
//
// GEMM, few and medium token counts (router_gemm_kernel<ME, NT, PASSES, WX>): each
// wave computes C^T[16 ME experts x 16 NT tokens] over one K range with
// v_mfma_f32_16x16x32_bf16 (A = weight tile, B = x^T: lane (token n16, group j) holds
// x[token][32 kc + 8 j .. + 8]) straight from registers, the loads of k-chunk kc + 2
// in flight while chunk kc is multiplied. Few tokens: the 4 waves of a workgroup take
// 4 consecutive K ranges of the same tile and add their results in LDS in wave order
// (one partial sum per logit per workgroup); medium (WX): they take 4 expert groups
// of the same tokens and K range, so the token fragments they all load are shared
// through L1, and each wave stores its own partial sums. Many tokens
// (router_gemm_tiled_kernel): 128 x 128 workgroup tiles staged through LDS (below).
// Rows past the last token read zeros (buffer bounds) and are not stored.
//
// Reduction and top-k: the partial sums of a logit are added in partial order and
// the logits stored; the top-k (larger value first, equal values to the lower
// expert index) over 64-bit (value, expert) keys. Few tokens (router_topk_wg_kernel,
// one workgroup per token): ranks of the keys in LDS, within 64-expert segments and
// then among the segments' k largest. Many tokens (router_topk_kernel, one wave per
// token): k rounds of a wave-wide maximum.
#include "router_internal.hpp"

namespace hpa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kBufDword3 = 0x00020000;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kBufDword3);
}

__device__ inline u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays NaN)
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One thread per 8 consecutive dims of one expert: both halves of 8 weights.
__global__ __launch_bounds__(256) void router_pack_kernel(const float* __restrict__ w, int E, int H,
                                                          uint8_t* __restrict__ packed) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int groups = H / 8;
  if (g >= int64_t(E) * groups) return;
  const int e = static_cast<int>(g / groups), k0 = static_cast<int>(g % groups) * 8;
  const f32x4* src = reinterpret_cast<const f32x4*>(w + int64_t(e) * H + k0);
  const f32x4 a = src[0], b = src[1];
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 hi, lo;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h2 = 0, l2 = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float x = v[2 * p + s];
      const uint32_t h = bf16_rne(x);
      const float r = x - __builtin_bit_cast(float, h << 16);     // exact: x and h agree in their top 8 bits
      h2 |= h << (16 * s);
      l2 |= bf16_rne(r) << (16 * s);
    }
    hi[p] = h2;
    lo[p] = l2;
  }
  const int64_t tile = int64_t(e / 16) * (H / 32) + k0 / 32;
  const int lane = 16 * ((k0 % 32) / 8) + e % 16;
  uint8_t* dst = packed + tile * 2048 + 16 * lane;
  *reinterpret_cast<u32x4*>(dst) = hi;
  *reinterpret_cast<u32x4*>(dst + 1024) = lo;
}

template <int ME, int NT>
struct Frag {
  u32x4 hi[ME], lo[ME], x[NT];
};

template <int ME, int NT, int PASSES, bool WX>
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* x, const uint8_t* packed, int T, int E,
                                                          int H, int slots, int n_eg, int kw, RouterArgs a) {
  __shared__ f32x4 red[WX ? 1 : 4][WX ? 1 : ME * NT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int m16 = lane & 15, j = lane >> 4;
  const int nkc = H / 32;
  const int wg = blockIdx.x;
  const int ksg = wg % slots;
  const int rest = wg / slots;
  // WX: the 4 waves take expert groups 4 q .. 4 q + 3 of K range ksg; otherwise K ranges
  // 4 ksg .. 4 ksg + 3 of expert group eg
  const int n_egw = WX ? n_eg / 4 : n_eg;
  const int eg = WX ? 4 * (rest % n_egw) + wave : rest % n_egw, tg = rest / n_egw;
  const int ks = WX ? ksg : 4 * ksg + wave;
  const int c0 = min(ks * kw, nkc), c1 = min(c0 + kw, nkc);
  const int eb0 = eg * ME, tok0 = tg * 16 * NT;
  const int rows = min(T - tok0, 16 * NT);
  const rsrc_t rw = make_rsrc(packed, static_cast<uint32_t>(int64_t(E) * H * 4));
  const rsrc_t rx = make_rsrc(x + int64_t(tok0) * H, static_cast<uint32_t>(rows * H * 2));

  // lane-constant parts of the offsets in VGPRs, the chunk's part in the scalar offset
  uint32_t xoff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) xoff[nt] = static_cast<uint32_t>(((16 * nt + m16) * H + 8 * j) * 2);
  const uint32_t woff = 16 * lane;
  auto load = [&](Frag<ME, NT>& f, int kc) {
    const uint32_t kx = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(64 * kc));
#pragma unroll
    for (int me = 0; me < ME; ++me) {
      const uint32_t tw = static_cast<uint32_t>(
          __builtin_amdgcn_readfirstlane(static_cast<int>((int64_t(eb0 + me) * nkc + kc) * 2048)));
      f.hi[me] = bload16(rw, woff, tw);
      if (PASSES == 2) f.lo[me] = bload16(rw, woff + 1024, tw);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) f.x[nt] = bload16(rx, xoff[nt], kx);
  };
  f32x4 acc[ME][NT];
#pragma unroll
  for (int me = 0; me < ME; ++me)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[me][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mul = [&](const Frag<ME, NT>& f) {
#pragma unroll
    for (int me = 0; me < ME; ++me)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[me][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.hi[me]), as_bf16x8(f.x[nt]), acc[me][nt], 0, 0, 0);
        if (PASSES == 2)
          acc[me][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.lo[me]), as_bf16x8(f.x[nt]), acc[me][nt], 0, 0, 0);
      }
  };
  // a ring of kDepth fragments: the loads of chunk kc + kDepth - 1 go out before chunk
  // kc is multiplied (chunk indices clamped into the range, so every load is issued
  // and in bounds). The steady loop has no branch around a load or a product, so the
  // waits before each product count only that fragment's loads; the last < kDepth
  // chunks, already loaded, are multiplied after it.
  constexpr int kDepth = 3;
  if (c0 < c1) {
    Frag<ME, NT> f[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) load(f[d], min(c0 + d, c1 - 1));
    int kc = c0;
    for (; kc + kDepth <= c1; kc += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load(f[(d + kDepth - 1) % kDepth], min(kc + d + kDepth - 1, c1 - 1));
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the products
        mul(f[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      if (kc + d < c1) mul(f[d]);
  }
  if constexpr (WX) {
#pragma unroll
    for (int me = 0; me < ME; ++me)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = 16 * nt + m16;
        if (tok < rows)
          *reinterpret_cast<f32x4*>(a.part + (int64_t(ksg) * T + tok0 + tok) * E + 16 * (eb0 + me) + 4 * j) =
              acc[me][nt];
      }
  } else {
#pragma unroll
    for (int me = 0; me < ME; ++me)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red[wave][me * NT + nt][lane] = acc[me][nt];
    __syncthreads();
    // thread -> (tile, lane) entries; the 4 waves' results added in wave order
    for (int idx = threadIdx.x; idx < ME * NT * 64; idx += 256) {
      const int r = idx / 64, l = idx % 64;
      const int me = r / NT, nt = r % NT;
      const int tok = 16 * nt + (l & 15);
      if (tok >= rows) continue;
      f32x4 s = red[0][r][l];
#pragma unroll
      for (int w = 1; w < 4; ++w) s += red[w][r][l];
      const int e = 16 * (eb0 + me) + 4 * (l >> 4);
      *reinterpret_cast<f32x4*>(a.part + (int64_t(ksg) * T + tok0 + tok) * E + e) = s;
    }
  }
}


// Many tokens: 128 experts x 128 tokens per workgroup over one K range. Each K-step
// (32 dims) of both weight halves (8 tiles x 2 KB, copied as they lie in the packed
// layout) and of x (128 tokens x 64 bytes, rearranged into 8 B-operand tiles of 1 KB)
// is staged in LDS, in three rotating stages (below). Waves 2 x 2: wave (we, wt) multiplies expert
// blocks 4 we .. 4 we + 3 with token blocks 4 wt .. 4 wt + 3 (16 accumulators), so
// every fragment read from LDS feeds 4 (or 8) MFMAs.
template <int PASSES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void router_gemm_tiled_kernel(RouterArgs a) {
  constexpr int kWPieces = PASSES == 2 ? 4 : 2;     // 16-byte weight pieces per thread per K-step
  constexpr int kXPieces = 2;
  constexpr int kXBase = 16384;                     // x tiles after the 8 weight pairs
  constexpr int kStage = 16384 + 8192;
  constexpr int kStages = 3;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6));
  const int we = wave & 1, wt = wave >> 1;
  const RouterPlan& p = a.p;
  const int nkc = a.H / 32;
  const int wg = blockIdx.x;
  const int ks = wg % p.partial_slots, rest = wg / p.partial_slots;
  const int eg = rest % p.n_eg, tg = rest / p.n_eg;
  const int c0 = min(ks * p.kw, nkc), c1 = min(c0 + p.kw, nkc);
  const int eb0 = eg * 8, tok0 = tg * 128;
  const int rows = min(a.T - tok0, 128);
  const rsrc_t rw = make_rsrc(a.packed, static_cast<uint32_t>(int64_t(a.E) * a.H * 4));
  const rsrc_t rx = make_rsrc(a.x + int64_t(tok0) * a.H, static_cast<uint32_t>(rows * a.H * 2));
  // piece i of the weight: both halves (PASSES 2: 128 pieces per 2 KB pair) or the hi
  // half only (64 pieces per pair); piece i of x: token c / 4, dims 8 (c % 4) .. + 8
  uint32_t wsrc[kWPieces], wdst[kWPieces], xsrc[kXPieces], xdst[kXPieces];
#pragma unroll
  for (int i = 0; i < kWPieces; ++i) {
    const int pc = i * 256 + tid;
    const int per = PASSES == 2 ? 128 : 64;
    const int eb = pc / per, r = (pc % per) * 16;
    wsrc[i] = static_cast<uint32_t>(int64_t(eb0 + eb) * nkc * 2048 + r);
    wdst[i] = static_cast<uint32_t>(eb * per * 16 + r);       // LDS: the staged halves packed
  }
  // x piece c: token block c / 64, fragment lane l = c % 64 (token 16 (c / 64) + l % 16,
  // dims 8 (l / 16) .. + 8), written at 16 l of its block's 1 KB: a wave's LDS stores
  // are one contiguous 1 KB (no bank conflicts), its global loads the same 16 rows x
  // 64 bytes in any lane order
#pragma unroll
  for (int i = 0; i < kXPieces; ++i) {
    const int c = i * 256 + tid;
    const int tb = c / 64, l = c % 64;
    const int t = 16 * tb + l % 16, jj = l / 16;
    xsrc[i] = static_cast<uint32_t>((t * a.H + 8 * jj) * 2);
    xdst[i] = static_cast<uint32_t>(kXBase + tb * 1024 + 16 * l);
  }
  struct Stg {
    u32x4 w[kWPieces], x[kXPieces];
  };
  auto gload = [&](Stg& g, int kc) {
    const uint32_t sw = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(kc * 2048));
    const uint32_t sx = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(kc * 64));
#pragma unroll
    for (int i = 0; i < kWPieces; ++i) g.w[i] = bload16(rw, wsrc[i], sw);
#pragma unroll
    for (int i = 0; i < kXPieces; ++i) g.x[i] = bload16(rx, xsrc[i], sx);
  };
  auto swrite = [&](const Stg& g, int stage) {
    uint8_t* st = lds + stage * kStage;
#pragma unroll
    for (int i = 0; i < kWPieces; ++i) *reinterpret_cast<u32x4*>(st + wdst[i]) = g.w[i];
#pragma unroll
    for (int i = 0; i < kXPieces; ++i) *reinterpret_cast<u32x4*>(st + xdst[i]) = g.x[i];
  };
  // all of this wave's LDS accesses complete, then the workgroup barrier (global loads
  // in flight are not waited for)
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  f32x4 acc[4][4];
#pragma unroll
  for (int ie = 0; ie < 4; ++ie)
#pragma unroll
    for (int it = 0; it < 4; ++it) acc[ie][it] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a wave's MFMA operands of one K-step: its 4 expert blocks (hi, lo) and 4 token blocks
  struct Frag {
    u32x4 ah[4], al[4], b[4];
  };
  auto fread = [&](Frag& f, int stage) {
    const uint8_t* st = lds + stage * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pair = (4 * we + i) * (PASSES == 2 ? 2048 : 1024);
      f.ah[i] = *reinterpret_cast<const u32x4*>(st + pair + 16 * lane);
      if (PASSES == 2) f.al[i] = *reinterpret_cast<const u32x4*>(st + pair + 1024 + 16 * lane);
      f.b[i] = *reinterpret_cast<const u32x4*>(st + kXBase + (4 * wt + i) * 1024 + 16 * lane);
    }
  };
  // all hi products, then all lo products: the two products into one accumulator
  // are 16 MFMAs apart, so none waits for the one before it
  auto mfma = [&](const Frag& f) {
#pragma unroll
    for (int ie = 0; ie < 4; ++ie)
#pragma unroll
      for (int it = 0; it < 4; ++it)
        acc[ie][it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.ah[ie]), as_bf16x8(f.b[it]), acc[ie][it], 0, 0, 0);
    if (PASSES == 2) {
#pragma unroll
      for (int ie = 0; ie < 4; ++ie)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          acc[ie][it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.al[ie]), as_bf16x8(f.b[it]), acc[ie][it], 0, 0, 0);
    }
  };
  // Three LDS stages and two fragment sets: while K-step kc is multiplied from
  // registers, the fragments of kc + 1 are read from LDS (written one K-step earlier)
  // and K-step kc + 2 is written from one register stage, whose global loads went
  // out one K-step earlier (loads past the range are clamped to its last K-step:
  // issued, in bounds, unused). One barrier per K-step: the stage written at kc was
  // last read at kc - 2, the stage read at kc was written at kc - 1. Stage and
  // fragment indices are compile-time: the loop is unrolled by 6, and the last
  // partial round is guarded by a uniform test around each whole step.
  if (c0 < c1) {
    Stg g;
    gload(g, c0);
    swrite(g, 0);
    gload(g, min(c0 + 1, c1 - 1));
    swrite(g, 1);
    gload(g, min(c0 + 2, c1 - 1));
    barrier();
    Frag f[2];
    fread(f[0], 0);
    auto step = [&](int kc, int d) {
      if (kc + 1 < c1) fread(f[(d + 1) % 2], (d + 1) % 3);
      __builtin_amdgcn_sched_barrier(0);
      mfma(f[d % 2]);
      __builtin_amdgcn_sched_barrier(0);
      if (kc + 2 < c1) swrite(g, (d + 2) % 3);
      gload(g, min(kc + 3, c1 - 1));
      barrier();
    };
    constexpr int kUnroll = 6;
    int kc = c0;
    for (; kc + kUnroll <= c1; kc += kUnroll) {
#pragma unroll
      for (int d = 0; d < kUnroll; ++d) step(kc + d, d);
    }
#pragma unroll
    for (int d = 0; d < kUnroll; ++d)
      if (kc + d < c1) step(kc + d, d);
  }
#pragma unroll
  for (int ie = 0; ie < 4; ++ie)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int tok = 16 * (4 * wt + it) + (lane & 15);
      if (tok < rows)
        *reinterpret_cast<f32x4*>(a.part + (int64_t(ks) * a.T + tok0 + tok) * a.E + 16 * (eb0 + 4 * we + ie) +
                                  4 * (lane >> 4)) = acc[ie][it];
    }
}

// A logit and its expert as one 64-bit key whose unsigned order is the top-k
// order: the float's bits mapped to an order-preserving uint32 (-0 taken as +0)
// above the complement of the expert index (equal values: lower index first).
// Key 0 is below every real key and stands for "no candidate".
__device__ inline uint64_t topk_key(float v, int e) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(o) << 32) | uint32_t(~e);
}
__device__ inline float key_value(uint64_t k) {
  const uint32_t o = uint32_t(k >> 32);
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ inline int key_expert(uint64_t k) { return int(~uint32_t(k)); }

// Many tokens: one wave per token (four per workgroup), 4 Q experts per lane:
// lane l holds experts 256 j + 4 l + r (j < Q, r < 4). Every logit is the sum of its
// partial sums in partial order (the loads of a batch of partials issued together,
// at clamped in-bounds addresses), stored as 16-byte rows. The top-k then takes k
// rounds of a wave-wide maximum over the lanes' largest remaining keys; keys are
// distinct, so exactly one lane owns each maximum and drops it, and lane r keeps
// the r-th result for one store at the end.
// Few tokens: one workgroup per token, Q experts per thread (E <= 256 Q): every logit's partial
// sums (loads of a batch issued together at clamped, in-bounds addresses, added in
// partial order), the logits stored; then the top-k by ranks over the keys in LDS
// (keys are distinct, so a rank is the count of larger keys). Pass 1: each key's
// rank within its segment of 64 experts; the k largest of every segment survive
// (every global top-k key does). Pass 2: each survivor's rank among the survivors,
// which for the global top-k is its global rank and for every other survivor is at
// least k; those below k are written at their rank.
template <int Q>
__global__ __launch_bounds__(256) void router_topk_wg_kernel(const float* part, int T, int E, int slots,
                                                          RouterArgs a) {
  constexpr int kBatch = 32 / Q;
  constexpr int kSegs = kRouterMaxExperts / 64;
  __shared__ uint64_t lk[kRouterMaxExperts];
  __shared__ uint64_t sk[kSegs * kRouterMaxTopK];
  const int t = blockIdx.x;
  const int64_t stride = int64_t(T) * E;
  const float* base = part + int64_t(t) * E;
  float v[Q];
  int id[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = threadIdx.x + 256 * q;
    v[q] = 0.f;
    id[q] = e < E ? e : -1;
  }
  for (int s0 = 0; s0 < slots; s0 += kBatch) {
    float pv[Q][kBatch];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        pv[q][i] = base[min(s0 + i, slots - 1) * stride + max(id[q], 0)];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (s0 + i < slots) v[q] += pv[q][i];
  }
  uint64_t key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    key[q] = 0;
    if (id[q] >= 0) {
      a.logits[int64_t(t) * E + id[q]] = v[q];
      key[q] = topk_key(v[q], id[q]);
      lk[id[q]] = key[q];
    }
  }
  const int k = a.top_k;
  if (k == 0) return;
  const int nseg = (E + 63) / 64, ns = nseg * k;
  for (int c = threadIdx.x; c < ns; c += 256) sk[c] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    if (id[q] < 0) continue;
    const int seg = id[q] / 64;                      // the same for the whole wave
    const int n = min(64, E - 64 * seg);          // a multiple of 16
    int rank = 0;
    if (n == 64) {                                   // a full segment: fixed offsets, no masks
      const uint64_t* sp = lk + 64 * seg;
#pragma unroll
      for (int j = 0; j < 64; ++j) rank += int(sp[j] > key[q]);
    } else {
      uint64_t w[64];
#pragma unroll
      for (int j = 0; j < 64; ++j) w[j] = lk[64 * seg + min(j, n - 1)];
#pragma unroll
      for (int j = 0; j < 64; ++j) rank += int((j < n) & (w[j] > key[q]));
    }
    if (rank < k) sk[seg * k + rank] = key[q];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < ns; c += 256) {
    const uint64_t kc = sk[c];
    if (kc == 0) continue;
    int rank = 0;
    for (int d0 = 0; d0 < ns; d0 += 16) {
      uint64_t w[16];
#pragma unroll
      for (int d = 0; d < 16; ++d) w[d] = sk[min(d0 + d, ns - 1)];
#pragma unroll
      for (int d = 0; d < 16; ++d) rank += int((d0 + d < ns) & (w[d] > kc));
    }
    if (rank < k) {
      a.topk_idx[int64_t(t) * k + rank] = key_expert(kc);
      a.topk_val[int64_t(t) * k + rank] = key_value(kc);
    }
  }
}

// v combined with the value of another lane of its row (DPP control CTRL: a permutation
// within quads or a rotation within the row of 16, so every source lane exists)
template <int CTRL>
__device__ inline uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
  return o > v ? o : v;
}
template <int CTRL>
__device__ inline int dpp_imin(int v) {
  const int o = __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
  return o < v ? o : v;
}

// the wave's largest (smallest) value, in every lane: within rows of 16 (quad swaps 1
// and 2, then row rotations by 4 and 8), then across the four rows' first lanes
__device__ inline uint32_t wave_umax(uint32_t v) {
  v = dpp_umax<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_umax<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_umax<0x124>(v);   // row_ror 4
  v = dpp_umax<0x128>(v);   // row_ror 8
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t y = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16 * r));
    m = y > m ? y : m;
  }
  return m;
}
__device__ inline int wave_imin(int v) {
  v = dpp_imin<0xB1>(v);
  v = dpp_imin<0x4E>(v);
  v = dpp_imin<0x124>(v);
  v = dpp_imin<0x128>(v);
  int m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) m = min(m, __builtin_amdgcn_readlane(v, 16 * r));
  return m;
}

// a logit's order-preserving 32-bit image (the high half of its key) and back
__device__ inline uint32_t value_order(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float order_value(uint32_t o) {
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// BATCH partial slices are loaded together: 8 when there are at most 8 (the tiled
// GEMM's K ranges), so no lane issues loads of clamped copies it does not add
template <int Q, int BATCH>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* part, int T, int E, int slots,
                                                          RouterArgs a) {
  constexpr int kBatch = BATCH;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                 // whole waves
  const int64_t stride = int64_t(T) * E;
  const float* base = part + int64_t(t) * E;
  f32x4 v[Q];
  int e0[Q];
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    e0[j] = 256 * j + 4 * lane;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int s0 = 0; s0 < slots; s0 += kBatch) {
    f32x4 pv[Q][kBatch];
#pragma unroll
    for (int j = 0; j < Q; ++j)
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        pv[j][i] = *reinterpret_cast<const f32x4*>(base + min(s0 + i, slots - 1) * stride + min(e0[j], E - 4));
    __builtin_amdgcn_sched_barrier(0);       // every load of the batch before the first sum
#pragma unroll
    for (int j = 0; j < Q; ++j)
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (s0 + i < slots) v[j] += pv[j][i];
      }
  }
  // per candidate: the value's order image (0: no candidate, below every real one)
  // and the expert index
  uint32_t ov[4 * Q];
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    const bool ok = e0[j] < E;                        // E is a multiple of 16: all four or none
    if (ok) *reinterpret_cast<f32x4*>(a.logits + int64_t(t) * E + e0[j]) = v[j];
#pragma unroll
    for (int r = 0; r < 4; ++r) ov[4 * j + r] = ok ? value_order(v[j][r]) : 0u;
  }
  // k rounds: the wave's largest value; among the candidates holding it the lowest
  // expert index (one holder -- the usual case -- is read from its lane, several are
  // reduced); that candidate drops out, and lane r keeps round r's result
  const int k = a.top_k;
  uint32_t mine_o = 0;
  int mine_e = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t lb = 0;
#pragma unroll
    for (int c = 0; c < 4 * Q; ++c) lb = ov[c] > lb ? ov[c] : lb;
    const uint32_t m = wave_umax(lb);
    int low = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4 * Q; ++c)
      if (ov[c] == m) low = min(low, 256 * (c / 4) + 4 * lane + c % 4);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(low != 0x7fffffff);
    const int win = __popcll(hit) == 1 ? __builtin_amdgcn_readlane(low, __builtin_ctzll(hit)) : wave_imin(low);
#pragma unroll
    for (int c = 0; c < 4 * Q; ++c)
      if (ov[c] == m && 256 * (c / 4) + 4 * lane + c % 4 == win) ov[c] = 0;
    if (lane == r) {
      mine_o = m;
      mine_e = win;
    }
  }
  if (lane < k) {
    a.topk_idx[int64_t(t) * k + lane] = mine_e;
    a.topk_val[int64_t(t) * k + lane] = order_value(mine_o);
  }
}

template <int ME, int NT, bool WX>
void gemm_launch(const RouterArgs& a, hipStream_t stream) {
  if (a.passes == 2)
    hipLaunchKernelGGL((router_gemm_kernel<ME, NT, 2, WX>), dim3(a.p.workgroups), dim3(256), 0, stream, a.x,
                       a.packed, a.T, a.E, a.H, a.p.partial_slots, a.p.n_eg, a.p.kw, a);
  else
    hipLaunchKernelGGL((router_gemm_kernel<ME, NT, 1, WX>), dim3(a.p.workgroups), dim3(256), 0, stream, a.x,
                       a.packed, a.T, a.E, a.H, a.p.partial_slots, a.p.n_eg, a.p.kw, a);
}

}  // namespace

hipError_t launch_router_pack(const float* w, int experts, int hidden, uint8_t* packed, hipStream_t stream) {
  const int64_t threads = int64_t(experts) * (hidden / 8);
  hipLaunchKernelGGL(router_pack_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream, w,
                     experts, hidden, packed);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
  if (a.p.tiled) {
    if (a.passes == 2)
      hipLaunchKernelGGL(router_gemm_tiled_kernel<2>, dim3(a.p.workgroups), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(router_gemm_tiled_kernel<1>, dim3(a.p.workgroups), dim3(256), 0, stream, a);
  } else if (a.p.me == 1 && a.p.nt == 1) gemm_launch<1, 1, false>(a, stream);
  else if (a.p.me == 1 && a.p.nt == 4) gemm_launch<1, 4, false>(a, stream);
  else if (a.p.wx) gemm_launch<2, 4, true>(a, stream);
  else gemm_launch<2, 4, false>(a, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.T <= kRouterWaveTopkMinTokens) {
    // few tokens: the ranking of one token spread over a workgroup is the shorter chain
    if (a.E <= 256) hipLaunchKernelGGL(router_topk_wg_kernel<1>, dim3(a.T), dim3(256), 0, stream, a.part, a.T, a.E,
                         a.p.partial_slots, a);
    else if (a.E <= 512) hipLaunchKernelGGL(router_topk_wg_kernel<2>, dim3(a.T), dim3(256), 0, stream, a.part, a.T,
                              a.E, a.p.partial_slots, a);
    else hipLaunchKernelGGL(router_topk_wg_kernel<4>, dim3(a.T), dim3(256), 0, stream, a.part, a.T, a.E,
                            a.p.partial_slots, a);
    return hipGetLastError();
  }
  const dim3 grid((a.T + 3) / 4);
  const bool few = a.p.partial_slots <= 8;
  if (a.E <= 256)
    hipLaunchKernelGGL((few ? router_topk_kernel<1, 8> : router_topk_kernel<1, 32>), grid, dim3(256), 0, stream, a.part,
                       a.T, a.E, a.p.partial_slots, a);
  else if (a.E <= 512)
    hipLaunchKernelGGL((few ? router_topk_kernel<2, 8> : router_topk_kernel<2, 16>), grid, dim3(256), 0, stream, a.part,
                       a.T, a.E, a.p.partial_slots, a);
  else
    hipLaunchKernelGGL((router_topk_kernel<4, 8>), grid, dim3(256), 0, stream, a.part, a.T, a.E, a.p.partial_slots, a);
  return hipGetLastError();
}

}  // namespace hpa

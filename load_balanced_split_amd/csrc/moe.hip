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
// The chain (no gather: tokens and activations are read in place by pair index):
//  moe_prepare_kernel   blocks 0 .. T-1 quantise one token row each to E4M3 (scale
//      amax / 448); block T builds the routing index: the pairs p = t K + k grouped
//      by expert (each group in pair order, by a counting sort) and the table of
//      pair blocks (expert, first pair, up to 16 pairs).
//  moe_gate_up_kernel   one wave per (pair block, 16 or 32 rows of I): for each 16-row
//      block, 16 gate and 16 up rows of W1 against the block's token codes on
//      v_mfma_f32_16x16x128_f8f6f4, per-channel and token scales, SwiGLU; writes the
//      fp32 activations and the largest magnitude of each 16-wide slice.
//  moe_quant_act_kernel one block per pair: the activation row's scale (max of its
//      slice maxima / 448) and E4M3 codes.
//  moe_down_kernel      one wave per (pair block, 32 rows of H): two 16-row tiles of W2
//      against the block's activation codes; scales and routing weight applied.
//  moe_merge_kernel     out[t] = sum over k, in k order, of the pair results -> bf16.
// With at most kMoeDirectMaxPairs pairs there is no routing index and two launches:
//  moe_gate_up_direct_kernel every pair its own block; the workgroup quantises the
//      pair's token itself.
//  moe_down_direct_kernel    one workgroup per (token, 16 rows of H), one wave per slot
//      of the token: requantisation, Down, scales and the merge in k order.
// Both paths give the same bits.
//
// Products: A = 16 weight rows, B = 16 pairs; per 128-wide k chunk a lane (row or
// pair m, group q) holds the 32 bytes [128 c + 32 q, + 32) of its row, both operands
// alike, and one MFMA consumes them -- the sum over k (the FP8 MFMA adds the 128
// exact products of a chunk more coarsely than an fp32 sum would). The grouped
// kernels' workgroups are one wave each so that a batch with a few active experts
// still spreads over every CU.
#include "hpa_internal.hpp"
#include "moe_internal.hpp"

#include <algorithm>
#include <cmath>

namespace hpa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kMoeThreads = 256;
constexpr int kPairsPerBlock = 16;
constexpr int kBufDword3 = 0x00020000;
// Weights are packed (hpa_moe_pack_weights): every 16-byte-per-lane load of a wave
// reads one contiguous 1 KB, whole lines read once, so they stream (nt).
constexpr int kPolicyWeights = 2;
// Up to this many pairs (tokens x top_k) every pair is its own block and the routing
// index is not built (a few pairs rarely share an expert): two launches instead of five.
constexpr int kMoeDirectMaxPairs = 16;

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kBufDword3);
}

__device__ inline u32x4 wload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), kPolicyWeights);
}

// activation codes (small, re-read by many waves): default policy
__device__ inline u32x4 aload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

// fp32 -> OCP E4M3 code: nearest value, ties to even mantissa, saturating at 448.
// Subnormal range (below 2^-6): the nearest multiple of 2^-9. Normal range: the fp32
// mantissa rounded to 3 bits, nearest, ties to even, by adding 2^19 - 1 plus the lowest
// kept bit and shifting (a carry moves into the exponent, as it should), then the
// exponent rebiased from 127 to 7 (subtracting 120 << 3).
__device__ inline uint32_t e4m3_code(float x) {
  const uint32_t sign = __builtin_signbit(x) ? 0x80u : 0u;
  const float a = fminf(fabsf(x), 448.0f);
  if (a < 0.015625f) return sign | static_cast<uint32_t>(rintf(a * 512.0f));
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  return sign | (((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - 960u);
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


// Quantise one token row (blocks 0 .. T-1), or build the routing index (block T).
__global__ __launch_bounds__(kMoeThreads) void moe_prepare_kernel(MoeArgs a) {
  __shared__ float red[4];
  // routing block: pairs are placed by four waves, wave w taking the w-th quarter of the
  // pair range; cntw[w][e] counts expert e's pairs in quarter w, then holds wave w's
  // running slot for e
  __shared__ int cntw[4][kMoeMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x < static_cast<unsigned>(a.T)) {
    const int t = blockIdx.x;
    const int pieces = a.H / 8;                               // 16-byte pieces of 8 bf16
    const uint16_t* row = a.x + int64_t(t) * a.H;
    // all loads first, with no branch (indexes past the row clamped to its last piece:
    // the maximum is unchanged, the piece is stored again with the same codes)
    constexpr int kPieces = kMoeMaxHidden / 8 / kMoeThreads;
    u32x4 v[kPieces];
#pragma unroll
    for (int j = 0; j < kPieces; ++j) v[j] = *reinterpret_cast<const u32x4*>(row + 8 * min(j * kMoeThreads + tid, pieces - 1));
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v[j][d] << 16)));
        amax = fmaxf(amax, fabsf(__builtin_bit_cast(float, v[j][d] & 0xffff0000u)));
      }
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax / 448.0f)));
    if (tid == 0) a.sx[t] = s;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      uint32_t w[2] = {0, 0};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = __builtin_bit_cast(float, v[j][d] << 16);
        const float hi = __builtin_bit_cast(float, v[j][d] & 0xffff0000u);
        w[d / 2] |= (e4m3_code(lo / s) | (e4m3_code(hi / s) << 8)) << (16 * (d % 2));
      }
      const uint2 pk = s > 0.f ? make_uint2(w[0], w[1]) : make_uint2(0u, 0u);   // a zero token: codes 0
      *reinterpret_cast<uint2*>(a.x8 + int64_t(t) * a.H + 8 * min(j * kMoeThreads + tid, pieces - 1)) = pk;
    }
    return;
  }
  // routing index: counts per expert and quarter, their prefix (list offsets) and the
  // pair blocks
  static_assert(kMoeThreads == 4 * 64, "one wave per quarter");
  const int Q = (a.P + 3) / 4;                      // pairs per quarter
  for (int e = tid; e < a.E; e += kMoeThreads) {
#pragma unroll
    for (int w = 0; w < 4; ++w) cntw[w][e] = 0;
  }
  __syncthreads();
  // the ids are read in batches of 16 per thread, all loads of a batch issued together
  constexpr int kIdBatch = 16;
  bool bad = false;
  for (int base = 0; base < a.P; base += kIdBatch * kMoeThreads) {
    int v[kIdBatch];
#pragma unroll
    for (int i = 0; i < kIdBatch; ++i) {
      const int p = base + i * kMoeThreads + tid;
      v[i] = p < a.P ? a.ids[p] : 0;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kIdBatch; ++i) {
      if (base + i * kMoeThreads >= a.P) break;               // uniform
      const int p = base + i * kMoeThreads + tid;
      if (p >= a.P) continue;
      if (v[i] >= 0 && v[i] < a.E) atomicAdd(&cntw[p / Q][v[i]], 1);
      else bad = true;
    }
  }
  if (bad && a.err) __hip_atomic_fetch_or(a.err, HPA_DEVERR_MOE_EXPERT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid < 64) {                   // wave 0: exclusive prefixes of counts and of block counts
    int carry = 0, bcarry = 0;
    for (int base = 0; base < a.E; base += 64) {
      const int e = base + lane;
      int cq[4] = {0, 0, 0, 0};
      if (e < a.E) {
#pragma unroll
        for (int w = 0; w < 4; ++w) cq[w] = cntw[w][e];
      }
      const int c = cq[0] + cq[1] + cq[2] + cq[3];
      const int nb = (c + kPairsPerBlock - 1) / kPairsPerBlock;
      int x = c, y = nb;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int xs = __shfl_up(x, o, 64), ys = __shfl_up(y, o, 64);
        if (lane >= o) {
          x += xs;
          y += ys;
        }
      }
      if (e < a.E) {
        // wave w's first slot for e: the expert's list offset plus its pairs in
        // earlier quarters
        int r = carry + x - c;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          cntw[w][e] = r;
          r += cq[w];
        }
        for (int b = 0; b < nb; ++b) {          // this expert's pair blocks
          const int g = bcarry + y - nb + b;
          a.blk[g] = e;
          a.blk[a.P + g] = carry + x - c + kPairsPerBlock * b;
          a.blk[2 * a.P + g] = min(kPairsPerBlock, c - kPairsPerBlock * b);
        }
      }
      carry += __shfl(x, 63, 64);
      bcarry += __shfl(y, 63, 64);
    }
    if (lane == 0) *a.nblk = bcarry;
  }
  __syncthreads();
  // wave w places the pairs of its quarter in pair order, 64 at a time: the lanes
  // holding the same expert are found by matching the bits of expert + 1 (0: skipped)
  // with ballots; a pair's slot is the wave's running slot for its expert plus the
  // matching lanes below it, and the lowest of those lanes advances it (LDS accesses of
  // a wave stay in order; each wave has its own row of running slots)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int q0 = wv * Q, q1 = min(a.P, q0 + Q);
  for (int base = q0; base < q1; base += kIdBatch * 64) {
    int v[kIdBatch];
#pragma unroll
    for (int i = 0; i < kIdBatch; ++i) {
      const int p = base + 64 * i + lane;
      v[i] = p < q1 ? a.ids[p] : -1;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kIdBatch; ++i) {
      if (base + 64 * i >= q1) break;                        // uniform
      const int p = base + 64 * i + lane;
      const int e = v[i] >= 0 && v[i] < a.E ? v[i] : -1;
      const uint32_t key = static_cast<uint32_t>(e + 1);
      uint64_t same = ~0ull;
#pragma unroll
      for (int b = 0; b < 11; ++b) {                         // kMoeMaxExperts + 1 < 2^11
        const uint64_t ones = __ballot((key >> b) & 1u);
        same &= ((key >> b) & 1u) ? ones : ~ones;
      }
      const uint64_t below = same & ((1ull << lane) - 1ull);
      if (e >= 0) {
        a.list[cntw[wv][e] + __popcll(below)] = p;
        if (below == 0) cntw[wv][e] += __popcll(same);
      }
    }
  }
}

// Gate-Up + SwiGLU: one wave per (pair block, 16 rows of I). DIRECT (a few pairs, no
// routing index): block gb is pair gb alone, a workgroup of kDirectWaves waves takes
// as many row blocks of it and quantises its token itself (the same arithmetic as the
// prepare kernel, so the same codes and scale) into LDS, from where lane group q of
// column 0 takes each chunk's 32 codes. Grouped: the block's table entry, then its
// pairs from the list, their token codes from the routing pass. The two kernels below
// pass the pointers and sizes of their first loads as leading arguments, which the
// launch preloads into scalar registers (struct arguments are not), and issue the
// first weight chunks as soon as the expert id is in.
constexpr int kDirectWaves = 2;
template <bool DIRECT, int NT>
__device__ __forceinline__ void gate_up(const int32_t* __restrict__ ids, const int32_t* __restrict__ nblk,
                                        const int32_t* __restrict__ blk, const int32_t* __restrict__ list,
                                        const uint8_t* __restrict__ w1, const uint16_t* __restrict__ x,
                                        const uint8_t* __restrict__ x8, int P, int K, int E, int H, int I,
                                        const MoeArgs& a) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[DIRECT ? kMoeMaxHidden : 16];
  __shared__ float red[kDirectWaves];
  // grouped: NT consecutive row blocks per wave, sharing each token-code fragment
  static_assert(!DIRECT || NT == 1, "one row block per wave in the few-pair kernel");
  const int wave = DIRECT ? static_cast<int>(threadIdx.x >> 6) : 0;
  const int nib = DIRECT ? I / (16 * kDirectWaves) : I / (16 * NT);   // workgroups per pair block
  // DIRECT: the pair is the fast index (the few pairs' first row blocks go out first);
  // grouped: the row block is (measured faster there)
  const int ib = (DIRECT ? static_cast<int>(blockIdx.x) / P : static_cast<int>(blockIdx.x) % nib) *
                     (DIRECT ? kDirectWaves : NT) + wave;          // the wave's first row block
  const int gb = DIRECT ? static_cast<int>(blockIdx.x) % P : static_cast<int>(blockIdx.x) / nib;
  const int lane = threadIdx.x & 63, m16 = lane & 15, q = lane >> 4;
  int e, n, praw = 0;
  bool live = true;
  if constexpr (DIRECT) {
    // no early exit for an id outside [0, E): the loads below do not wait for the
    // test; such a pair streams expert 0, stores nothing and is reported once
    e = ids[gb];
    live = e >= 0 && e < E;
    e = live ? e : 0;
    n = 1;
  } else {
    // the block count and the block's table entry in one round trip (gb < BMAX <= P:
    // the entry is in bounds, also past the count); the empty asm takes all four
    // values before the exit test, which keeps the entry's loads ahead of it
    int nbk = *nblk, first;
    e = blk[gb];
    first = blk[P + gb];
    n = blk[2 * P + gb];
    asm volatile("" : "+s"(nbk), "+s"(e), "+s"(first), "+s"(n));
    if (gb >= nbk) return;
    praw = list[first + min(m16, n - 1)];          // a lane past the block re-reads its last pair
  }
  const bool valid = m16 < n;
  const int nch = H / 128;
  const rsrc_t rw = make_rsrc(w1 + int64_t(e) * 2 * I * H, static_cast<uint32_t>(int64_t(2) * I * H));
  const rsrc_t rx = make_rsrc(x8, static_cast<uint32_t>(int64_t(a.T) * H));
  // packed tiles of row block rb: 2 KB per 128-wide chunk, chunks consecutive
  uint32_t og[NT], ou[NT];
  // the epilogue's scales, requested before the weight stream
  const float* s1e = a.s1 + int64_t(e) * 2 * I;
  f32x4 sg[NT], su[NT], accg[NT], accu[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    og[j] = static_cast<uint32_t>((ib + j) * nch * 2048 + 16 * lane);
    ou[j] = static_cast<uint32_t>((I / 16 + ib + j) * nch * 2048 + 16 * lane);
    sg[j] = *reinterpret_cast<const f32x4*>(s1e + (ib + j) * 16 + 4 * q);
    su[j] = *reinterpret_cast<const f32x4*>(s1e + I + (ib + j) * 16 + 4 * q);
    accg[j] = accu[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int p = 0;
  uint32_t ox = 0;                                   // grouped: set once the pair is in
  float sx_t = 0.f, sdirect = 0.f;
  constexpr int kDepth = DIRECT ? 8 : 4;   // DIRECT: few waves, each streams a whole pair's rows
  u32x4 ag[kDepth][NT][2], au[kDepth][NT][2], bx[kDepth][2];
  // DIRECT: the pair's token (the same for every thread), 8 bf16 per 16-byte piece,
  // H / 8 <= 512 pieces, kTokPieces per thread. Its loads go out first, so that waiting
  // for them does not wait for the weight loads issued after them, and none of this
  // branches (the compiler would move a load under a branch to its use and wait
  // there): indexes past the row are clamped to its last piece, which leaves the
  // maximum unchanged and stores that piece's codes again.
  constexpr int kThreads = 64 * kDirectWaves;
  constexpr int kTokPieces = DIRECT ? kMoeMaxHidden / 8 / kThreads : 1;
  u32x4 tok[kTokPieces];
  auto load_token = [&] {
    const uint16_t* row = x + int64_t(gb / K) * H;
#pragma unroll
    for (int j = 0; j < kTokPieces; ++j)
      tok[j] = *reinterpret_cast<const u32x4*>(row + 8 * min(j * kThreads + static_cast<int>(threadIdx.x), H / 8 - 1));
  };
  auto quantise_token = [&] {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < kTokPieces; ++j) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        m = fmaxf(m, fabsf(__builtin_bit_cast(float, tok[j][d] << 16)));
        m = fmaxf(m, fabsf(__builtin_bit_cast(float, tok[j][d] & 0xffff0000u)));
      }
    }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kDirectWaves; ++w) m = fmaxf(m, red[w]);
    sdirect = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, m / 448.0f)));
#pragma unroll
    for (int j = 0; j < kTokPieces; ++j) {
      uint32_t w[2] = {0, 0};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = __builtin_bit_cast(float, tok[j][d] << 16);
        const float hi = __builtin_bit_cast(float, tok[j][d] & 0xffff0000u);
        w[d / 2] |= (e4m3_code(lo / sdirect) | (e4m3_code(hi / sdirect) << 8)) << (16 * (d % 2));
      }
      const uint2 pk = sdirect > 0.f ? make_uint2(w[0], w[1]) : make_uint2(0u, 0u);   // a zero token: codes 0
      *reinterpret_cast<uint2*>(codes + 8 * min(j * kThreads + static_cast<int>(threadIdx.x), H / 8 - 1)) = pk;
    }
    __syncthreads();
  };
  auto load_codes = [&](int slot, int c) {     // DIRECT: the token's codes from LDS
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    bx[slot][0] = valid ? *reinterpret_cast<const u32x4*>(codes + 128 * c + 32 * q) : z;
    bx[slot][1] = valid ? *reinterpret_cast<const u32x4*>(codes + 128 * c + 32 * q + 16) : z;
  };
  auto wload = [&](int slot, int c) {
    const uint32_t st = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(2048 * c));
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      ag[slot][j][0] = wload16(rw, og[j], st);
      ag[slot][j][1] = wload16(rw, og[j] + 1024, st);
      au[slot][j][0] = wload16(rw, ou[j], st);
      au[slot][j][1] = wload16(rw, ou[j] + 1024, st);
    }
  };
  auto load = [&](int slot, int c) {
    const uint32_t sc = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(128 * c));
    wload(slot, c);
    if constexpr (DIRECT) {
      load_codes(slot, c);
    } else {
      bx[slot][0] = aload16(rx, ox, sc);
      bx[slot][1] = aload16(rx, ox + 16, sc);
    }
  };
  auto mul = [&](int slot) {
    const i32x8 B = operand(bx[slot][0], bx[slot][1]);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      accg[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(ag[slot][j][0], ag[slot][j][1]), B, accg[j],
                                                                 0, 0, 0, 0, 0, 0);
      accu[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(au[slot][j][0], au[slot][j][1]), B, accu[j],
                                                                 0, 0, 0, 0, 0, 0);
    }
  };
  auto wprologue = [&] {
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) wload(d, min(d, nch - 1));
  };
  // chunk c lives in ring slot c % kDepth (compile-time: the loop is unrolled by kDepth);
  // the loads of chunk c + kDepth - 1 go out before chunk c is multiplied. The first
  // chunks' weight loads go out before the token is quantised (DIRECT) or while the
  // pair list is loading (grouped).
  if constexpr (DIRECT) {
    load_token();
    __builtin_amdgcn_sched_barrier(0);
    wprologue();
    __builtin_amdgcn_sched_barrier(0);
    quantise_token();
    p = valid ? gb : 0;
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) load_codes(d, min(d, nch - 1));
  } else {
    wprologue();
    __builtin_amdgcn_sched_barrier(0);
    p = valid ? praw : 0;
    const int t = p / K;
    // padding pair columns read past the buffer: zeros
    ox = valid ? static_cast<uint32_t>(t * H + 32 * q) : 0x80000000u;
    sx_t = a.sx[t];
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) {
      const uint32_t sc = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(128 * min(d, nch - 1)));
      bx[d][0] = aload16(rx, ox, sc);
      bx[d][1] = aload16(rx, ox + 16, sc);
    }
  }
  int c = 0;
  for (; c + kDepth <= nch; c += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      load((d + kDepth - 1) % kDepth, min(c + d + kDepth - 1, nch - 1));
      mul(d);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (c + d < nch) mul(d);
  if (!live) {
    if (ib == 0 && lane == 0 && a.err)
      __hip_atomic_fetch_or(a.err, HPA_DEVERR_MOE_EXPERT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // lane (m16, q) holds gate / up rows 16 (ib + j) + 4 q + i (i < 4) of pair column m16
  const float sxm = valid ? (DIRECT ? sdirect : sx_t) : 0.f;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    f32x4 act;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = accg[j][i] * sxm * sg[j][i];
      const float u = accu[j][i] * sxm * su[j][i];
      act[i] = g / (1.0f + expf(-g)) * u;
      amax = fmaxf(amax, fabsf(act[i]));
    }
    if (valid) *reinterpret_cast<f32x4*>(a.act + int64_t(p) * I + (ib + j) * 16 + 4 * q) = act;
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (valid && q == 0) a.amax[int64_t(p) * (I / 16) + ib + j] = amax;
  }
}

__global__ __launch_bounds__(64 * kDirectWaves) void moe_gate_up_direct_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ w1, const uint16_t* __restrict__ x, int P, int K,
    int E, int H, int I, MoeArgs a) {
  gate_up<true, 1>(ids, nullptr, nullptr, nullptr, w1, x, nullptr, P, K, E, H, I, a);
}

// NT row blocks per wave: 2 pays where pair blocks are full enough to share their token
// codes (128 tokens, 8 pairs per expert: 129.4 -> 126.3 us per call), 1 where they hold
// a pair or two (32 tokens: 104 against 106 us)
template <int NT>
__global__ __launch_bounds__(64) void moe_gate_up_kernel(const int32_t* __restrict__ nblk,
                                                         const int32_t* __restrict__ blk,
                                                         const int32_t* __restrict__ list,
                                                         const uint8_t* __restrict__ w1,
                                                         const uint8_t* __restrict__ x8, int P, int K, int H, int I,
                                                         MoeArgs a) {
  gate_up<false, NT>(nullptr, nblk, blk, list, w1, nullptr, x8, P, K, a.E, H, I, a);
}

// Requantise one pair's activation row: scale = max of its slice maxima / 448.
__global__ __launch_bounds__(kMoeThreads) void moe_quant_act_kernel(MoeArgs a) {
  __shared__ float red[4];
  const int p = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(kMoeMaxInter / 16 <= kMoeThreads, "one slice maximum per thread");
  constexpr int kPieces = kMoeMaxInter / 4 / kMoeThreads;       // pieces of 4 per thread
  // the slice maxima (one per thread) and the row are loaded together, with no branch
  // (indexes past the end clamped: the maximum is unchanged, the piece is stored again
  // with the same codes). Every pair is requantised, also one whose expert id is
  // outside [0, E): its row is in no pair block, so nothing reads its codes or scale.
  const float amax_t = a.amax[int64_t(p) * (a.I / 16) + min(tid, a.I / 16 - 1)];
  const float* row = a.act + int64_t(p) * a.I;
  f32x4 v[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) v[j] = *reinterpret_cast<const f32x4*>(row + 4 * min(j * kMoeThreads + tid, a.I / 4 - 1));
  float amax = wave_max(amax_t);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax / 448.0f)));
  if (tid == 0) a.sa[p] = s;
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    if (j * kMoeThreads >= a.I / 4) break;          // uniform
    uint32_t w = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) w |= e4m3_code(v[j][d] / s) << (8 * d);
    w = s > 0.f ? w : 0u;
    *reinterpret_cast<uint32_t*>(a.act8 + int64_t(p) * a.I + 4 * min(j * kMoeThreads + tid, a.I / 4 - 1)) = w;
  }
}

// Down + scales + routing weight: one wave per (pair block, 16 NT rows of H), the NT
// row tiles sharing each activation-code fragment. As in Gate-Up: the first loads'
// pointers and sizes are preloaded arguments, the block count and table entry come in
// one round trip, the first weight chunks go out while the pair list is loading.
constexpr int kDownTiles = 2;   // 1: 134 us at 128 tokens; 2: 130 us; 4: 130 us, 2 us slower at 32
template <int NT>
__global__ __launch_bounds__(64) void moe_down_kernel(const int32_t* __restrict__ nblk, const int32_t* __restrict__ blk,
                                                      const int32_t* __restrict__ list, const uint8_t* __restrict__ w2,
                                                      const uint8_t* __restrict__ act8, int P, int H, int I,
                                                      MoeArgs a) {
  const int ntiles = H / (16 * NT);
  const int nb = static_cast<int>(blockIdx.x) % ntiles;
  const int gb = static_cast<int>(blockIdx.x) / ntiles;
  const int lane = threadIdx.x, m16 = lane & 15, q = lane >> 4;
  int nbk = *nblk, e = blk[gb], first = blk[P + gb], n = blk[2 * P + gb];
  asm volatile("" : "+s"(nbk), "+s"(e), "+s"(first), "+s"(n));   // all four before the exit test
  if (gb >= nbk) return;
  const int praw = list[first + min(m16, n - 1)];   // a lane past the block re-reads its last pair
  const bool valid = m16 < n;
  const int nch = I / 128;
  const rsrc_t rw = make_rsrc(w2 + int64_t(e) * H * I, static_cast<uint32_t>(int64_t(H) * I));
  const rsrc_t ra = make_rsrc(act8, static_cast<uint32_t>(int64_t(P) * I));
  const int n0 = nb * 16 * NT;
  uint32_t ow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) ow[j] = static_cast<uint32_t>((nb * NT + j) * nch * 2048 + 16 * lane);   // packed row blocks
  // the epilogue's scales, requested before the weight stream
  f32x4 s2[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) s2[j] = *reinterpret_cast<const f32x4*>(a.s2 + int64_t(e) * H + n0 + 16 * j + 4 * q);
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int kDepth = 4;
  u32x4 aw[kDepth][NT][2], ba[kDepth][2];
  auto wload = [&](int slot, int c) {
    const uint32_t st = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(2048 * c));
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      aw[slot][j][0] = wload16(rw, ow[j], st);
      aw[slot][j][1] = wload16(rw, ow[j] + 1024, st);
    }
  };
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d) wload(d, min(d, nch - 1));
  __builtin_amdgcn_sched_barrier(0);
  const int p = valid ? praw : 0;
  const uint32_t oa = valid ? static_cast<uint32_t>(p * I + 32 * q) : 0x80000000u;
  const float fsa = a.sa[p], fwt = a.wts[p];        // unconditional (p is a pair): no branch, no wait here
  auto aload = [&](int slot, int c) {
    const uint32_t sc = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(128 * c));
    ba[slot][0] = aload16(ra, oa, sc);
    ba[slot][1] = aload16(ra, oa + 16, sc);
  };
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d) aload(d, min(d, nch - 1));
  auto mul = [&](int slot) {
    const i32x8 B = operand(ba[slot][0], ba[slot][1]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(aw[slot][j][0], aw[slot][j][1]), B, acc[j], 0, 0,
                                                                0, 0, 0, 0);
  };
  int c = 0;
  for (; c + kDepth <= nch; c += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int nx = min(c + d + kDepth - 1, nch - 1), slot = (d + kDepth - 1) % kDepth;
      wload(slot, nx);
      aload(slot, nx);
      mul(d);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (c + d < nch) mul(d);
  if (valid) {
    const float f = fsa * fwt;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      f32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = acc[j][i] * f * s2[j][i];
      *reinterpret_cast<f32x4*>(a.ybuf + int64_t(p) * H + n0 + 16 * j + 4 * q) = y;
    }
  }
}

// Few pairs: requantisation, Down and the top-k merge in one launch. Workgroup (token
// t, 16 rows n0 .. n0 + 15 of H) has one wave per slot k of the token. Wave k takes the
// activation scale of pair p = t K + k from the slice maxima Gate-Up wrote (the same
// maximum as over the row), encodes the row into its own LDS region (the grouped
// path's requantisation, same codes and scale), streams its expert's 16 rows of W2
// against it, and the workgroup adds the K results in k order (the grouped path's
// merge order, so both paths give the same bits). Dynamic LDS: K * I bytes.
template <int VP>   // activation pieces of 4 per lane: I <= 256 VP
__global__ __launch_bounds__(64 * kMoeMaxTopK) void moe_down_direct_kernel(const int32_t* __restrict__ ids, const uint8_t* __restrict__ w2,
    const float* __restrict__ act, const float* __restrict__ amaxs, const float* __restrict__ wts, int T, int K, int H,
    int I, MoeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int t = static_cast<int>(blockIdx.x) % T, nb = static_cast<int>(blockIdx.x) / T;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63, m16 = lane & 15, q = lane >> 4;
  const int p = t * K + wave;
  const int nch = I / 128, n0 = nb * 16;
  // Everything the wave needs is requested before the first wait, and nothing is
  // loaded under a branch (the compiler would move such a load to its use and wait
  // there): the expert id; the slice maxima (I / 16 <= 64 kSlices; indexes past the end
  // clamped to the last entry, which leaves the maximum unchanged) and the activation
  // row (I / 4 pieces of 4, VP per lane, clamped alike), neither of which waits for
  // the id; then, once the id is in, the
  // epilogue's scales and the first weight chunks.
  const int e = ids[p];
  const float wt = wts[p];
  constexpr int kSlices = VP / 4 > 0 ? VP / 4 : 1;
  float sl[kSlices];
  f32x4 v[VP];
  const float* arow = act + int64_t(p) * I;
  const float* mrow = amaxs + int64_t(p) * (I / 16);
#pragma unroll
  for (int j = 0; j < kSlices; ++j) sl[j] = mrow[min(j * 64 + lane, I / 16 - 1)];
#pragma unroll
  for (int j = 0; j < VP; ++j) v[j] = *reinterpret_cast<const f32x4*>(arow + 4 * min(j * 64 + lane, I / 4 - 1));
  __builtin_amdgcn_sched_barrier(0);
  const bool live = e >= 0 && e < a.E;             // uniform in the wave
  const int ee = live ? e : 0;                     // no valid expert: expert 0's rows, result unused
  const rsrc_t rw = make_rsrc(w2 + int64_t(ee) * H * I, static_cast<uint32_t>(int64_t(H) * I));
  const uint32_t ow = static_cast<uint32_t>(nb * nch * 2048 + 16 * lane);
  const f32x4 s2 = *reinterpret_cast<const f32x4*>(a.s2 + int64_t(ee) * H + n0 + 4 * q);
  constexpr int kDepth = 4;
  u32x4 aw[kDepth][2], ba[kDepth][2];
  auto wload = [&](int slot, int c) {
    const uint32_t st = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(2048 * c));
    aw[slot][0] = wload16(rw, ow, st);
    aw[slot][1] = wload16(rw, ow + 1024, st);
  };
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d) wload(d, min(d, nch - 1));
  __builtin_amdgcn_sched_barrier(0);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kSlices; ++j) amax = fmaxf(amax, sl[j]);
  amax = wave_max(amax);
  const float s = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax / 448.0f)));
  const float f = live ? s * wt : 0.f;
  uint8_t* codes = lds + wave * I;
#pragma unroll
  for (int j = 0; j < VP; ++j) {
    uint32_t w = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) w |= e4m3_code(v[j][d] / s) << (8 * d);
    w = s > 0.f ? w : 0u;                            // a zero row: codes 0 (selected, not branched)
    // a lane past the end stores the last piece's codes again (the same value; no
    // branch, so the encode stays where the loads have landed)
    *reinterpret_cast<uint32_t*>(codes + 4 * min(j * 64 + lane, I / 4 - 1)) = w;
  }
  __syncthreads();
  // B operand: column 0 is the pair, lane group q takes each chunk's 32 codes
  const bool col0 = m16 == 0;
  auto cload = [&](int slot, int c) {
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    ba[slot][0] = col0 ? *reinterpret_cast<const u32x4*>(codes + 128 * c + 32 * q) : z;
    ba[slot][1] = col0 ? *reinterpret_cast<const u32x4*>(codes + 128 * c + 32 * q + 16) : z;
  };
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (live) {
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) cload(d, min(d, nch - 1));
    int c = 0;
    for (; c + kDepth <= nch; c += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int nx = min(c + d + kDepth - 1, nch - 1), slot = (d + kDepth - 1) % kDepth;
        wload(slot, nx);
        cload(slot, nx);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(aw[d][0], aw[d][1]),
                                                               operand(ba[d][0], ba[d][1]), acc, 0, 0, 0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d)
      if (c + d < nch)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(aw[d][0], aw[d][1]),
                                                               operand(ba[d][0], ba[d][1]), acc, 0, 0, 0, 0, 0, 0);
  }
  __syncthreads();                                 // every wave is done with its codes
  // lane (0, q) holds rows n0 + 4 q + i; a slot with no valid expert stores +0, which
  // leaves the sum (started at +0, so never -0) unchanged: the grouped merge skips it
  float* ys = reinterpret_cast<float*>(lds);
  if (col0) {
    f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live) {
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = acc[i] * f * s2[i];
    }
    *reinterpret_cast<f32x4*>(ys + wave * 16 + 4 * q) = y;
  }
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += ys[k * 16 + lane];
    a.out[int64_t(t) * H + n0 + lane] = f32_to_bf16(sum);
  }
}

// out[t][n .. n + 3] = bf16 of the sum over k (in k order) of the pair results; slots
// whose expert id is outside [0, E) add nothing (the routing block reported them).
__global__ __launch_bounds__(kMoeThreads) void moe_merge_kernel(MoeArgs a) {
  const int t = blockIdx.y;
  const int nq = blockIdx.x * kMoeThreads + threadIdx.x;     // 4-dim piece
  if (4 * nq >= a.H) return;
  // all ids, then all K rows, loaded before the first sum (two round trips); a row of
  // a skipped slot is loaded (it is in the workspace) but not added
  int e[kMoeMaxTopK];
  f32x4 y[kMoeMaxTopK];
#pragma unroll
  for (int k = 0; k < kMoeMaxTopK; ++k) e[k] = k < a.K ? a.ids[t * a.K + k] : -1;
#pragma unroll
  for (int k = 0; k < kMoeMaxTopK; ++k)
    y[k] = *reinterpret_cast<const f32x4*>(a.ybuf + int64_t(t * a.K + min(k, a.K - 1)) * a.H + 4 * nq);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kMoeMaxTopK; ++k)
    if (e[k] >= 0 && e[k] < a.E) s += y[k];
  uint2 o;
  o.x = f32_to_bf16(s[0]) | (uint32_t(f32_to_bf16(s[1])) << 16);
  o.y = f32_to_bf16(s[2]) | (uint32_t(f32_to_bf16(s[3])) << 16);
  *reinterpret_cast<uint2*>(a.out + int64_t(t) * a.H + 4 * nq) = o;
}

// Packs row-major E4M3 weights [E][N][K] into MFMA-operand tiles: tile (e, rb, c) =
// rows 16 rb .. + 16 and dims 128 c .. + 128, at ((e N/16 + rb) K/128 + c) 2048 bytes;
// inside it lane l = m + 16 q (row m) holds dims 128 c + 32 q .. + 32, its first 16
// bytes at 16 l and its last 16 at 1024 + 16 l. One thread per 16-byte piece.
__global__ __launch_bounds__(kMoeThreads) void moe_pack_kernel(const uint8_t* __restrict__ w, int E, int N, int K,
                                                               uint8_t* __restrict__ packed) {
  const int64_t o = int64_t(blockIdx.x) * kMoeThreads + threadIdx.x;     // output piece
  const int64_t total = int64_t(E) * N * K / 16;
  if (o >= total) return;
  const int64_t tile = o / 128;
  const int j = static_cast<int>(o % 128), half = j / 64, l = j % 64;
  const int nchunk = K / 128;
  const int c = static_cast<int>(tile % nchunk);
  const int64_t erb = tile / nchunk;                                      // e * N/16 + rb
  const int64_t row = erb * 16 + (l % 16);                                 // e * N + 16 rb + m
  const int64_t col = int64_t(128) * c + 32 * (l / 16) + 16 * half;
  *reinterpret_cast<u32x4*>(packed + 16 * o) = *reinterpret_cast<const u32x4*>(w + row * K + col);
}

}  // namespace

hipError_t launch_moe(const MoeArgs& a, hipStream_t stream) {
  if (a.P <= kMoeDirectMaxPairs) {
    // a few pairs: one pair per block, no routing index; Gate-Up quantises the tokens,
    // Down requantises the activations and merges
    hipLaunchKernelGGL(moe_gate_up_direct_kernel, dim3(static_cast<unsigned>(a.P * (a.I / (16 * kDirectWaves)))),
                       dim3(64 * kDirectWaves), 0, stream, a.ids, a.w1, a.x, a.P, a.K, a.E, a.H, a.I, a);
    hipLaunchKernelGGL(a.I <= 1024 ? moe_down_direct_kernel<4>
                       : a.I <= 2048 ? moe_down_direct_kernel<8> : moe_down_direct_kernel<kMoeMaxInter / 256>,
                       dim3(static_cast<unsigned>(a.T * (a.H / 16))), dim3(64 * a.K), static_cast<size_t>(a.K) * a.I,
                       stream, a.ids, a.w2, a.act, a.amax, a.wts, a.T, a.K, a.H, a.I, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(moe_prepare_kernel, dim3(a.T + 1), dim3(kMoeThreads), 0, stream, a);
  const int gt = a.P >= 4 * a.E ? 2 : 1;           // row blocks per Gate-Up wave
  hipLaunchKernelGGL(gt == 2 ? moe_gate_up_kernel<2> : moe_gate_up_kernel<1>,
                     dim3(static_cast<unsigned>(int64_t(a.BMAX) * (a.I / (16 * gt)))), dim3(64), 0, stream, a.nblk, a.blk,
                     a.list, a.w1, a.x8, a.P, a.K, a.H, a.I, a);
  hipLaunchKernelGGL(moe_quant_act_kernel, dim3(a.P), dim3(kMoeThreads), 0, stream, a);
  hipLaunchKernelGGL(moe_down_kernel<kDownTiles>, dim3(static_cast<unsigned>(int64_t(a.BMAX) * (a.H / (16 * kDownTiles)))),
                     dim3(64), 0, stream, a.nblk, a.blk, a.list, a.w2, a.act8, a.P, a.H, a.I, a);
  hipLaunchKernelGGL(moe_merge_kernel, dim3((a.H / 4 + kMoeThreads - 1) / kMoeThreads, a.T), dim3(kMoeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

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

}  // namespace hpa

extern "C" hpa_status hpa_moe_pack_weights(const void* w, int32_t experts, int32_t rows, int32_t cols, void* packed,
                                            hipStream_t stream) {
  using namespace hpa;
  if (experts < 1 || experts > kMoeMaxExperts || rows < 16 || rows % 16 != 0 || rows > 2 * kMoeMaxInter ||
      cols < 128 || cols % 128 != 0 || cols > kMoeMaxHidden)
    return report_status(HPA_ERR_UNSUPPORTED, "experts %d, rows %d, cols %d (rows a multiple of 16 up to %d, cols "
                         "a multiple of 128 up to %d)", experts, rows, cols, 2 * kMoeMaxInter, kMoeMaxHidden);
  if (!w || !packed) return report_status(HPA_ERR_INVALID_ARG, "w or packed is NULL");
  if (reinterpret_cast<uintptr_t>(w) % 16 != 0 || reinterpret_cast<uintptr_t>(packed) % 16 != 0)
    return report_status(HPA_ERR_INVALID_ARG, "w and packed must be 16-byte aligned");
  if (w == packed) return report_status(HPA_ERR_INVALID_ARG, "w and packed must not be the same buffer");
  const int64_t pieces = int64_t(experts) * rows * cols / 16;
  hipLaunchKernelGGL(moe_pack_kernel, dim3(static_cast<unsigned>((pieces + kMoeThreads - 1) / kMoeThreads)),
                     dim3(kMoeThreads), 0, stream, static_cast<const uint8_t*>(w), experts, rows, cols,
                     static_cast<uint8_t*>(packed));
  if (hipGetLastError() != hipSuccess) return report_status(HPA_ERR_LAUNCH, "MoE pack launch failed");
  return HPA_OK;
}

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
  a.x8 = reinterpret_cast<uint8_t*>(wb + ws.x8);
  a.sx = reinterpret_cast<float*>(wb + ws.sx);
  a.list = reinterpret_cast<int32_t*>(wb + ws.list);
  a.blk = reinterpret_cast<int32_t*>(wb + ws.blk);
  a.nblk = reinterpret_cast<int32_t*>(wb + ws.nblk);
  a.act = reinterpret_cast<float*>(wb + ws.act);
  a.amax = reinterpret_cast<float*>(wb + ws.amax);
  a.act8 = reinterpret_cast<uint8_t*>(wb + ws.act8);
  a.sa = reinterpret_cast<float*>(wb + ws.sa);
  a.ybuf = reinterpret_cast<float*>(wb + ws.ybuf);
  a.out = static_cast<uint16_t*>(out);
  a.err = device_error;
  a.T = tokens;
  a.E = experts;
  a.K = top_k;
  a.H = hidden;
  a.I = inter;
  a.P = tokens * top_k;
  // pair blocks: at most one partial block per expert with pairs, and never more than pairs
  a.BMAX = std::min<int>(a.P, (a.P + 15) / 16 + std::min(experts, a.P));
  if (launch_moe(a, stream) != hipSuccess) return report_status(HPA_ERR_LAUNCH, "MoE launch failed");
  return HPA_OK;
}

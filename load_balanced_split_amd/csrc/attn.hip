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
// The 8 query heads of a KV head fill half of the 16-wide N side. The pages are
// stored pre-tiled for these products (layout in hpa_internal.hpp): every load
// is 16 bytes per lane and reads one contiguous 1 KB, i.e. whole 128-byte lines,
// so the K/V stream can use the non-temporal (streaming) policy without a line
// ever being fetched twice. Rows of K are assigned to MFMA rows so that the
// score registers a lane holds after Q*K^T are exactly the tokens it feeds into
// P*V.
#include "hpa_internal.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

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

// Descriptors must live in SGPRs; every base and size here is workgroup-uniform, so
// readfirstlane only pins them there (a no-op when they already are) and keeps the
// compiler from wrapping buffer loads in per-lane loops.
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kBufDword3);
}

// Cache policy bits of a buffer load: 2 = nt (streaming: KV bytes are read once),
// 16 = sc1 (device scope).
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;
constexpr int kPolicyAgent = 16;   // sc1: coherent across the device (every XCD's L2)

template <int POLICY = kPolicyDefault>
__device__ inline u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), POLICY);
}

template <int POLICY = kPolicyDefault>
__device__ inline float bload_f32(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), 0, POLICY));
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
  int L;                 // live length of the item's request when the source knows it, else -1
  int nsplit, pbase;     // splits of sequence s and its first partial slot (fused schedule)
};

// The split combine (m: running max in log2 units, l: sum of weights, acc: weighted
// V sum). Every combine of split results goes through the two functions below, in
// the order fixed by kMergeGroup and kMergeBlock, so all schedules produce the same
// bits.
//
// reduce(): the first cnt of N results, max-first: M = their largest m; each result
// weighted by 2^(m - M) (independent exponentials, not a chain through a running
// max); l and acc summed in index order. Entries at or past cnt must hold finite
// values (callers load a copy of a valid result there); they are weighted by 0.
template <int N>
__device__ inline void reduce(const float (&m)[N], const float (&l)[N], const f32x4 (&a)[N], int cnt, float& M,
                              float& L, f32x4& A) {
  float mx = m[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, i < cnt ? m[i] : -INFINITY);
  L = 0.f;
  A = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float w = i < cnt ? __builtin_amdgcn_exp2f(m[i] - mx) : 0.f;
    L = fmaf(l[i], w, L);
#pragma unroll
    for (int e = 0; e < 4; ++e) A[e] = fmaf(a[i][e], w, A[e]);
  }
  M = mx;
}

// fold (mk, lk, ak) into the running (M, L, A): the last level, over block results
__device__ inline void fold(float& M, float& L, f32x4& A, float mk, float lk, const f32x4& ak) {
  const float Mn = fmaxf(M, mk);
  const float fo = __builtin_amdgcn_exp2f(M - Mn), fk = __builtin_amdgcn_exp2f(mk - Mn);
  L = fmaf(L, fo, lk * fk);
#pragma unroll
  for (int e = 0; e < 4; ++e) A[e] = fmaf(A[e], fo, ak[e] * fk);
  M = Mn;
}

// Shared state of the 4 waves for the end-of-item combine.
// Per-wave exchange areas of the VALU products: the item's q for every head at
// each lane group's dims [c][j][h], the scores of one unit before their sum over
// lane groups [block][row][j][h], and P [k-step][j][h]. Empty in MFMA builds.
struct ValuLds {
  bf16x8 q[kWaves][4][4][kValuMaxGroup];
  float s[kWaves][4][16][4][kValuMaxGroup];
  bf16x8 p[kWaves][2][4][kValuMaxGroup];
};
struct NoValuLds {};

struct CombineLds {
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  float o[kWaves][kMaxGroup][kORow];
  int flag;                   // an arrival count, broadcast to the workgroup
  int claim[2];               // dynamic tail: claimed chunk, broadcast (two slots, alternating)
  [[no_unique_address]] std::conditional_t<kValuProducts, ValuLds, NoValuLds> v;
};

// Accumulator registers per lane. MFMA: the 8 C tiles of O^T[16 d x 16 heads]
// (lane: head m16, dims 16 n + 4 j .. + 3). VALU products: o(h, n) = element n % 4
// of register 2 h + n / 4, dim 16 n + m16 of head h, summed over the lane's tokens only.
constexpr int kAccRegs = kValuProducts ? 2 * kValuMaxGroup : 8;

// a . b + acc over 8 bf16 pairs, in fp32 (VALU dot2 instructions)
[[maybe_unused]] __device__ inline float dot8(bf16x8 a, bf16x8 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}

// Orders a wave's LDS accesses around an exchange between its own lanes (LDS
// executes one wave's instructions in order; this keeps the compiler from
// moving them across).
[[maybe_unused]] __device__ inline void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Global view of a device pointer: atomics through it are global_* instructions,
// counted on the vector memory counter only (a flat one also holds up LDS waits).
typedef __attribute__((address_space(1))) int32_t gint32_t;

// Sticky device error bits (in the plan header, or where the caller redirected them;
// callers check a.err when it may be null).
__device__ inline void report_error(const AttnArgs& a, int bits) {
  __hip_atomic_fetch_or((gint32_t*)a.err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Dynamic tail: the last positions of the plan are cut into D chunks that the
// persistent workers claim one at a time on a device-scope counter, each when it
// runs out of work, so faster workers end up with more of them. Claims return
// 0, 1, 2, ...; one at or past D means the queue is empty. When the source hands
// out the last item a worker holds it sets `want`; the worker's next stream then
// issues the claim (one lane of wave 0) just before a unit's loads and puts the
// returned chunk into LDS right after the previous unit's compute, whose wait
// already covers it, so the claim never drains the K/V stream. take() (one
// barrier) reads it when the next item is needed. The last workgroup to finish
// returns both counters to 0, so the next launch starts from an empty count.
struct TailQueue {
  int32_t* ctr;           // [chunks claimed, workgroups finished]
  int* slots;             // CombineLds::claim
  int D;
  int k = 0;              // claims taken (selects the slot)
  bool want = false;      // uniform: a claim is wanted and not issued yet
  bool issued = false;    // uniform: claim k is in its LDS slot (or on its way there)
  bool empty = false;

  __device__ bool open() const { return D > 0 && !empty; }
  // a global (not flat) atomic: it is counted on the vector memory counter only
  __device__ int fetch() const {
    return __hip_atomic_fetch_add((gint32_t*)ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ int* slot() const { return slots + (k & 1); }
  // uniform; the next chunk, or -1 once the queue is empty
  __device__ int take() {
    if (!issued && threadIdx.x == 0) *slot() = fetch();       // not issued ahead: claim now
    __syncthreads();   // claims k and k + 2 share a slot: claim k + 1's barrier separates them
    const int c = __builtin_amdgcn_readfirstlane(*slot());
    ++k;
    want = issued = false;
    if (c >= D) {
      empty = true;
      return -1;
    }
    return c;
  }
  // called once by each of the `participants` workgroups after its last take()
  __device__ void finish(int participants) const {
    gint32_t* g = (gint32_t*)ctr;
    if (D > 0 && threadIdx.x == 0 &&
        __hip_atomic_fetch_add(g + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == participants - 1) {
      // every other workgroup's last claim returned before it counted itself in
      __hip_atomic_store(g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(g + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

// Scalar view of read-only device arrays: a load through it returns one value
// for the whole wave into scalar registers and is waited for on the scalar
// counter, so it never orders behind the K/V stream's vector loads. Only for
// memory no kernel of the step writes while this one runs.
typedef const __attribute__((address_space(4))) int32_t cint32_t;
typedef const __attribute__((address_space(4))) float cfloat_t;
__device__ inline int sload(const int32_t* base, int64_t i) { return ((cint32_t*)base)[i]; }
__device__ inline float sloadf(const float* base, int64_t i) { return ((cfloat_t*)base)[i]; }

// Everything about one item that is uniform across the workgroup. open() issues
// the scalar loads (length, scales) and returns at once; they are first waited
// for one item later, when the item becomes current.
struct ItemState {
  Item it;
  int b, g;         // request and KV head of sequence it.s
  int L;            // live length of request b
  float kscale, vscale;
  bool valid;       // a work-list entry that fits this launch
};

// Per-workgroup driver: 4 waves on one item at a time; wave w takes the item's
// units w, w+4, ... Items are software-pipelined: while item k streams, item
// k+1's length, q and first page ids are in flight and item k+2's descriptor is
// being read; the issue slot after a wave's last unit of item k takes its first
// unit of item k+1, so the K/V stream of a wave never drains at an item boundary.
template <bool FP8, bool INMERGE = false>
struct Worker {
  const AttnArgs& a;
  CombineLds& lds;
  uint32_t units_done = 0;
  uint64_t* trec = nullptr;   // instrumented build: this wave's record
  TailQueue tq{};             // the dynamic tail (D = 0: none)
  int titem = 0;
  int lane, wave, m16, j;
  uint32_t loff;         // per-lane byte offset inside each 1 KB load
  bf16x8 q[4], qn[4];    // q operand of the current and of the next item
  UnitBuf bufA, bufB;

  __device__ Worker(const AttnArgs& args, CombineLds& l)
      : a(args), lds(l), lane(threadIdx.x & 63),
        wave(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6))),
        m16(threadIdx.x & 15), j((threadIdx.x & 63) >> 4) {
    loff = 16 * lane;
  }

  // Issue the 16 loads of one unit: tokens [half * UNIT, half * UNIT + UNIT) of one
  // (page, KV head). rk / rv cover that page's K and V (num_records 0 when the
  // unit does not exist or its page id is bad: the loads then return zeros).
  // Load i of K (of V) reads unit bytes [1024 i, 1024 i + 1024): register k[i]
  // is then score block i / 4, k-chunk i % 4 (bf16) or block i / 2, k-chunks
  // 2 (i % 2), +1 (E4M3); register v[i] is output rows 16 i .. 16 i + 15.
  __device__ void issue(UnitBuf& buf, rsrc_t rk, rsrc_t rv, int half) const {
    using C = Cfg<FP8>;
    const uint32_t ub = half * C::UNIT * kHeadDim * C::EB;
#pragma unroll
    for (int i = 0; i < 8; ++i)   // the immediate offset field holds < 4096: 4 KB steps go to soffset
      buf.k[i] = bload16<kPolicyStream>(rk, loff + 1024 * (i & 3), ub + 4096 * (i >> 2));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      buf.v[i] = bload16<kPolicyStream>(rv, loff + 1024 * (i & 3), ub + 4096 * (i >> 2));
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

  // the VALU products' LDS (only ever used in builds that have it)
  __device__ ValuLds& vl() const { return *reinterpret_cast<ValuLds*>(&lds.v); }

  // VALU products: the current item's q for every head, where each lane group
  // reads it (lane (h, j) holds head h at lane group j's dims).
  __device__ void valu_stage_q(const bf16x8 (&qc)[4]) {
    if constexpr (kValuProducts) {
      if (m16 < kValuMaxGroup) {
#pragma unroll
        for (int c = 0; c < 4; ++c) vl().q[wave][c][j][m16] = qc[c];
      }
      wave_lds_sync();
    }
  }

  // VALU products: S^T in the MFMA C layout (lane (h, j): tokens row_token(b, 4 j + i)
  // of head h). Lane (m16, j) first sums its 32 dims of token row m16 for every head,
  // then the four lane groups' sums of each (token, head) meet in LDS.
  __device__ void valu_scores(const UnitBuf& buf, f32x4 (&sc)[Cfg<FP8>::NBLK]) {
    if constexpr (kValuProducts) {
      using C = Cfg<FP8>;
      float part[C::NBLK][kValuMaxGroup];
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b)
#pragma unroll
        for (int h = 0; h < kValuMaxGroup; ++h) part[b][h] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8 qh[kValuMaxGroup];
#pragma unroll
        for (int h = 0; h < kValuMaxGroup; ++h) qh[h] = vl().q[wave][c][j][h];
#pragma unroll
        for (int b = 0; b < C::NBLK; ++b) {
          const bf16x8 kb = k_operand(buf, b, c);
#pragma unroll
          for (int h = 0; h < kValuMaxGroup; ++h) part[b][h] = dot8(kb, qh[h], part[b][h]);
        }
      }
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b) {
        f32x4* dst = reinterpret_cast<f32x4*>(&vl().s[wave][b][m16][j][0]);
        dst[0] = f32x4{part[b][0], part[b][1], part[b][2], part[b][3]};
        dst[1] = f32x4{part[b][4], part[b][5], part[b][6], part[b][7]};
      }
      wave_lds_sync();
      const int h = m16 & (kValuMaxGroup - 1);
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* r = &vl().s[wave][b][4 * j + i][0][h];
          const float x = (r[0] + r[kValuMaxGroup]) + (r[2 * kValuMaxGroup] + r[3 * kValuMaxGroup]);
          sc[b][i] = m16 < kValuMaxGroup ? x : 0.f;
        }
      }
    }
  }

  // VALU products: o(h, n) += sum over the lane's tokens of P(token, h) V(token, 16 n + m16);
  // lane (m16, j) takes P of its tokens for every head from lanes (h, j) through LDS.
  __device__ void valu_pv(const UnitBuf& buf, const bf16x8 (&pk)[Cfg<FP8>::KSTEPS], f32x4 (&o)[kAccRegs]) {
    if constexpr (kValuProducts) {
      using C = Cfg<FP8>;
      if (m16 < kValuMaxGroup) {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) vl().p[wave][ks][j][m16] = pk[ks];
      }
      wave_lds_sync();
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        bf16x8 ph[kValuMaxGroup];
#pragma unroll
        for (int h = 0; h < kValuMaxGroup; ++h) ph[h] = vl().p[wave][ks][j][h];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const bf16x8 vn = v_operand(buf, n, ks);
#pragma unroll
          for (int h = 0; h < kValuMaxGroup; ++h)
            o[2 * h + (n >> 2)][n & 3] = dot8(vn, ph[h], o[2 * h + (n >> 2)][n & 3]);
        }
      }
    }
  }

  // Online-softmax update with one unit: tokens [tok0, tok0 + UNIT) of the sequence.
  __device__ void compute(UnitBuf& buf, const bf16x8 (&q)[4], int tok0, int L, float qk_scale,
                          float& m_run, float& l_part, f32x4 (&o)[kAccRegs]) {
    using C = Cfg<FP8>;

    f32x4 sc[C::NBLK];
    if constexpr (kValuProducts) {
      valu_scores(buf, sc);
    } else {
#pragma unroll
      for (int b = 0; b < C::NBLK; ++b) {
        sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(buf, b, c), q[c], sc[b], 0, 0, 0);
      }
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
    if constexpr (kValuProducts) {
      // head h's factor sits in lane h (lane group 0)
#pragma unroll
      for (int h = 0; h < kValuMaxGroup; ++h) {
        const float ah = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
        o[2 * h] *= ah;
        o[2 * h + 1] *= ah;
      }
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] *= alpha;
    }
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
    if constexpr (kValuProducts) {
      valu_pv(buf, pk, o);
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
          o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_operand(buf, n, ks), pk[ks], o[n], 0, 0, 0);
      }
    }
    if (kTraceBuild) {   // the unit's data has been consumed by now
      if (trec && lane == 0 && units_done < kTraceUnits)
        trec[4 + kTraceStart + 3 * kTraceItems + units_done] = __builtin_amdgcn_s_memrealtime();
      ++units_done;
    }
  }

  __device__ bool bad_pid(int pid) const { return pid < 0 || pid >= a.num_pages; }

  // Descriptor -> uniform facts of the item; issues its scalar loads, waits for none.
  __device__ ItemState open(const Item& it) const {
    ItemState st;
    st.it = it;
    st.valid = it.s >= 0 && it.s < a.batch * a.hkv && it.t0 >= 0 && it.t1 > it.t0 &&
               it.t1 <= a.max_pages && it.slot < a.slots;
    const int s = st.valid ? it.s : 0;
    // integer division runs on the VALU: bring the (uniform) result back to an SGPR
    st.b = a.hkv == 1 ? s : __builtin_amdgcn_readfirstlane(s / a.hkv);
    st.g = s - st.b * a.hkv;
    st.L = it.L >= 0 ? it.L : sload(a.seq_lens, st.b);
    st.kscale = FP8 ? sloadf(a.k_scale, st.g) : 1.f;
    st.vscale = FP8 ? sloadf(a.v_scale, st.g) : 1.f;
    if (!st.valid && threadIdx.x == 0 && a.err) report_error(a, HPA_DEVERR_PLAN);
    return st;
  }

  // units of the item: UPT per tile, minus a trailing half-tile that starts past L
  __device__ int units(const ItemState& st) const {
    using C = Cfg<FP8>;
    if (!st.valid) return 0;
    int nu = (st.it.t1 - st.it.t0) * C::UPT;
    if (C::UPT > 1 && st.it.t1 * kPage - C::UNIT >= st.L) nu -= 1;
    return nu;
  }

  // page id of unit u's tile (tile clamped into the item, so the read is in
  // bounds); a scalar load, -1 for an invalid item
  __device__ int page_of(const ItemState& st, int u) const {
    using C = Cfg<FP8>;
    if (!st.valid) return -1;
    const int t = st.it.t0 + min(u / C::UPT, st.it.t1 - st.it.t0 - 1);
    return sload(a.page_table, int64_t(st.b) * a.max_pages + t);
  }

  // first token of unit u
  __device__ int tok0(const ItemState& st, int u) const {
    using C = Cfg<FP8>;
    return (st.it.t0 + u / C::UPT) * kPage + (u % C::UPT) * C::UNIT;
  }

  // unit u -> K/V resources of its (page, KV head) (empty past the item or for a bad page id)
  __device__ bool unit_rsrc(const ItemState& st, int nu, int u, int pid, rsrc_t& rk, rsrc_t& rv) const {
    using C = Cfg<FP8>;
    constexpr uint32_t page_bytes = kPage * kHeadDim * C::EB;
    const bool ok = u < nu && !bad_pid(pid);
    const uint64_t off = ok ? (uint64_t(pid) * a.hkv + st.g) * page_bytes : 0;
    rk = make_rsrc(a.k_cache + off, ok ? page_bytes : 0);
    rv = make_rsrc(a.v_cache + off, ok ? page_bytes : 0);
    return ok;
  }

  // Q^T operand of an item (lane: head m16, dims chunk_dim(c, j) .. +8; zeros for
  // heads >= G and for an invalid item). Vector loads, waited for at first use.
  __device__ void load_q(const ItemState& st, bf16x8 (&dst)[4]) const {
    const rsrc_t rq = make_rsrc(a.q + (int64_t(st.b) * a.hq + st.g * a.group) * kHeadDim,
                                st.valid ? a.group * kHeadDim * 2 : 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = as_bf16x8(bload16(rq, (m16 * kHeadDim + chunk_dim<FP8>(c, j)) * 2, 0));
  }

  __device__ void report_bad_page() const {
    if (lane == 0 && a.err) report_error(a, HPA_DEVERR_PAGE_ID);
  }

  // Stream this wave's units of item st; unit `wave` is already in bufA (okA: it
  // exists) and pidB is the page of unit wave + 4. The next unit's 16 loads are
  // always issued before the current unit is computed; after the wave's last
  // unit of st, that slot takes its first unit of the next item (nst, npid), so
  // on return bufA holds it. Returns whether that unit exists.
  __device__ bool stream(const ItemState& st, bool okA, int pidB, float& m_run, float& l_part,
                         f32x4 (&o)[kAccRegs], bool more, const ItemState& nst, int npid) {
    using C = Cfg<FP8>;
    valu_stage_q(q);
    const int nu = units(st);
    const float qk_scale = a.sm_scale * kLog2e * st.kscale;
    bool any_bad = false;
    rsrc_t rk, rv;
    int pidA = -1;
    // a wanted tail claim: issued before this item's second unit's loads, stored to
    // LDS after its first unit's compute (wave 0's first unit exists in every item)
    bool claim = tq.want;
    const bool claimer = claim && wave == 0 && lane == 0;
    int ticket = 0;
    for (int u = wave;; u += 2 * kWaves) {
      const int uB = u + kWaves, uA = uB + kWaves;
      const bool okB = unit_rsrc(st, nu, uB, pidB, rk, rv);
      any_bad |= uB < nu && !okB;
      if (claim && claimer) ticket = tq.fetch();
      issue(bufB, rk, rv, uB % C::UPT);
      if (uA < nu) pidA = page_of(st, uA);
      if (okA) compute(bufA, q, tok0(st, u), st.L, qk_scale, m_run, l_part, o);
      if (claim) {
        if (claimer) *tq.slot() = ticket;
        tq.want = false;
        tq.issued = true;
        claim = false;
      }
      if (uA < nu) {
        okA = unit_rsrc(st, nu, uA, pidA, rk, rv);
        any_bad |= !okA;
        if (uA + kWaves < nu) pidB = page_of(st, uA + kWaves);
        issue(bufA, rk, rv, uA % C::UPT);
      } else {
        const int nnu = more ? units(nst) : 0;
        okA = unit_rsrc(nst, nnu, wave, npid, rk, rv);
        any_bad |= wave < nnu && !okA;
        issue(bufA, rk, rv, wave % C::UPT);
      }
      if (okB) compute(bufB, q, tok0(st, uB), st.L, qk_scale, m_run, l_part, o);
      if (uA >= nu) break;
    }
    if (any_bad) report_bad_page();
    return okA;
  }

  // The 4 waves' (m, l, acc) meet in LDS; one log-sum-exp combine; the output row
  // (unsplit sequence) or a partial slot (split sequence) is written.
  __device__ void combine(const ItemState& st, float m_run, float l_part, const f32x4 (&o)[kAccRegs]) {
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if constexpr (kValuProducts) {
      if (m16 < a.group && j == 0) {
        lds.m[wave][m16] = m_run;
        lds.l[wave][m16] = l_tot;
      }
      // sum o(h, n) over the four lane groups; lane group 0 stores dim 16 n + m16 of each head
#pragma unroll
      for (int r = 0; r < kAccRegs; ++r) {
        f32x4 x = o[r];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] += __shfl_xor(x[e], 16, 64);
          x[e] += __shfl_xor(x[e], 32, 64);
        }
        const int h = r >> 1;
        if (j == 0 && h < a.group) {
#pragma unroll
          for (int e = 0; e < 4; ++e) lds.o[wave][h][16 * (4 * (r & 1) + e) + m16] = x[e];
        }
      }
    } else if (m16 < a.group) {
      if (j == 0) {
        lds.m[wave][m16] = m_run;
        lds.l[wave][m16] = l_tot;
      }
#pragma unroll
      for (int n = 0; n < 8; ++n)
        *reinterpret_cast<f32x4*>(&lds.o[wave][m16][16 * n + 4 * j]) = o[n];
    }
    __syncthreads();
    // thread t combines dims d0 .. d0 + 3 of head (t / 32) (+ 8 per pass): all of a
    // pass's LDS reads are issued before the first is used, and each output is one
    // 8-byte (bf16 row) or 16-byte (partial) store
    constexpr int kQuads = kHeadDim / 4, kHeadsPerPass = kAttnThreads / kQuads;
    const int d0 = 4 * (threadIdx.x % kQuads);
#pragma unroll
    for (int pass = 0; pass < kMaxGroup / kHeadsPerPass; ++pass) {
      const int hh = pass * kHeadsPerPass + static_cast<int>(threadIdx.x / kQuads);
      if (!st.valid || hh >= a.group) break;
      float mw[kWaves], lw[kWaves];
      f32x4 ow[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = lds.m[w][hh];
        lw[w] = lds.l[w][hh];
        ow[w] = *reinterpret_cast<const f32x4*>(&lds.o[w][hh][d0]);
      }
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
      float Ls = 0.f;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - M);   // 0 for idle waves
        Ls += f * lw[w];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += f * ow[w][e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= st.vscale;
      if (st.it.slot < 0) {
        uint2 packed;
        packed.x = f32_to_bf16_rne(acc[0] / Ls) | (uint32_t(f32_to_bf16_rne(acc[1] / Ls)) << 16);
        packed.y = f32_to_bf16_rne(acc[2] / Ls) | (uint32_t(f32_to_bf16_rne(acc[3] / Ls)) << 16);
        *reinterpret_cast<uint2*>(a.out + (int64_t(st.b) * a.hq + st.g * a.group + hh) * kHeadDim + d0) = packed;
      } else {
        const int64_t sl = st.it.slot;
        float* pa = a.part_acc + (sl * a.group + hh) * kHeadDim + d0;
        if (INMERGE) {
#pragma unroll
          for (int e = 0; e < 4; ++e) store_partial(pa + e, acc[e]);
        } else {
          *reinterpret_cast<f32x4*>(pa) = acc;
        }
        if (d0 == 0) {
          store_partial(a.part_m + sl * a.group + hh, M);
          store_partial(a.part_l + sl * a.group + hh, Ls);
        }
      }
    }
    __syncthreads();
    if (INMERGE && st.valid && st.it.slot >= 0) arrive(st);
  }

  // Partials are read by other workgroups in the in-kernel merge: there every
  // access to them is device-coherent (sc1: the compiler's agent-scope atomic
  // store here, sc1 buffer loads in arrive()), so no L2-wide write-back or
  // invalidate is ever needed.
  __device__ static void store_partial(float* p, float v) {
    if (INMERGE) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
  }

  // In-kernel merge of split sequences (fused schedule). A split's partial is
  // complete in memory before its workgroup counts itself in (wait for its own
  // stores, barrier, one device-scope atomic add on the counter of its group of
  // kMergeGroup consecutive splits). The workgroup that sees the group's last
  // arrival reduces the group's splits -- the merge kernel's group step -- and
  // either writes the output (one group) or stores the group result in the
  // group's first slot and counts the group in on the sequence's counter; the
  // workgroup that sees the last group reduces the group results block by block,
  // folds the blocks in order and writes the output. Counters are returned to 0 by
  // whoever saw the last arrival. Nothing waits on another workgroup.
  __device__ int count_in(int32_t* ctr) {
    __builtin_amdgcn_s_waitcnt(0);          // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) lds.flag = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int seen = __builtin_amdgcn_readfirstlane(lds.flag);
    __syncthreads();                        // lds.flag is reused by the next arrival
    return seen;
  }

  __device__ void write_row(const ItemState& st, int hh, int q4, float FL, const f32x4& FA) const {
    uint16_t* orow = a.out + (int64_t(st.b) * a.hq + st.g * a.group + hh) * kHeadDim + 4 * q4;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = f32_to_bf16_rne(FA[e] / FL);
  }

  __device__ void arrive(const ItemState& st) {
    const int n = st.it.nsplit, pb = st.it.pbase, G = a.group;
    const int gg = (st.it.slot - pb) / kMergeGroup;
    const int gslot = pb + gg * kMergeGroup, gsize = min(kMergeGroup, n - gg * kMergeGroup);
    const int ngrp = (n + kMergeGroup - 1) / kMergeGroup;
    if (count_in(a.gctr + gslot) != gsize - 1) return;
    if (threadIdx.x == 0) __hip_atomic_store(a.gctr + gslot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Partials are read with device-coherent (sc1) buffer loads -- what the relaxed
    // agent-scope atomic loads compile to, without their ordering: every load of a
    // reduction goes out before the first is used.
    const rsrc_t racc = make_rsrc(a.part_acc, static_cast<uint32_t>(int64_t(a.slots) * G * kHeadDim * 4));
    const rsrc_t rm = make_rsrc(a.part_m, static_cast<uint32_t>(int64_t(a.slots) * G * 4));
    const rsrc_t rl = make_rsrc(a.part_l, static_cast<uint32_t>(int64_t(a.slots) * G * 4));
    // one thread per (head, 4-dim quad)
    for (int idx = threadIdx.x; idx < G * (kHeadDim / 4); idx += kAttnThreads) {
      const int hh = idx / (kHeadDim / 4), q4 = idx % (kHeadDim / 4);
      float mk[kMergeGroup], lk[kMergeGroup];
      f32x4 ak[kMergeGroup];
#pragma unroll
      for (int i = 0; i < kMergeGroup; ++i) {
        const int64_t r = int64_t(gslot + min(i, gsize - 1)) * G + hh;   // in bounds; extra ones unused
        mk[i] = bload_f32<kPolicyAgent>(rm, static_cast<uint32_t>(r * 4));
        lk[i] = bload_f32<kPolicyAgent>(rl, static_cast<uint32_t>(r * 4));
        ak[i] = __builtin_bit_cast(f32x4, bload16<kPolicyAgent>(racc, static_cast<uint32_t>((r * kHeadDim + 4 * q4) * 4), 0));
      }
      float M, L;
      f32x4 A;
      reduce(mk, lk, ak, gsize, M, L, A);
      if (ngrp == 1) {
        // the block and fold levels over the one group result, as the merge kernel
        // takes them (its block reads copies of the one written slot)
        float bm[kMergeBlock], bl[kMergeBlock];
        f32x4 ba[kMergeBlock];
#pragma unroll
        for (int j = 0; j < kMergeBlock; ++j) {
          bm[j] = M;
          bl[j] = L;
          ba[j] = A;
        }
        float FM = -INFINITY, FL = 0.f;
        f32x4 FA = f32x4{0.f, 0.f, 0.f, 0.f};
        reduce(bm, bl, ba, 1, M, L, A);
        fold(FM, FL, FA, M, L, A);
        write_row(st, hh, q4, FL, FA);
      } else {
        const int64_t r = int64_t(gslot) * G + hh;       // the group result replaces split 0 of the group
        float* pa = a.part_acc + r * kHeadDim + 4 * q4;
#pragma unroll
        for (int e = 0; e < 4; ++e) __hip_atomic_store(pa + e, A[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (q4 == 0) {
          __hip_atomic_store(a.part_m + r, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.part_l + r, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (ngrp == 1) return;
    if (count_in(a.sctr + st.it.s) != ngrp - 1) return;
    if (threadIdx.x == 0) __hip_atomic_store(a.sctr + st.it.s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // blocks of kMergeBlock group results: loaded together, reduced, folded in order
    for (int idx = threadIdx.x; idx < G * (kHeadDim / 4); idx += kAttnThreads) {
      const int hh = idx / (kHeadDim / 4), q4 = idx % (kHeadDim / 4);
      float FM = -INFINITY, FL = 0.f;
      f32x4 FA = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int b0 = 0; b0 < ngrp; b0 += kMergeBlock) {
        float mg[kMergeBlock], lg[kMergeBlock];
        f32x4 ag[kMergeBlock];
#pragma unroll
        for (int i = 0; i < kMergeBlock; ++i) {
          const int g = min(b0 + i, ngrp - 1);                          // copies of the block's last past it
          const int64_t r = int64_t(pb + g * kMergeGroup) * G + hh;
          mg[i] = bload_f32<kPolicyAgent>(rm, static_cast<uint32_t>(r * 4));
          lg[i] = bload_f32<kPolicyAgent>(rl, static_cast<uint32_t>(r * 4));
          ag[i] = __builtin_bit_cast(f32x4, bload16<kPolicyAgent>(racc, static_cast<uint32_t>((r * kHeadDim + 4 * q4) * 4), 0));
        }
        float M, L;
        f32x4 A;
        reduce(mg, lg, ag, min(kMergeBlock, ngrp - b0), M, L, A);
        fold(FM, FL, FA, M, L, A);
      }
      write_row(st, hh, q4, FL, FA);
    }
  }

  __device__ void stamp(int k) {
    if (kTraceBuild && trec && titem < kTraceItems && lane == 0)
      trec[4 + kTraceStart + 3 * titem + k] = __builtin_amdgcn_s_memrealtime();
  }

  // start-up stamp k of the instrumented build, after all of the wave's loads so far
  __device__ void start_stamp(int k) {
    if (kTraceBuild && trec) {
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) trec[4 + k] = __builtin_amdgcn_s_memrealtime();
    }
  }

  // Walk the items a source hands out (src.next(Item&) -> bool, uniform; it only
  // issues the descriptor's loads, which are first used one item later).
  template <class Source>
  __device__ void run(Source& src) {
    using C = Cfg<FP8>;
    start_stamp(0);
    Item it;
    if (!src.next(it, tq)) return;
    start_stamp(1);
    ItemState st = open(it);
    load_q(st, q);
    int pidB = page_of(st, wave + kWaves);
    const int pid0 = page_of(st, wave);
    start_stamp(2);
    const int nu0 = units(st);
    rsrc_t rk, rv;
    bool okA = unit_rsrc(st, nu0, wave, pid0, rk, rv);
    if (wave < nu0 && !okA) report_bad_page();
    issue(bufA, rk, rv, wave % C::UPT);
    start_stamp(3);
    Item nit;
    bool more = src.next(nit, tq);
    src.fix(st.it);              // a source may settle the first item's partial slot only now
    for (;;) {
      ItemState nst{};
      int npid = -1, npidB = -1;
      if (more) {                  // prefetch: the next item's length, q and first pages
        nst = open(nit);
        load_q(nst, qn);
        npid = page_of(nst, wave);
        npidB = page_of(nst, wave + kWaves);
      }
      Item nnit;
      const bool more2 = more && src.next(nnit, tq);
      float m_run = -INFINITY, l_part = 0.f;
      f32x4 o[kAccRegs];
#pragma unroll
      for (int n = 0; n < kAccRegs; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      stamp(0);
      okA = stream(st, okA, pidB, m_run, l_part, o, more, nst, npid);
      stamp(1);
      combine(st, m_run, l_part, o);
      stamp(2);
      ++titem;
      if (!more) break;
      st = nst;
      pidB = npidB;
#pragma unroll
      for (int c = 0; c < 4; ++c) q[c] = qn[c];
      nit = nnit;
      more = more2;
    }
  }
};

// Items of worker w from the planner's work list (scalar loads; next() only
// issues them, the entry is checked when the driver opens it), then those of
// the tail chunks it claims (virtual workers Ws + c).
template <bool INMERGE = false>
struct PlanSource {
  const AttnArgs& a;
  int i, i1;
  int Ws, cap;
  bool bad = false;   // a chunk's item range did not fit the work list (reported by the caller:
                      // a one-lane branch here would make the compiler treat i as divergent)
  __device__ bool next(Item& it, TailQueue& q) {
    while (i >= i1) {
      if (!q.open()) return false;
      const int c = q.take();
      if (c < 0) return false;
      i = sload(a.plan, a.po.worker_off + Ws + c);
      i1 = sload(a.plan, a.po.worker_off + Ws + c + 1);
      if (i < 0 || i1 < i || i1 > cap) {
        bad = true;
        i1 = i;
      }
    }
    it = Item{sload(a.plan, a.po.item_s + i), sload(a.plan, a.po.item_t0 + i), sload(a.plan, a.po.item_t1 + i),
              sload(a.plan, a.po.item_slot + i), -1, 0, 0};
    if constexpr (INMERGE) {
      // the in-kernel merge needs the sequence's split count and slot base (a bad
      // sequence index is caught when the item is opened; read sequence 0 then)
      const int sq = (it.s >= 0 && it.s < a.batch * a.hkv) ? it.s : 0;
      it.nsplit = sload(a.plan, a.po.num_splits + sq);
      it.pbase = sload(a.plan, a.po.partial_base + sq);
    }
    ++i;
    if (i == i1 && q.open()) q.want = true;   // the last item held: claim the next chunk
    return true;
  }
  __device__ void fix(Item&) const {}
};

template <bool FP8, bool INMERGE>
__global__ __launch_bounds__(kAttnThreads, kAttnBlocksPerCu) void attn_balanced_kernel(AttnArgs a) {
  __shared__ CombineLds lds;
  WaveTrace tr(a);
  const int w = blockIdx.x;
  const int W = gridDim.x;
  const int Wp = sload(a.plan, a.po.header + H_WP), Ws = sload(a.plan, a.po.header + H_WS);
  const int D = sload(a.plan, a.po.header + H_ND);
  // a plan made for another launch shape (worker count, batch or KV heads) is refused
  // before any of its arrays is read: they sit at offsets that depend on that shape
  if (sload(a.plan, a.po.header + H_W) != W || sload(a.plan, a.po.header + H_B) != a.batch ||
      sload(a.plan, a.po.header + H_HKV) != a.hkv || sload(a.plan, a.po.header + H_S) != a.batch * a.hkv ||
      Wp < 0 || Wp > W || Ws < 0 || Ws > Wp || D < 0 || D > kTailChunksPerWorker * W) {
    if (w == 0 && threadIdx.x == 0) report_error(a, HPA_DEVERR_PLAN);
    return;
  }
  if constexpr (INMERGE) {
    // no merge kernel follows: empty (or invalid) sequences get their zero rows here
    const int S = a.batch * a.hkv;
    for (int s = w; s < S; s += W) {
      if (sload(a.plan, a.po.num_splits + s) == 0) {
        const int b = s / a.hkv, g = s - b * a.hkv;
        uint16_t* row = a.out + (int64_t(b) * a.hq + g * a.group) * kHeadDim;
        for (int i = threadIdx.x; i < a.group * kHeadDim; i += kAttnThreads) row[i] = 0;
      }
    }
  }
  if (w >= Wp) return;
  const int cap = (1 + kTailChunksPerWorker) * W + a.batch * a.hkv;   // the work list's size bound
  int i0 = 0, i1 = 0;
  if (w < Ws) {
    i0 = sload(a.plan, a.po.worker_off + w);
    i1 = sload(a.plan, a.po.worker_off + w + 1);
    if (i0 < 0 || i1 < i0 || i1 > cap) {
      if (threadIdx.x == 0) report_error(a, HPA_DEVERR_PLAN);
      i1 = i0;                            // still take part in the tail, so its counters return to 0
    }
  }
  PlanSource<INMERGE> src{a, i0, i1, Ws, cap};
  Worker<FP8, INMERGE> r(a, lds);
  r.trec = tr.rec;
  r.tq = TailQueue{a.qctr, lds.claim, D};
  r.run(src);
  r.tq.finish(Wp);
  if (src.bad && threadIdx.x == 0) report_error(a, HPA_DEVERR_PLAN);
  tr.units = r.units_done;
}

// One item per workgroup: chunk k of sequence s (static split-KV).
struct SingleSource {
  Item item;
  bool given;
  __device__ bool next(Item& it, TailQueue&) {
    if (given) return false;
    given = true;
    it = item;
    return true;
  }
  __device__ void fix(Item&) const {}
};

template <bool FP8>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_static_kernel(AttnArgs a) {
  __shared__ CombineLds lds;
  WaveTrace tr(a);
  const int s = blockIdx.x / a.static_splits, k = blockIdx.x - s * a.static_splits;
  const int b = s / a.hkv;
  int L = a.seq_lens[b];
  if (L < 0 || L > a.max_pages * kPage) {
    if (k == 0 && threadIdx.x == 0 && a.err) report_error(a, HPA_DEVERR_SEQ_LEN);
    return;
  }
  const int n = (L + kPage - 1) / kPage;
  if (n == 0) return;
  const int chunk = a.static_chunk > 0 ? a.static_chunk : (n + a.static_splits - 1) / a.static_splits;
  const int t0 = k * chunk, t1 = min(n, t0 + chunk);
  if (t0 >= t1) return;
  const int nchunks = (n + chunk - 1) / chunk;
  SingleSource src{Item{s, t0, t1, nchunks > 1 ? s * a.static_splits + k : -1, L, 0, 0}, false};
  Worker<FP8> r(a, lds);
  r.trec = tr.rec;
  r.run(src);
  tr.units = r.units_done;
}

// ---- fused schedule: the planner's closed forms evaluated inside the persistent kernel ----
// Each workgroup recomputes the position prefix sum C (tiles plus item_cost
// virtual tiles per non-empty sequence) and the partial-slot bases PB from
// seq_lens in LDS (the same integer arithmetic as plan_kernel, so the items and
// slots are identical), then walks its own range. The worker holding split 0
// of a sequence records (num_splits, partial_base) for the merge kernel.
struct FusedPlanLds {
  int C[kFusedMaxSeqs + 1];
  int PB[kFusedMaxSeqs];
  int L[kFusedMaxSeqs];       // live length of each sequence's request (0 if invalid)
  int tot[kFusedMaxSeqs / 64];
};

// Exclusive-scan the per-chunk totals P.tot[0..nch) and add each chunk's offset to
// arr[chunk * 64 + lane] for the chunks this wave owns; returns the grand total.
__device__ inline int add_chunk_offsets(FusedPlanLds& P, int* arr, int S, int nch, int lane, int wave) {
  const int t = lane < nch ? P.tot[lane] : 0;
  const int xi = wave_incl_scan(t);
  const int total = __builtin_amdgcn_readfirstlane(__shfl(xi, 63, 64));   // same in every lane
  const int off = xi - t;
  for (int ch = wave; ch < nch; ch += kWaves) {
    const int o = __shfl(off, ch, 64);
    const int s = ch * 64 + lane;
    if (s < S) arr[s] += o;
  }
  return total;
}

// The fused schedules always plan with the library's fixed parameters: as
// compile-time constants the partition's divisions by them become multiplies
// and the tail code (no tail) drops out.
constexpr int kFusedCost = HPA_FUSED_ITEM_COST;
constexpr int kFusedMinTiles = HPA_FUSED_MIN_TILES;
constexpr int kFusedTailDen = HPA_FUSED_TAIL_DEN;
constexpr int kFusedTailChunk = HPA_FUSED_TAIL_CHUNK;

template <bool INMERGE>
struct FusedSource {
  const AttnArgs& a;
  FusedPlanLds& P;
  Partition part;
  int S;
  int v;                      // the virtual worker whose positions [pos, e) are being walked
  int pos, e, s;
  // First item served from the register plan (no LDS read, no barrier, no division
  // before its loads): sequence s, positions [r0, c1) of it, [lo, t1) its part; its
  // split rank and split count are settled by fix().
  bool reg_first = false;
  int rf_c0 = 0, rf_c1 = 0, rf_lo = 0, rf_t1 = 0, rf_L = 0;
  bool split_later = false;
  // Register plan: the partial-slot bases P.PB are not in LDS yet when the first item is
  // handed out. They are computed (wave 0) and published, with one barrier, on the
  // second call, i.e. behind the first unit's loads; fix() then settles the first
  // item's slot (kSlotLater until then) and its record for the merge kernel.
  bool pb_ready = true;
  bool first_later = false;   // the first item's slot and record wait for fix()
  int calls = 0;
  int first_split = 0;
  __device__ void publish_pb(int lane, int wave) {
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < S; base += 64) {
        const int sq = base + lane;
        int val = 0;
        if (sq < S) {
          const int c0 = P.C[sq], c1 = P.C[sq + 1];
          if (c1 > c0) {
            const int ns = part.owner(c1 - 1) - part.owner(c0 + kFusedCost) + 1;
            val = ns > 1 ? ns : 0;
          }
        }
        const int incl = wave_incl_scan(val);
        if (sq < S) P.PB[sq] = carry + incl - val;
        carry += __builtin_amdgcn_readlane(incl, 63);
      }
    }
    __syncthreads();
    pb_ready = true;
  }
  __device__ void fix(Item& it) {
    if (!first_later) return;
    first_later = false;
    if (split_later) {        // the register-served first item: its split rank and count now
      split_later = false;
      const int first = __builtin_amdgcn_readfirstlane(part.owner(rf_c0 + kFusedCost));
      first_split = v - first;
      it.nsplit = __builtin_amdgcn_readfirstlane(part.owner(rf_c1 - 1)) - first + 1;
      if (it.nsplit <= 1) it.slot = -1;
    }
    const int pb = __builtin_amdgcn_readfirstlane(P.PB[it.s]);
    if (it.nsplit > 1) it.slot = pb + first_split;
    it.pbase = pb;
    if (!INMERGE && first_split == 0 && threadIdx.x == 0) {   // record for the merge kernel
      a.plan[a.po.num_splits + it.s] = it.nsplit;
      a.plan[a.po.partial_base + it.s] = pb;
    }
  }
  // positions [C[s], C[s+1]) of a non-empty sequence: item_cost virtual ones, then its tiles
  __device__ bool next(Item& it, TailQueue& q) {
    if (!pb_ready && calls > 0) publish_pb(threadIdx.x & 63, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    if (calls++ == 0 && reg_first) {
      // a split item's slot is only known once the bases are: an in-range placeholder
      // until fix() (nothing reads it before); a single item's slot becomes -1 there
      it = Item{s, rf_lo - rf_c0 - kFusedCost, rf_t1 - rf_c0 - kFusedCost, 0, rf_L, 0, -1};
      first_later = split_later = true;
      pos = rf_t1;
      if (pos + kFusedCost >= e && q.open()) q.want = true;
      ++s;
      return true;
    }
    for (;;) {
      while (pos < e) {
        const int c0 = __builtin_amdgcn_readfirstlane(P.C[s]);
        const int c1 = __builtin_amdgcn_readfirstlane(P.C[s + 1]);
        if (c1 > c0) {
          const int r0 = c0 + kFusedCost;
          const int t1 = min(e, c1), lo = max(pos, r0);
          pos = t1;
          if (lo < t1) {
            const int first = __builtin_amdgcn_readfirstlane(part.owner(r0));
            const int split = v - first;
            const int ns = __builtin_amdgcn_readfirstlane(part.owner(c1 - 1)) - first + 1;
            if (!pb_ready) {          // only the first item: its slot is settled by fix()
              first_split = split;
              first_later = true;
              // a split item's slot is only known once the bases are: an in-range
              // placeholder until fix() (nothing reads it before)
              it = Item{s, lo - r0, t1 - r0, ns > 1 ? 0 : -1, __builtin_amdgcn_readfirstlane(P.L[s]), ns, -1};
              if (pos + kFusedCost >= e && q.open()) q.want = true;
              ++s;
              return true;
            }
            const int pb = __builtin_amdgcn_readfirstlane(P.PB[s]);
            it = Item{s, lo - r0, t1 - r0, ns > 1 ? pb + split : -1, __builtin_amdgcn_readfirstlane(P.L[s]), ns, pb};
            // the last item held: claim the next chunk (the next sequence's tiles start
            // item_cost positions after this item's end). Set before the one-lane store
            // below: after it, the compiler takes the flag, and with it the item
            // index, for divergent and reads the page table with vector loads.
            if (pos + kFusedCost >= e && q.open()) q.want = true;
            if (!INMERGE && split == 0 && threadIdx.x == 0) {   // record for the merge kernel
              a.plan[a.po.num_splits + s] = ns;
              a.plan[a.po.partial_base + s] = pb;
            }
            ++s;
            return true;
          }
        }
        ++s;
      }
      if (!q.open()) return false;
      const int c = q.take();
      if (c < 0) return false;
      v = part.Ws + c;
      pos = part.begin(v);
      e = part.begin(v + 1);
      s = __builtin_amdgcn_readfirstlane(seq_of_tile(P.C, S, pos));
    }
  }
};

// Register planner for batches of up to kRegPlanSeqs sequences: every wave
// evaluates the per-sequence prefix sums by itself (lane l of chunk k holds
// sequence 64k + l; DPP scans, no LDS, no barrier); wave 0 then publishes them
// to LDS. Same integer arithmetic as plan_kernel; C holds positions (tiles plus
// item_cost virtual tiles per non-empty sequence), N their total. The partial-slot
// bases are left to FusedSource, off the path to the first K/V loads.
constexpr int kRegPlanChunks = kRegPlanSeqs / 64;

struct RegPlan {
  int L[kRegPlanChunks], C[kRegPlanChunks], n[kRegPlanChunks];
  int N;
  Partition part;
  bool bad;

  // chunks at or past S (a uniform test) are skipped whole: their lanes would hold
  // no sequence, and nothing reads them
  __device__ void build(const AttnArgs& a, const int32_t* seq_lens, int hkv, int S, int W, int lane) {
    int carry = 0;
    bool bad_lane = false;
    // every chunk's lengths are requested before the first is used (one round trip);
    // lanes past S read the last sequence's length (in bounds, S >= 1) and drop it
    int Lraw[kRegPlanChunks];
#pragma unroll
    for (int k = 0; k < kRegPlanChunks; ++k) {
      const int s = min(64 * k + lane, S - 1);
      Lraw[k] = seq_lens[hkv == 1 ? s : s / hkv];
    }
#pragma unroll
    for (int k = 0; k < kRegPlanChunks; ++k) {
      L[k] = n[k] = C[k] = 0;
      if (64 * k >= S) continue;
      const int s = 64 * k + lane;
      int Lk = 0;
      if (s < S) {
        Lk = Lraw[k];
        if (Lk < 0 || Lk > a.max_pages * kPage) {
          bad_lane = true;
          Lk = 0;
        }
      }
      L[k] = Lk;
      n[k] = tiles_of(Lk);
      const int np = n[k] > 0 ? n[k] + kFusedCost : 0;   // positions: virtual tiles first
      const int incl = wave_incl_scan(np);
      C[k] = carry + incl - np;
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    N = carry;
    part = Partition::make(N, N, W, kFusedMinTiles, kFusedTailDen, kFusedTailChunk);
    bad = __builtin_amdgcn_ballot_w64(bad_lane) != 0;
  }
};

// seq_lens, batch and hkv also lead the argument list as scalars, which are preloaded
// into SGPRs at dispatch (struct arguments are not): the lengths, the first loads of
// the launch, do not wait for the argument block.
template <bool FP8, bool INMERGE>
__global__ __launch_bounds__(kAttnThreads, kAttnBlocksPerCu) void attn_fused_kernel(const int32_t* seq_lens, int batch,
                                                                                  int hkv, AttnArgs a) {
  __shared__ CombineLds lds;
  __shared__ FusedPlanLds P;
  WaveTrace tr(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int S = batch * hkv, nch = (S + 63) / 64;
  const int W = gridDim.x, w = blockIdx.x;
  int N, bad, pos = 0, pend = 0, s0 = 0;
  Partition part;
  // register plan: the first item, read straight from the registers (rf_*), and
  // whether the LDS copy of the plan may be read before the next barrier (no)
  bool reg_first = false, lds_ready = true;
  int rf_c0 = 0, rf_c1 = 0, rf_lo = 0, rf_t1 = 0, rf_L = 0;
  if (S <= kRegPlanSeqs) {
    RegPlan R;
    R.build(a, seq_lens, hkv, S, W, lane);
    N = R.N;
    part = R.part;
    bad = R.bad;
    // lane value x of sequence q (wave-uniform q < S): chunk q / 64, lane q % 64
    auto at = [&](const int (&x)[kRegPlanChunks], int q) {
      int v = 0;
#pragma unroll
      for (int k = 0; k < kRegPlanChunks; ++k)
        if (64 * k < S && (q >> 6) == k) v = __builtin_amdgcn_readlane(x[k], q & 63);
      return v;
    };
    if (w < part.Ws) {
      // this worker's static positions and the sequence holding the first one (largest
      // s with C[s] <= pos: C is non-decreasing, so count the lanes at or below pos)
      pos = __builtin_amdgcn_readfirstlane(part.begin(w));
      pend = __builtin_amdgcn_readfirstlane(part.begin(w + 1));
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < kRegPlanChunks; ++k)
        if (64 * k < S) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(64 * k + lane < S && R.C[k] <= pos));
      s0 = cnt - 1;
      // pos lies in [C[s0], C[s0+1]): s0 is non-empty; its real tiles are the positions
      // [C[s0] + cost, C[s0+1]); the first item is their part inside [pos, pend) if any
      rf_c0 = at(R.C, s0);
      const int n0 = at(R.n, s0);
      rf_c1 = rf_c0 + (n0 > 0 ? n0 + kFusedCost : 0);
      rf_lo = max(pos, rf_c0 + kFusedCost);
      rf_t1 = min(pend, rf_c1);
      rf_L = at(R.L, s0);
      reg_first = rf_lo < rf_t1;
    }
    // empty (or invalid) sequences own no tile: their zero rows are spread over the workers
    for (int q = w; q < S; q += W) {
      if (at(R.n, q) == 0) {
        const int b = q / a.hkv, g = q - b * a.hkv;
        uint16_t* row = a.out + (int64_t(b) * a.hq + g * a.group) * kHeadDim;
        for (int i = threadIdx.x; i < a.group * kHeadDim; i += kAttnThreads) row[i] = 0;
      }
    }
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < kRegPlanChunks; ++k) {
        const int s = 64 * k + lane;
        if (s < S) {
          P.C[s] = R.C[k];
          P.L[s] = R.L[k];
        }
      }
      if (lane == 0) P.C[S] = N;
    }
    // The other waves read this LDS copy only after the barrier the source takes on its
    // second call (behind the first unit's loads), or right here if the first item is
    // not served from registers.
    lds_ready = false;
    if (!reg_first) {
      __syncthreads();
      lds_ready = true;
    }
  } else {
    // tile counts and their chunk-local exclusive prefix sums
    bad = 0;
    for (int ch = wave; ch < nch; ch += kWaves) {
      const int s = ch * 64 + lane;
      int n = 0;
      if (s < S) {
        int L = seq_lens[s / hkv];
        if (L < 0 || L > a.max_pages * kPage) {
          bad = 1;
          L = 0;
        }
        n = tiles_of(L);
        if (n > 0) n += kFusedCost;                  // positions: virtual tiles first
        P.L[s] = L;
      }
      const int x = wave_incl_scan(n);
      if (s < S) P.C[s] = x - n;
      if (lane == 63) P.tot[ch] = x;
    }
    bad = __builtin_amdgcn_readfirstlane(__syncthreads_or(bad));
    N = add_chunk_offsets(P, P.C, S, nch, lane, wave);
    if (threadIdx.x == 0) P.C[S] = N;
    __syncthreads();
    part = Partition::make(N, N, W, kFusedMinTiles, kFusedTailDen, kFusedTailChunk);
    // partial-slot bases: exclusive prefix of (num_splits > 1 ? num_splits : 0)
    for (int ch = wave; ch < nch; ch += kWaves) {
      const int s = ch * 64 + lane;
      int v = 0;
      if (s < S) {
        const int c0 = P.C[s], c1 = P.C[s + 1];
        if (c1 > c0) {
          const int ns = part.owner(c1 - 1) - part.owner(c0 + kFusedCost) + 1;
          v = ns > 1 ? ns : 0;
        }
      }
      const int x = wave_incl_scan(v);
      if (s < S) P.PB[s] = x - v;
      if (lane == 63) P.tot[ch] = x;
    }
    __syncthreads();
    add_chunk_offsets(P, P.PB, S, nch, lane, wave);
    __syncthreads();
    if (w < part.Ws) {
      pos = __builtin_amdgcn_readfirstlane(part.begin(w));
      pend = __builtin_amdgcn_readfirstlane(part.begin(w + 1));
      s0 = __builtin_amdgcn_readfirstlane(seq_of_tile(P.C, S, pos));
    }
  }
  if (w == 0 && threadIdx.x == 0 && bad && a.err) report_error(a, HPA_DEVERR_SEQ_LEN);
  if (S > kRegPlanSeqs) {
    // empty (or invalid) sequences own no tile: their zero rows are spread over the workers
    for (int s = w; s < S; s += W) {
      if (P.C[s + 1] == P.C[s]) {
        const int b = s / a.hkv, g = s - b * a.hkv;
        uint16_t* row = a.out + (int64_t(b) * a.hq + g * a.group) * kHeadDim;
        for (int i = threadIdx.x; i < a.group * kHeadDim; i += kAttnThreads) row[i] = 0;
      }
    }
  }
  if (w >= part.Wp) return;
  // workers without a static range go straight to the tail chunks
  FusedSource<INMERGE> src{a, P, part, S, w, pos, pend, __builtin_amdgcn_readfirstlane(s0)};
  src.pb_ready = S > kRegPlanSeqs;     // the register plan leaves the partial-slot bases for later
  src.reg_first = reg_first;
  src.rf_c0 = rf_c0;
  src.rf_c1 = rf_c1;
  src.rf_lo = rf_lo;
  src.rf_t1 = rf_t1;
  src.rf_L = rf_L;
  (void)lds_ready;
  Worker<FP8, INMERGE> r(a, lds);
  r.trec = tr.rec;
  r.tq = TailQueue{a.qctr, lds.claim, part.D};
  r.run(src);
  r.tq.finish(part.Wp);
  tr.units = r.units_done;
}

// Merge: block (s, h) combines the 128 dims of head h of sequence s; blocks of
// unsplit sequences return at once. THREADS = 32 dim-quads x LANES lane groups:
// lane group j reduces split groups j, j + LANES, ... (16 consecutive splits each,
// max-first), lane group 0 reduces each block of 16 group results the same way and
// folds the block results in order, so every schedule's partials combine with the
// same arithmetic in the same order, whatever the block size. Empty sequences get a
// zero row. Grids of at most one block per CU take 256 threads and issue two
// passes' loads together (a long sequence's many splits in one round trip); larger
// grids take 128 threads (measured: on 1024 blocks the merge takes 3.7 instead of
// 5.5 µs, on 256 blocks 6.0 instead of 4.4; 512 threads on 256 blocks, one pass for
// up to 256 splits: 4.0 instead of 3.6).
constexpr int kMergeDims = kHeadDim;   // head dims per merge block (splitting them measured slower:
                                       // the merge is bound by dispatch and round trips, not bytes)
constexpr int kMergeQuads = kMergeDims / 4;

// The merge kernel's own arguments: everything it reads, in two 64-byte lines, so
// the launch arguments cost one round trip.
struct MergeArgs {
  const int32_t* seq_lens;
  const int32_t* plan;
  const float* part_acc;
  const float* part_m;
  const float* part_l;
  uint16_t* out;
  int num_splits, partial_base, header;   // plan offsets (int32 words)
  int hkv, hq, group, max_pages, workers;
  int slots, static_splits, static_chunk;
  int batch;
};

// The arrays and offsets the first loads need also lead the argument list as scalars:
// leading scalar arguments are preloaded into SGPRs at dispatch (struct arguments are
// not), so the metadata loads do not wait for the argument block.
// TWO: the first two passes' loads go out together (a second register set: fewer
// blocks per CU, so it is launched only when the grid has at most one block per CU).
template <MergeMode MODE, bool TWO>
__global__ __launch_bounds__(TWO ? 256 : 128) void merge_kernel(const int32_t* seq_lens, const int32_t* plan,
                                                                const float* part_acc, const float* part_m,
                                                                const float* part_l, int hkv, int off_splits,
                                                                int off_base, MergeArgs a) {
  constexpr int kMergeThreads = TWO ? 256 : 128;
  constexpr int kMergeLanes = kMergeThreads / kMergeQuads;
  __shared__ float gm[kMergeBlock], gl[kMergeBlock];
  __shared__ f32x4 gacc[kMergeBlock][kMergeQuads];
  const int hh = blockIdx.y, d0 = blockIdx.z * kMergeDims;
  const int s = blockIdx.x;
  // every fact this block needs is one scalar load away from its sequence index,
  // and all of those loads go out together
  const int L = sload(seq_lens, s / hkv);
  int n = 0, base = 0, planned_w = a.workers, planned_b = a.batch, planned_hkv = hkv;
  if constexpr (MODE != MERGE_STATIC) {
    n = sload(plan, off_splits + s);
    base = sload(plan, off_base + s);
    if constexpr (MODE == MERGE_PLAN) {
      planned_w = sload(plan, a.header + H_W);
      planned_b = sload(plan, a.header + H_B);
      planned_hkv = sload(plan, a.header + H_HKV);
    }
  }
  if constexpr (MODE == MERGE_STATIC) {
    if (L < 0 || L > a.max_pages * kPage) return;
    const int nt = (L + kPage - 1) / kPage;
    const int chunk = nt == 0 ? 1 : (a.static_chunk > 0 ? a.static_chunk : (nt + a.static_splits - 1) / a.static_splits);
    n = (nt + chunk - 1) / chunk;
    base = s * a.static_splits;
  }
  // One test on all loaded values (bitwise, not short-circuit), so that all three
  // loads are issued before the first wait. Fused schedule: zero rows of empty
  // requests were written by the attention kernel, the others read the split count
  // and slot base recorded by their split-0 worker. Planned: skip a plan made for
  // another launch shape.
  bool skip = (n == 1) | (n < 0) | ((n > 1) & ((base < 0) | (base + n > a.slots)));
  if constexpr (MODE == MERGE_FUSED) skip |= (L <= 0) | (L > a.max_pages * kPage);
  if constexpr (MODE == MERGE_PLAN) skip |= (planned_w != a.workers) | (planned_b != a.batch) | (planned_hkv != hkv);
  if (skip) return;
  const int b = s / a.hkv, g = s - b * a.hkv;
  uint16_t* orow = a.out + (int64_t(b) * a.hq + g * a.group + hh) * kHeadDim + d0;
  const int tid = threadIdx.x;
  if (n == 0) {
    if (tid < kMergeDims) orow[tid] = 0;
    return;
  }
  const int q4 = tid % kMergeQuads, lj = tid / kMergeQuads;
  const int G = a.group;
  const int ngrp = (n + kMergeGroup - 1) / kMergeGroup;
  float FM = -INFINITY, FL = 0.f;
  f32x4 FA = f32x4{0.f, 0.f, 0.f, 0.f};
  // A group's loads all go out before its reduction.
  struct GroupLoads {
    float m[kMergeGroup], l[kMergeGroup];
    f32x4 acc[kMergeGroup];
  };
  auto load_group = [&](GroupLoads& gs, int gg) {
    if (gg >= ngrp) return;          // lane groups past the last group load nothing
    const int k0 = gg * kMergeGroup, k1 = min(n, k0 + kMergeGroup);
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i) {
      const int64_t r = (int64_t(base) + min(k0 + i, k1 - 1)) * G + hh;   // in bounds; copies of the last past k1
      gs.m[i] = part_m[r];
      gs.l[i] = part_l[r];
      gs.acc[i] = *reinterpret_cast<const f32x4*>(part_acc + r * kHeadDim + d0 + 4 * q4);
    }
  };
  // one pass: every lane group reduces its group g0 + lj into the group's LDS slot;
  // a pass that completes a block of kMergeBlock groups (or the last group) is
  // followed by lane group 0 reducing the block and folding it into the result
  auto group_pass = [&](const GroupLoads& gs, int g0) {
    const int gg = g0 + lj;
    if (gg < ngrp) {
      float M, L;
      f32x4 A;
      reduce(gs.m, gs.l, gs.acc, min(kMergeGroup, n - gg * kMergeGroup), M, L, A);
      const int slot = gg % kMergeBlock;
      if (q4 == 0) {
        gm[slot] = M;
        gl[slot] = L;
      }
      gacc[slot][q4] = A;
    }
    const int gend = g0 + kMergeLanes;            // uniform
    if (gend % kMergeBlock == 0 || gend >= ngrp) {
      __syncthreads();
      if (lj == 0) {
        const int b0 = g0 / kMergeBlock * kMergeBlock, bcnt = min(kMergeBlock, ngrp - b0);
        float bm[kMergeBlock], bl[kMergeBlock];
        f32x4 ba[kMergeBlock];
#pragma unroll
        for (int j = 0; j < kMergeBlock; ++j) {
          const int jj = min(j, bcnt - 1);         // written slots only
          bm[j] = gm[jj];
          bl[j] = gl[jj];
          ba[j] = gacc[jj][q4];
        }
        float M, L;
        f32x4 A;
        reduce(bm, bl, ba, bcnt, M, L, A);
        fold(FM, FL, FA, M, L, A);
      }
      __syncthreads();
    }
  };
  static_assert(kMergeBlock % kMergeLanes == 0, "a pass never straddles two blocks");
  // TWO: the first two passes' loads go out together (up to 256 splits: one round trip)
  GroupLoads ga, gb;
  const bool two = TWO && ngrp > kMergeLanes;   // uniform
  load_group(ga, lj);
  if (two) load_group(gb, kMergeLanes + lj);
  group_pass(ga, 0);
  if (two) group_pass(gb, kMergeLanes);
  for (int g0 = (two ? 2 : 1) * kMergeLanes; g0 < ngrp; g0 += kMergeLanes) {
    load_group(ga, g0 + lj);
    group_pass(ga, g0);
  }
  if (lj == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[4 * q4 + e] = f32_to_bf16_rne(FA[e] / FL);
  }
}

}  // namespace

int attn_blocks_per_cu(bool fp8) {
  int nb = 0, nf = 0;
  hipError_t e = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_balanced_kernel<true, false>, kAttnThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_balanced_kernel<false, false>, kAttnThreads, 0);
  int nm = 0;
  hipError_t h = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nm, attn_balanced_kernel<true, true>, kAttnThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nm, attn_balanced_kernel<false, true>, kAttnThreads, 0);
  hipError_t f = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nf, attn_fused_kernel<true, false>, kAttnThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nf, attn_fused_kernel<false, false>, kAttnThreads, 0);
  int ns = 0;
  hipError_t g = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&ns, attn_fused_kernel<true, true>, kAttnThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&ns, attn_fused_kernel<false, true>, kAttnThreads, 0);
  if (e != hipSuccess || f != hipSuccess || g != hipSuccess || h != hipSuccess || nb <= 0 || nf <= 0 || ns <= 0 ||
      nm <= 0)
    return 1;
  return std::min(std::min(nb, nm), std::min(nf, ns));
}

int attn_static_blocks_per_cu(bool fp8) {
  int n = 0;
  hipError_t e = fp8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_static_kernel<true>, kAttnThreads, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_static_kernel<false>, kAttnThreads, 0);
  return (e != hipSuccess || n <= 0) ? 1 : n;
}

hipError_t launch_attn_balanced(const AttnArgs& a, bool fp8, bool merge_in_kernel, int num_workers,
                                hipStream_t stream) {
  if (fp8 && merge_in_kernel)
    hipLaunchKernelGGL((attn_balanced_kernel<true, true>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a);
  else if (fp8)
    hipLaunchKernelGGL((attn_balanced_kernel<true, false>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a);
  else if (merge_in_kernel)
    hipLaunchKernelGGL((attn_balanced_kernel<false, true>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_balanced_kernel<false, false>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a);
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

hipError_t launch_attn_fused(const AttnArgs& a, bool fp8, bool merge_in_kernel, int num_workers, hipStream_t stream) {
  if (fp8 && merge_in_kernel)
    hipLaunchKernelGGL((attn_fused_kernel<true, true>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a.seq_lens, a.batch, a.hkv, a);
  else if (fp8)
    hipLaunchKernelGGL((attn_fused_kernel<true, false>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a.seq_lens, a.batch, a.hkv, a);
  else if (merge_in_kernel)
    hipLaunchKernelGGL((attn_fused_kernel<false, true>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a.seq_lens, a.batch, a.hkv, a);
  else
    hipLaunchKernelGGL((attn_fused_kernel<false, false>), dim3(num_workers), dim3(kAttnThreads), 0, stream, a.seq_lens, a.batch, a.hkv, a);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, MergeMode mode, hipStream_t stream) {
  const int S = a.batch * a.hkv;
  if (S == 0) return hipSuccess;
  const MergeArgs m{a.seq_lens, a.plan, a.part_acc, a.part_m, a.part_l, a.out,
                    a.po.num_splits, a.po.partial_base, a.po.header,
                    a.hkv, a.hq, a.group, a.max_pages, a.workers,
                    static_cast<int>(a.slots), a.static_splits, a.static_chunk, a.batch};
  const dim3 grid(S, a.group, kHeadDim / kMergeDims);
  const bool two = int64_t(S) * a.group <= a.workers;   // at most one block per worker (CU)
  if (mode == MERGE_PLAN)
    hipLaunchKernelGGL((two ? merge_kernel<MERGE_PLAN, true> : merge_kernel<MERGE_PLAN, false>), grid, dim3(two ? 256 : 128), 0,
                       stream, m.seq_lens, m.plan, m.part_acc, m.part_m, m.part_l, m.hkv, m.num_splits, m.partial_base, m);
  else if (mode == MERGE_FUSED)
    hipLaunchKernelGGL((two ? merge_kernel<MERGE_FUSED, true> : merge_kernel<MERGE_FUSED, false>), grid, dim3(two ? 256 : 128), 0,
                       stream, m.seq_lens, m.plan, m.part_acc, m.part_m, m.part_l, m.hkv, m.num_splits, m.partial_base, m);
  else
    hipLaunchKernelGGL((two ? merge_kernel<MERGE_STATIC, true> : merge_kernel<MERGE_STATIC, false>), grid, dim3(two ? 256 : 128), 0,
                       stream, m.seq_lens, m.plan, m.part_acc, m.part_m, m.part_l, m.hkv, m.num_splits, m.partial_base, m);
  return hipGetLastError();
}

}  // namespace hpa

// Internal declarations of the fused FP8 MoE layer (moe.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "hpa.h"

namespace hpa {

constexpr int kMoeMaxHidden = 4096;      // H: multiple of 128 (one token row quantised in LDS)
constexpr int kMoeMaxInter = 4096;       // I: multiple of 128
constexpr int kMoeMaxTokens = 1024;      // decode batches
constexpr int kMoeMaxTopK = 16;
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxPairs = 16384;      // tokens x top_k

struct MoeArgs {
  const uint16_t* x;       // [T][H] bf16 bits
  const int32_t* ids;      // [T][K]
  const float* wts;        // [T][K]
  const uint8_t* w1;       // [E][2I][H] E4M3
  const float* s1;         // [E][2I]
  const uint8_t* w2;       // [E][H][I] E4M3
  const float* s2;         // [E][H]
  uint8_t* x8;             // [T][H] the tokens' E4M3 codes
  float* sx;               // [T] their scales
  int32_t* list;           // [P] pairs grouped by expert, each group in pair order
  int32_t* blk;            // [3][P] pair blocks of up to 16 pairs: expert, first list index, count
  int32_t* nblk;           // [1] number of pair blocks
  float* act;              // [P][I] fp32 SwiGLU output
  float* amax;             // [P][I / 16] largest |act| of each 16-wide slice
  uint8_t* act8;           // [P][I] requantised activations
  float* sa;               // [P] their scales
  float* ybuf;             // [P][H] fp32 weighted Down output of each pair
  uint16_t* out;           // [T][H] bf16
  int32_t* err;            // sticky device error word (may be null)
  int T, E, K, H, I, P, BMAX;
};

// Workspace arrays (byte offsets, 256-byte aligned).
struct MoeWorkspace {
  size_t x8, sx, list, blk, nblk, act, amax, act8, sa, ybuf, total;
};

inline MoeWorkspace moe_workspace(int64_t T, int64_t K, int64_t H, int64_t I) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t P = static_cast<size_t>(T * K);
  MoeWorkspace w{};
  size_t o = 0;
  w.x8 = o;   o += al(T * H);
  w.sx = o;   o += al(T * 4);
  w.list = o; o += al(P * 4);
  w.blk = o;  o += al(3 * P * 4);
  w.nblk = o; o += al(4);
  w.act = o;  o += al(P * I * 4);
  w.amax = o; o += al(P * (I / 16) * 4);
  w.act8 = o; o += al(P * I);
  w.sa = o;   o += al(P * 4);
  w.ybuf = o; o += al(P * H * 4);
  w.total = o;
  return w;
}

hpa_status moe_check_shape(int32_t tokens, int32_t experts, int32_t top_k, int32_t hidden, int32_t inter);
hipError_t launch_moe(const MoeArgs& a, hipStream_t stream);

}  // namespace hpa

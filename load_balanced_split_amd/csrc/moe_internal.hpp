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
  float* act;              // [P][I] fp32 SwiGLU output
  float* amax;             // [P][I / 64] largest |act| of each 64-wide slice
  float* ybuf;             // [P][H] fp32 weighted Down output of each pair
  uint16_t* out;           // [T][H] bf16
  int32_t* err;            // sticky device error word (may be null)
  int T, E, K, H, I, P, PB, IT, HT;
};

struct MoeWorkspace {
  size_t act, amax, ybuf, total;
};

inline MoeWorkspace moe_workspace(int64_t T, int64_t K, int64_t H, int64_t I) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t P = static_cast<size_t>(T * K);
  MoeWorkspace w{};
  w.act = 0;
  w.amax = al(P * I * 4);
  w.ybuf = w.amax + al(P * (I / 64) * 4);
  w.total = w.ybuf + al(P * H * 4);
  return w;
}

hpa_status moe_check_shape(int32_t tokens, int32_t experts, int32_t top_k, int32_t hidden, int32_t inter);
hipError_t launch_moe(const MoeArgs& a, hipStream_t stream);

}  // namespace hpa

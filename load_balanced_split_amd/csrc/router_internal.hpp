// Internal declarations of the split-precision router GEMM (router.hip, router_host.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "hpa.h"

namespace hpa {

// Split-precision router GEMM (router.hip). The decomposition is a pure function
// of the shape, so the workspace size query and the launch agree.
constexpr int kRouterMaxExperts = 1024;
constexpr int kRouterMaxTopK = 32;
constexpr int kRouterMaxHidden = 1 << 16;
constexpr int kRouterMaxTokens = 1 << 20;
constexpr int kRouterTargetWaves = 4096;   // 4 per SIMD of 256 compute units
constexpr int kRouterTiledMinTokens = 256; // above this, LDS-staged 128 x 128 tiles
constexpr int kRouterTiledTargetWgs = 512; // two such workgroups per compute unit
constexpr int kRouterWaveTopkMinTokens = 512;  // above this, one wave (not one workgroup) per token's top-k
struct RouterPlan {
  int me, nt;            // 16-expert blocks and 16-token blocks per wave
  int wx;                // 1: a workgroup's 4 waves take 4 expert groups of one K range (they
                         // share the token fragments through L1); 0: 4 K ranges of one tile
                         // (added in LDS)
  int tiled;             // 1: 128-expert x 128-token workgroup tiles staged through LDS
                         // (many tokens; n_eg, n_tg then count such tiles)
  int kw;                // 32-dim k-chunks per K range
  int n_eg, n_tg;        // expert groups (me blocks) and token groups (nt blocks)
  int partial_slots;     // partial sums per logit
  int64_t workgroups;
  static RouterPlan make(int tokens, int experts, int hidden) {
    RouterPlan p{};
    const int neb = experts / 16, nkc = hidden / 32;
    p.nt = tokens <= 16 ? 1 : 4;
    p.me = tokens > 64 && neb % 2 == 0 ? 2 : 1;
    p.n_eg = neb / p.me;
    p.n_tg = (tokens + 16 * p.nt - 1) / (16 * p.nt);
    p.wx = tokens > 64 && p.n_eg % 4 == 0 ? 1 : 0;
    if (tokens > kRouterTiledMinTokens && experts % 128 == 0) {
      p.tiled = 1;
      p.wx = 0;
      p.n_eg = experts / 128;
      p.n_tg = (tokens + 127) / 128;
      const int64_t t = int64_t(p.n_eg) * p.n_tg;
      int64_t ranges = (kRouterTiledTargetWgs + t - 1) / t;
      ranges = std::min<int64_t>(std::max<int64_t>(ranges, 1), std::max(1, nkc / 8));
      p.kw = static_cast<int>((nkc + ranges - 1) / ranges);
      p.partial_slots = static_cast<int>(ranges);
      p.workgroups = t * ranges;
      return p;
    }
    const int64_t tiles = int64_t(p.n_eg) * p.n_tg;
    if (p.wx) {
      // workgroups of 4 expert groups; enough K ranges for ~2 workgroups per compute unit
      const int64_t wg_tiles = tiles / 4;
      int64_t ranges = (kRouterTargetWaves / 8 + wg_tiles - 1) / wg_tiles;
      ranges = std::min<int64_t>(std::max<int64_t>(ranges, 1), std::max(1, nkc / 8));
      p.kw = static_cast<int>((nkc + ranges - 1) / ranges);
      p.partial_slots = static_cast<int>(ranges);
      p.workgroups = wg_tiles * ranges;
      return p;
    }
    int64_t ranges = tiles > 0 ? (kRouterTargetWaves + tiles - 1) / tiles : 1;
    ranges = std::min<int64_t>(std::max<int64_t>(ranges, 1), std::max(1, nkc / 2));   // at least 2 chunks each
    ranges = (ranges + 3) / 4 * 4;
    p.kw = static_cast<int>((nkc + ranges - 1) / ranges);
    p.partial_slots = static_cast<int>(ranges / 4);
    p.workgroups = tiles * p.partial_slots;
    return p;
  }
};
struct RouterArgs {
  const uint16_t* x;       // [T][H] bf16 bits
  const uint8_t* packed;   // packed weight (router.hip)
  float* part;             // [partial_slots][T][E]
  float* logits;           // [T][E]
  int32_t* topk_idx;       // [T][top_k]
  float* topk_val;         // [T][top_k]
  int T, E, H, passes, top_k;
  RouterPlan p;
};
hipError_t launch_router_pack(const float* w, int experts, int hidden, uint8_t* packed, hipStream_t stream);
hipError_t launch_router(const RouterArgs& a, hipStream_t stream);

}  // namespace hpa

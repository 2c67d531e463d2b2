// Ancestor walk: visiting consecutive tokens t of one head in order, keep for
// each pyramid level l >= 1 the running sum of the contributions of t's
// selected ancestors at levels >= l, so that a token only adds its own
// level-0 term.  The level-l sum changes only when t crosses a multiple of
// p^l; levels above kWalkLevels fold into one "top" sum that is recomputed at
// multiples of p^(kWalkLevels+1).  Coarse subsequence rows are thus read once
// per span instead of once per token.
//
// Contribution of a selected entry e at level l: w_l * src[pos(e)], with
// w_l = 1 (mean: the caller divides by the count) or 1/p^l (pool backward,
// as the float reciprocal, exact for power-of-two p).
// NT = number of source tensors (0 keeps counts only), E = elements per lane.
// All register arrays are indexed with compile-time constants only.
#pragma once

#include "common.h"

namespace lh {

constexpr int kWalkLevels = 4;

__device__ __forceinline__ bool on_boundary(int32_t t, const Geo& g, int l) {
  return g.log2p >= 0 ? (t & ((1 << (g.log2p * l)) - 1)) == 0 : (t % g.pw[l]) == 0;
}

template <int NT, int E>
struct AncestorWalk {
  static constexpr int kNT = NT > 0 ? NT : 1;
  static constexpr int kTop = kWalkLevels + 1;
  float A[kTop + 1][kNT][E];  // A[l], l = 1..kWalkLevels: levels >= l; A[kTop]: levels >= kTop
  int cnt[kTop + 1];
  bool started = false;

  // posf(l, j): subsequence position of entry j of level l (-1: not selected)
  template <typename PosF>
  __device__ __forceinline__ void add_entry(float (&acc)[kNT][E], int& c, int l, int32_t j,
                                            const PosF& posf, const float* const* src,
                                            const Geo& g, bool mean, int lane) {
    const int32_t r = posf(l, j);
    if (r < 0) return;
    ++c;
    if constexpr (NT > 0) {
      const float w = mean ? 1.0f : g.inv_pw[l];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const float* row = src[i] + (int64_t)r * g.d + E * lane;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const f32x4 q = *reinterpret_cast<const f32x4*>(row + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][e + k] += q[k] * w;
        }
      }
    }
  }

  __device__ __forceinline__ void clear(int slot) {
    cnt[slot] = 0;
#pragma unroll
    for (int i = 0; i < kNT; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) A[slot][i][e] = 0.f;
  }

  // Bring the level sums up to date for token t.
  template <typename PosF>
  __device__ __forceinline__ void advance(int32_t t, const PosF& posf, const float* const* src,
                                          const Geo& g, bool mean, int lane) {
    if (!started || (g.L > kTop && on_boundary(t, g, kTop))) {
      clear(kTop);
      for (int l = kTop; l < g.L; ++l)
        add_entry(A[kTop], cnt[kTop], l, div_pw(t, g, l), posf, src, g, mean, lane);
    }
#pragma unroll
    for (int l = kWalkLevels; l >= 1; --l) {
      if (started && (l >= g.L || !on_boundary(t, g, l))) continue;
      cnt[l] = cnt[l + 1];
#pragma unroll
      for (int i = 0; i < kNT; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) A[l][i][e] = A[l + 1][i][e];
      if (l < g.L) add_entry(A[l], cnt[l], l, div_pw(t, g, l), posf, src, g, mean, lane);
    }
    started = true;
  }
};

}  // namespace lh

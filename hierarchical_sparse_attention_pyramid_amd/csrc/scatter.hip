// Token-side broadcast kernels.
//
//  * forward scatter (gist.science technical summary §2.C, bitsgeniais phase
//    4): out[t] = mean over t's selected ancestors e of os[pos(e)], ancestors
//    visited from level 0 upwards;
//  * backward of gather + pooling: dX[t] = sum over t's selected ancestors e
//    of dXs[pos(e)] / p^level(e) (the adjoint of "copy entry e into the
//    subsequence" composed with "entry e = mean of its p^level tokens").
//
// Sources are float32 rows (the attention output, or the float32 gradients
// of the subsequence); outputs are in the storage type.
// Both are pulls: every output row is written by exactly one row group, which
// reads at most L subsequence rows, so the result is deterministic and no
// atomics are needed.  Coarse rows are shared by up to p^level tokens and are
// served from cache.
#include "kernels.h"

namespace lh {

namespace {

constexpr int kTokensPerGroup = 4;

template <typename Tsrc, typename Tout, int NT>
__global__ __launch_bounds__(256) void bcast_kernel(BcastArgs a) {
  const Geo& g = a.g;
  const int d = g.d;
  const int lpr = d / 8;
  const int rgs = 256 / lpr;
  const int rg = threadIdx.x / lpr, lane = threadIdx.x % lpr;
  const int64_t bh = blockIdx.y;
  const int32_t* pos = a.pos + bh * g.M;
  const Tsrc* src[NT];
  Tout* out[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    src[i] = a.src[i] + bh * (int64_t)g.S * d + 8 * lane;
    out[i] = static_cast<Tout*>(a.out[i]) + bh * (int64_t)g.N * d + 8 * lane;
  }
  const bool pow2 = g.log2p >= 0;
  const int64_t t0 = ((int64_t)blockIdx.x * rgs + rg) * kTokensPerGroup;
  for (int tt = 0; tt < kTokensPerGroup; ++tt) {
    const int64_t t = t0 + tt;
    if (t >= g.N) break;
    float acc[NT][8];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    int cnt = 0;
    for (int l = 0; l < g.L; ++l) {
      const int32_t r = pos[g.base[l] + div_pw((int32_t)t, g, l)];
      if (r < 0) continue;
      ++cnt;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float v[8];
        Row8<Tsrc>::load(src[i] + (int64_t)r * d, v);
        if (a.mean) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] += v[e];
        } else if (pow2) {
          const float w = 1.0f / static_cast<float>(g.pw[l]);  // exact
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] += v[e] * w;
        } else {
          const float dv = static_cast<float>(g.pw[l]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] += v[e] / dv;
        }
      }
    }
    if (a.mean) {
      const float c = static_cast<float>(cnt);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = acc[i][e] / c;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) Row8<Tout>::store(out[i] + t * d, acc[i]);
  }
}

}  // namespace

hipError_t launch_bcast(const BcastArgs& a, int dtype, int ntensors, int64_t BH, hipStream_t st) {
  const int rgs = 256 / (a.g.d / 8);
  const int64_t per_block = (int64_t)rgs * kTokensPerGroup;
  const dim3 grid((unsigned)((a.g.N + per_block - 1) / per_block), (unsigned)BH);
  if (dtype == 1) {
    if (ntensors == 3) bcast_kernel<float, __bf16, 3><<<grid, 256, 0, st>>>(a);
    else bcast_kernel<float, __bf16, 1><<<grid, 256, 0, st>>>(a);
  } else {
    if (ntensors == 3) bcast_kernel<float, float, 3><<<grid, 256, 0, st>>>(a);
    else bcast_kernel<float, float, 1><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace lh

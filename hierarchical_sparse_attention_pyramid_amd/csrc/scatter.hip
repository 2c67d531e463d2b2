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
// Both are pulls: every output row is written by exactly one row group, so
// the result is deterministic and no atomics are needed.  A row group walks
// 64 consecutive tokens with an ancestor walk (walk.h): the contribution of
// an ancestor at level l is loaded once per p^l tokens, and the level-0 loads
// of four tokens are issued together.  Sums run from the coarsest level down
// to level 0.
#include "kernels.h"

#include "walk.h"

namespace lh {

namespace {

#ifndef LH_BC_TOK
#define LH_BC_TOK 64
#endif
#ifndef LH_BC_U
#define LH_BC_U 4
#endif
#ifndef LH_BC_NTS
#define LH_BC_NTS 1
#endif
constexpr int kE = 4;                    // elements per lane (16-byte float32 source loads)
constexpr int kTokPerGroup = LH_BC_TOK;  // consecutive tokens walked by one row group
constexpr int kU = LH_BC_U;              // tokens whose level-0 loads are issued together
constexpr bool kStreamOut = LH_BC_NTS != 0;  // outputs are written once: streaming stores

template <typename Tout> struct Out4;
template <> struct Out4<float> {
  static __device__ __forceinline__ void store(float* p, const float (&x)[kE]) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < kE; ++e) v[e] = x[e];
    st<kStreamOut>(reinterpret_cast<f32x4*>(p), v);
  }
};
template <> struct Out4<__bf16> {
  static __device__ __forceinline__ void store(__bf16* p, const float (&x)[kE]) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < kE; ++e) v[e] = static_cast<__bf16>(x[e]);
    st<kStreamOut>(reinterpret_cast<bf16x4*>(p), v);
  }
};

template <typename Tout, int NT>
__global__ __launch_bounds__(256) void bcast_kernel(BcastArgs a) {
  const Geo& g = a.g;
  const int lpr = g.d / kE;
  const int rgs = 256 / lpr;
  const int rg = threadIdx.x / lpr, lane = threadIdx.x % lpr;
  const int64_t bh = blockIdx.y;
  const int32_t* pos = a.pos + bh * g.M;
  const bool mean = a.mean != 0;
  const float* src[NT];
  Tout* out[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    src[i] = a.src[i] + bh * (int64_t)g.S * g.d;
    out[i] = static_cast<Tout*>(a.out[i]) + bh * (int64_t)g.N * g.d + kE * lane;
  }
  const int32_t t0 = ((int32_t)blockIdx.x * rgs + rg) * kTokPerGroup;
  if (t0 >= g.N) return;  // no block-wide barrier in this kernel
  const int32_t t1 = min(t0 + kTokPerGroup, g.N);
  AncestorWalk<NT, kE> w;
  for (int32_t t = t0; t < t1; t += kU) {
    int32_t r0[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) r0[u] = t + u < t1 ? pos[t + u] : -1;
    float v0[kU][NT][kE];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        f32x4 q = {0.f, 0.f, 0.f, 0.f};
        if (r0[u] >= 0) q = *reinterpret_cast<const f32x4*>(src[i] + (int64_t)r0[u] * g.d + kE * lane);
#pragma unroll
        for (int e = 0; e < kE; ++e) v0[u][i][e] = q[e];
      }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (t + u >= t1) break;
      w.advance(t + u, pos, src, g, mean, lane);
      const int c = w.cnt[1] + (r0[u] >= 0 ? 1 : 0);
      const float rc = mean ? 1.0f / static_cast<float>(c) : 1.0f;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float o[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) o[e] = (w.A[1][i][e] + v0[u][i][e]) * rc;
        Out4<Tout>::store(out[i] + (int64_t)(t + u) * g.d, o);
      }
    }
  }
}

}  // namespace

hipError_t launch_bcast(const BcastArgs& a, int dtype, int ntensors, int64_t BH, hipStream_t st) {
  const int rgs = 256 / (a.g.d / kE);
  const int64_t per_block = (int64_t)rgs * kTokPerGroup;
  const dim3 grid((unsigned)((a.g.N + per_block - 1) / per_block), (unsigned)BH);
  if (dtype == 1) {
    if (ntensors == 3) bcast_kernel<__bf16, 3><<<grid, 256, 0, st>>>(a);
    else bcast_kernel<__bf16, 1><<<grid, 256, 0, st>>>(a);
  } else {
    if (ntensors == 3) bcast_kernel<float, 3><<<grid, 256, 0, st>>>(a);
    else bcast_kernel<float, 1><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace lh

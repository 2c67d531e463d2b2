// Token-side broadcast kernels.
//
//  * forward scatter (gist.science technical summary §2.C, bitsgeniais phase
//    4): out[t] = mean over t's selected ancestors e of os[pos(e)], ancestors
//    visited from level 0 upwards;
//  * backward of gather + pooling: dX[t] = sum over t's selected ancestors e
//    of dXs[pos(e)] / p^level(e) (the adjoint of "copy entry e into the
//    subsequence" composed with "entry e = mean of its p^level tokens").
//
// The causal reading of the forward scatter (bitsgeniais phase 4: no token
// sees the future) sends entry (l, j)'s output to the p^l tokens from its end
// token on, so token t receives, per level, entry (t + 1) / p^l - 1.  That is
// the span rule applied to the virtual token u = t + 1 with every entry index
// lowered by one, which is how both kernels run it: they walk u in
// [0, N + shift), look positions up through vpos(l, J) = pos(l, J - shift)
// (-1 outside the level) and write token u - shift.  A token that no selected
// entry feeds (causal only) gets zeros.
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
#ifndef LH_BC_FAST
#define LH_BC_FAST 1
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

template <typename Tout, int NT, int SH>
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
    out[i] = static_cast<Tout*>(a.out[i]) + a.lout.head(bh) + kE * lane;
  }
  const int32_t nv = g.N + SH;  // virtual tokens u = t + SH
  auto vpos = [&](int l, int32_t j) {
    if constexpr (SH == 0) {
      return pos[g.base[l] + j];
    } else {
      const int32_t jj = j - SH;
      return jj >= 0 && jj < g.nlev[l] ? pos[g.base[l] + jj] : -1;
    }
  };
  const int32_t t0 = ((int32_t)blockIdx.x * rgs + rg) * kTokPerGroup;
  if (t0 >= nv) return;  // no block-wide barrier in this kernel
  const int32_t t1 = min(t0 + kTokPerGroup, nv);
  AncestorWalk<NT, kE> w;
  for (int32_t t = t0; t < t1; t += kU) {
    int32_t r0[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) r0[u] = t + u < t1 ? vpos(0, t + u) : -1;
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
      w.advance(t + u, vpos, src, g, mean, lane);
      const int c = w.cnt[1] + (r0[u] >= 0 ? 1 : 0);
      // span reading: every token has a contributor; causal: 0 for an unfed token
      const float rc = mean ? (SH == 0 || c > 0 ? 1.0f / static_cast<float>(c) : 0.0f) : 1.0f;
      // causal: virtual token 0 (no token) writes zeros to row 0, which the
      // same lanes' next store (token 0) overwrites; no branch per token
      const int32_t row = SH == 0 ? t + u : max(t + u - SH, 0);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float o[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) o[e] = (w.A[1][i][e] + v0[u][i][e]) * rc;
        Out4<Tout>::store(out[i] + (int64_t)row * a.lout.sn, o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fast path for p a power of two >= 4.  The walk above loads, at every level
// boundary, an ancestor's position and then (dependent) its row, level by
// level; here every load of a row group is issued ahead of its use:
//   * the workgroup first stages in LDS the positions of its tokens and of
//     all their ancestors (one coalesced burst);
//   * a row group covers TOK tokens (64; 32 or 16 when 64 would leave fewer
//     than 1,024 workgroups, which also shortens each group's chain of
//     chunks; TOK divides every p^l >= TOK), so the "outer" levels with
//     p^l >= TOK contribute the same rows to all of its tokens: they are
//     summed once, their loads issued together;
//   * the (at most two) inner levels change at chunk starts only (chunks of
//     4 tokens, p >= 4); the rows of chunk c+1 (level 0 and the inner levels
//     that change there) are loaded before chunk c is stored, from two
//     alternating register buffers.
// One tensor per row group (gridDim.z = number of tensors).
#ifndef LH_BC_FAST_TOK
#define LH_BC_FAST_TOK 0  // 0: chosen per launch; else forced (16, 32 or 64)
#endif
constexpr int kFastU = 4;
constexpr int kFastInner = 2;      // inner levels handled (p = 4: levels 1, 2)
constexpr int kFastOuter = 8;      // outer levels summed with loads in flight together
constexpr int kPosCache = 1536;    // ints: 1024 tokens + ancestors (p >= 4)

struct FastBuf {
  float r0[kFastU][kE];            // level-0 rows (zero when not selected)
  int s0[kFastU];
  float ri[kFastInner][kE];        // inner-level rows that change at the chunk start
  int si[kFastInner];
};

template <typename Tout, int SH, int TOK>
__global__ __launch_bounds__(256) void bcast_fast(BcastArgs a) {
  constexpr int kFastTok = TOK;
  static_assert(TOK == 16 || TOK == 32 || TOK == 64, "row-group token counts");
  const Geo& g = a.g;
  const int lpr = g.d / kE;
  const int rgs = 256 / lpr;
  const int BT = rgs * kFastTok;  // tokens per workgroup
  const int rg = threadIdx.x / lpr, lane = threadIdx.x % lpr;
  const int64_t bh = blockIdx.y;
  const int z = blockIdx.z;
  const int32_t B0 = (int32_t)blockIdx.x * BT;
  const int32_t* pos = a.pos + bh * g.M;
  const int lg = g.log2p;
  const int32_t nv = g.N + SH;  // virtual tokens u = t + SH
  __shared__ int32_t sp[kPosCache];
  __shared__ int32_t soff[kMaxLevels];  // start of level l's run in sp

  // ---- stage positions vpos: virtual tokens [B0, B0 + BT), then each
  // level's ancestors of them, one run per level (run l: max(1, BT / p^l)
  // entries from entry B0 / p^l; at most 256 for l >= 1 since BT <= 1024 and
  // p >= 4).  A thread issues every position load it makes before its first
  // LDS store: the staging costs one memory latency, not one per level.
  const int lbt = __builtin_ctz(BT);  // BT is a power of two (TOK tokens x 8 or 16 row groups)
  {
    constexpr int kTok = 1024 / 256;  // level-0 entries per thread
    int32_t p0[kTok], pl[kMaxLevels];
#pragma unroll
    for (int k = 0; k < kTok; ++k) {
      const int i = threadIdx.x + k * 256;
      const int32_t t = B0 + i - SH;
      p0[k] = i < BT && (SH == 0 || t >= 0) && t < g.N ? pos[t] : -1;
    }
#pragma unroll
    for (int l = 1; l < kMaxLevels; ++l) {
      const int n = lg * l >= lbt ? 1 : BT >> (lg * l);
      const int32_t j = (B0 >> (lg * l)) - SH + (int)threadIdx.x;
      pl[l] = l < g.L && (int)threadIdx.x < n && (SH == 0 || j >= 0) && j < g.nlev[l]
                  ? pos[g.base[l] + j] : -1;
    }
#pragma unroll
    for (int k = 0; k < kTok; ++k)
      if (threadIdx.x + k * 256 < BT) sp[threadIdx.x + k * 256] = p0[k];
    int off = BT;
#pragma unroll
    for (int l = 1; l < kMaxLevels; ++l) {
      if (l >= g.L) break;
      const int n = lg * l >= lbt ? 1 : BT >> (lg * l);
      if (threadIdx.x == 0) soff[l] = off;
      if ((int)threadIdx.x < n) sp[off + threadIdx.x] = pl[l];
      off += n;
    }
  }
  __syncthreads();
  const int32_t t0 = B0 + rg * kFastTok;
  if (t0 >= nv) return;  // no barrier below
  const int32_t t1 = min(t0 + kFastTok, nv);

  const float* src = a.src[z] + bh * (int64_t)g.S * g.d + kE * lane;
  Tout* out = static_cast<Tout*>(a.out[z]) + a.lout.head(bh) + kE * lane;
  const bool mean = a.mean != 0;

  // levels 1 .. lam-1 are inner (p^l < TOK), lam .. L-1 outer
  constexpr int kLogTok = TOK == 64 ? 6 : TOK == 32 ? 5 : 4;
  int lam = 1;
  while (lam < g.L && (lg * lam) < kLogTok) ++lam;
  const int nin = lam - 1;  // <= 2 since p >= 4

  auto level_pos = [&](int l, int32_t j) { return sp[soff[l] + (j - (B0 >> (lg * l)))]; };
  auto load_row = [&](int32_t r, float (&x)[kE]) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(src + (int64_t)r * g.d);
#pragma unroll
    for (int e = 0; e < kE; ++e) x[e] = q[e];
  };

  // ---- outer levels: the same ancestors for all 64 tokens of the group
  float A[kFastInner + 1][kE];  // A[k]: sum over levels >= k+1 ... A[nin]: outer
  int C[kFastInner + 1];
  {
    float rows[kFastOuter][kE];
    int sel[kFastOuter];
#pragma unroll
    for (int k = 0; k < kFastOuter; ++k) {
      const int l = lam + k;
      sel[k] = 0;
#pragma unroll
      for (int e = 0; e < kE; ++e) rows[k][e] = 0.f;
      if (l < g.L) {
        const int32_t pe = level_pos(l, t0 >> (lg * l));
        if (pe >= 0) {
          load_row(pe, rows[k]);
          sel[k] = 1;
        }
      }
    }
    float acc[kE] = {0.f, 0.f, 0.f, 0.f};
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kFastOuter; ++k) {
      const float w = mean ? 1.0f : g.inv_pw[min(lam + k, kMaxLevels - 1)];
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] += rows[k][e] * w;
      cnt += sel[k];
    }
    for (int l = lam + kFastOuter; l < g.L; ++l) {  // very deep pyramids: one at a time
      const int32_t pe = level_pos(l, t0 >> (lg * l));
      if (pe >= 0) {
        float x[kE];
        load_row(pe, x);
        const float w = mean ? 1.0f : g.inv_pw[l];
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[e] += x[e] * w;
        ++cnt;
      }
    }
#pragma unroll
    for (int k = 0; k <= kFastInner; ++k) {
      C[k] = cnt;
#pragma unroll
      for (int e = 0; e < kE; ++e) A[k][e] = acc[e];
    }
  }

  // ---- chunk pipeline over the group's tokens
  auto issue = [&](int32_t c, FastBuf& b) {
#pragma unroll
    for (int u = 0; u < kFastU; ++u) {
      const int32_t t = c + u;
      const int32_t p0 = t < t1 ? sp[t - B0] : -1;
      b.s0[u] = p0 >= 0;
#pragma unroll
      for (int e = 0; e < kE; ++e) b.r0[u][e] = 0.f;
      if (p0 >= 0) load_row(p0, b.r0[u]);
    }
#pragma unroll
    for (int k = 0; k < kFastInner; ++k) {
      const int l = k + 1;
      b.si[k] = 0;
#pragma unroll
      for (int e = 0; e < kE; ++e) b.ri[k][e] = 0.f;
      if (l <= nin && (c & ((1 << (lg * l)) - 1)) == 0) {
        const int32_t pe = level_pos(l, c >> (lg * l));
        if (pe >= 0) {
          load_row(pe, b.ri[k]);
          b.si[k] = 1;
        }
      }
    }
  };
  auto process = [&](int32_t c, const FastBuf& b) {
    // inner levels that change at c, top down: A[l-1] = A[l] + row_l (A[nin] = outer)
#pragma unroll
    for (int k = kFastInner - 1; k >= 0; --k) {
      const int l = k + 1;
      if (l <= nin && (c & ((1 << (lg * l)) - 1)) == 0) {
        const float w = mean ? 1.0f : g.inv_pw[l];
        C[k] = C[k + 1] + b.si[k];
#pragma unroll
        for (int e = 0; e < kE; ++e) A[k][e] = A[k + 1][e] + b.ri[k][e] * w;
      }
    }
#pragma unroll
    for (int u = 0; u < kFastU; ++u) {
      const int32_t t = c + u;
      if (t >= t1) break;
      const int cnt = C[0] + b.s0[u];
      // span reading: every token has a contributor; causal: 0 for an unfed token
      const float rc =
          mean ? (SH == 0 || cnt > 0 ? 1.0f / static_cast<float>(cnt) : 0.0f) : 1.0f;
      float o[kE];
#pragma unroll
      for (int e = 0; e < kE; ++e) o[e] = (A[0][e] + b.r0[u][e]) * rc;
      // causal: virtual token 0 (no token) writes zeros to row 0, which the
      // same lanes' next store (token 0) overwrites; no branch per token
      Out4<Tout>::store(out + (int64_t)(SH == 0 ? t : max(t - SH, 0)) * a.lout.sn, o);
    }
  };
  if (nin == 0) {  // A[0] must be the outer sum
#pragma unroll
    for (int e = 0; e < kE; ++e) A[0][e] = A[kFastInner][e];
    C[0] = C[kFastInner];
  } else if (nin == 1) {  // A[1] plays the outer sum for level 1
#pragma unroll
    for (int e = 0; e < kE; ++e) A[1][e] = A[kFastInner][e];
    C[1] = C[kFastInner];
  }
  FastBuf ba, bb;
  issue(t0, ba);
  for (int32_t c = t0; c < t1; c += 2 * kFastU) {
    if (c + kFastU < t1) issue(c + kFastU, bb);
    process(c, ba);
    if (c + kFastU >= t1) break;
    if (c + 2 * kFastU < t1) issue(c + 2 * kFastU, ba);
    process(c + kFastU, bb);
  }
}

}  // namespace

hipError_t launch_bcast(const BcastArgs& a, int dtype, int ntensors, int64_t BH, hipStream_t st) {
  const int rgs = 256 / (a.g.d / kE);
  const int64_t nv = (int64_t)a.g.N + a.shift;  // virtual tokens
  // the shift is a template parameter: the span reading's kernels carry no
  // virtual-token bookkeeping at all
  if (ntensors < 1 || ntensors > 3) return hipErrorInvalidValue;
  if (a.shift != 0 && (ntensors != 1 || a.mean == 0)) return hipErrorInvalidValue;
  if (LH_BC_FAST && a.g.log2p >= 2) {
    // tokens per row group: 64 unless that leaves under 1,024 workgroups
    int tok = 64;
    auto blocks = [&](int t) { return (nv + (int64_t)rgs * t - 1) / ((int64_t)rgs * t); };
    if (LH_BC_FAST_TOK != 0) tok = LH_BC_FAST_TOK;
    else while (tok > 16 && blocks(tok) * BH * ntensors < 1024) tok /= 2;
    const dim3 grid((unsigned)blocks(tok), (unsigned)BH, (unsigned)ntensors);
    auto go = [&](auto kern) { kern<<<grid, 256, 0, st>>>(a); };
    if (dtype == 1) {
      if (a.shift) {
        if (tok == 64) go(bcast_fast<__bf16, 1, 64>);
        else if (tok == 32) go(bcast_fast<__bf16, 1, 32>);
        else go(bcast_fast<__bf16, 1, 16>);
      } else {
        if (tok == 64) go(bcast_fast<__bf16, 0, 64>);
        else if (tok == 32) go(bcast_fast<__bf16, 0, 32>);
        else go(bcast_fast<__bf16, 0, 16>);
      }
    } else {
      if (a.shift) {
        if (tok == 64) go(bcast_fast<float, 1, 64>);
        else if (tok == 32) go(bcast_fast<float, 1, 32>);
        else go(bcast_fast<float, 1, 16>);
      } else {
        if (tok == 64) go(bcast_fast<float, 0, 64>);
        else if (tok == 32) go(bcast_fast<float, 0, 32>);
        else go(bcast_fast<float, 0, 16>);
      }
    }
    return hipGetLastError();
  }
  const int64_t per_block = (int64_t)rgs * kTokPerGroup;
  const dim3 grid((unsigned)((nv + per_block - 1) / per_block), (unsigned)BH);
  if (dtype == 1) {
    if (ntensors == 3) bcast_kernel<__bf16, 3, 0><<<grid, 256, 0, st>>>(a);
    else if (ntensors == 2) bcast_kernel<__bf16, 2, 0><<<grid, 256, 0, st>>>(a);
    else if (a.shift) bcast_kernel<__bf16, 1, 1><<<grid, 256, 0, st>>>(a);
    else bcast_kernel<__bf16, 1, 0><<<grid, 256, 0, st>>>(a);
  } else {
    if (ntensors == 3) bcast_kernel<float, 3, 0><<<grid, 256, 0, st>>>(a);
    else if (ntensors == 2) bcast_kernel<float, 2, 0><<<grid, 256, 0, st>>>(a);
    else if (a.shift) bcast_kernel<float, 1, 1><<<grid, 256, 0, st>>>(a);
    else bcast_kernel<float, 1, 0><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace lh

// Causal flash-style attention on bf16 inputs with gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, float32 accumulation).  This is the "stock dense
// attention on the gathered subsequence" of the gist.science technical
// summary, §2.C, and, at S = N, the dense baseline.
//
// MFMA 32x32x16 operand layout (wave of 64 lanes, lane = 32*h + c):
//   A (32 x 16): lane holds row c, k = 8h .. 8h+7 (8 bf16)
//   B (16 x 32): lane holds column c, k = 8h .. 8h+7
//   D (32 x 32): lane holds column c, rows 8*(i/4) + 4h + (i%4), i = 0..15
// A contraction index may be permuted as long as A and B agree.  Chunk c of
// a D-layout block (elements 8c..8c+7) covers rows 16c + {4h..4h+3} and
// 16c + 8 + {4h..4h+3}; feeding it as a B operand therefore pairs with an A
// operand whose lane reads two runs of 4 consecutive rows of the transposed
// tile.  Those transposed tiles are staged in LDS.
//
// Forward: each wave owns 64 queries and computes S^T = K Q^T (keys x
// queries), so every lane holds one query column: the softmax statistics are
// per lane (one cross-half shuffle), and O^T = V^T P^T accumulates with P^T
// straight from registers.
// Backward: a key-block pass (dK, dV; keys stationary) and a query-block pass
// (dQ; queries stationary), both atomic-free, recomputing P from the stored
// log-sum-exp.
#include "kernels.h"

namespace lh {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<__bf16>(0.f);
  return z;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

// A operand from a transposed LDS tile: row `r` of the tile, runs at column
// col and col + 8 (4 elements each).
__device__ __forceinline__ bf16x8 load_tr(const __bf16* tile, int stride, int r, int col) {
  const __bf16* p = tile + r * stride + col;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 8);
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = lo[e];
    a[e + 4] = hi[e];
  }
  return a;
}

// Stage rows [r0, r0+R) of a [S][D] tensor into LDS row-major (stride RS)
// and/or transposed (tile[dim][row], stride TS); rows >= S read as zero.
template <int D, int R, int NTHR>
__device__ __forceinline__ void stage_rows(const __bf16* src, int S, int r0, __bf16* rowmajor,
                                           int RS, __bf16* transposed, int TS, int tid) {
  constexpr int kUnits = (R / 4) * (D / 8);  // 4 rows x 8 dims per unit
  for (int u = tid; u < kUnits; u += NTHR) {
    const int rg = u / (D / 8), dg = u % (D / 8);
    bf16x8 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * rg + i;
      r[i] = row < S ? *reinterpret_cast<const bf16x8*>(src + (int64_t)row * D + dg * 8) : zero8();
      if (rowmajor) *reinterpret_cast<bf16x8*>(rowmajor + (4 * rg + i) * RS + dg * 8) = r[i];
    }
    if (transposed) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 t;
        t[0] = r[0][e];
        t[1] = r[1][e];
        t[2] = r[2][e];
        t[3] = r[3][e];
        *reinterpret_cast<bf16x4*>(transposed + (dg * 8 + e) * TS + 4 * rg) = t;
      }
    }
  }
}

// ------------------------------------------------------------------ forward

template <int D>
struct FwdCfg {
  static constexpr int kWaves = 2;
  static constexpr int kQW = 64;                 // queries per wave (2 x 32)
  static constexpr int kQB = kWaves * kQW;       // queries per workgroup
  static constexpr int kKT = 64;                 // keys per tile
  static constexpr int kKS = D + 8;              // K tile row stride (elements)
  static constexpr int kVS = kKT + 4;            // V^T tile row stride
};

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_bf16(const __bf16* __restrict__ Q,
                                                     const __bf16* __restrict__ K,
                                                     const __bf16* __restrict__ V,
                                                     float* __restrict__ O,
                                                     float* __restrict__ LSE, int S, float sl2) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[C::kKT * C::kKS];
  __shared__ __attribute__((aligned(16))) __bf16 sVt[D * C::kVS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int64_t bh = blockIdx.y;
  const int qblk = gridDim.x - 1 - blockIdx.x;  // late (heavy) query blocks first
  const int q0 = qblk * C::kQB;
  const int qw0 = q0 + wave * C::kQW;
  const __bf16* Qh = Q + bh * (int64_t)S * D;
  const __bf16* Kh = K + bh * (int64_t)S * D;
  const __bf16* Vh = V + bh * (int64_t)S * D;

  bf16x8 qreg[2][D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw0 + qb * 32 + c32;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      qreg[qb][dc] = row < S ? *reinterpret_cast<const bf16x8*>(Qh + (int64_t)row * D + dc * 16 + 8 * h)
                             : zero8();
  }
  f32x16 oacc[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[qb][mb] = zero16();
  float mrow[2] = {neg_inf(), neg_inf()};
  float lsum[2] = {0.f, 0.f};

  const int kend = min(S, q0 + C::kQB);
  const int ntiles = (kend + C::kKT - 1) / C::kKT;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * C::kKT;
    __syncthreads();
    stage_rows<D, C::kKT, 128>(Kh, S, k0, sK, C::kKS, nullptr, 0, tid);
    stage_rows<D, C::kKT, 128>(Vh, S, k0, nullptr, 0, sVt, C::kVS, tid);
    __syncthreads();
    if (qw0 >= S || k0 > qw0 + C::kQW - 1) continue;  // nothing visible for this wave

    f32x16 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = zero16();
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (kb * 32 + c32) * C::kKS + dc * 16 + 8 * h);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = mfma32(a, qreg[qb][dc], sacc[kb][qb]);
      }
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qbase = qw0 + qb * 32;
      if (k0 > qbase + 31) continue;
      const int query = qbase + c32;
      const bool diag = k0 + C::kKT - 1 > qbase;
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          float s = sacc[kb][qb][i] * sl2;
          if (diag && key > query) s = neg_inf();
          sacc[kb][qb][i] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[qb], mx);
      const float alpha = fexp2(mrow[qb] - mnew);
      mrow[qb] = mnew;
      lsum[qb] *= alpha;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) oacc[qb][mb] *= alpha;
      bf16x8 pk[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = fexp2(sacc[kb][qb][8 * c + e] - mnew);
            lsum[qb] += pv;
            pk[kb][c][e] = static_cast<__bf16>(pv);
          }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) {
            const bf16x8 a = load_tr(sVt, C::kVS, mb * 32 + c32, kb * 32 + 16 * c + 4 * h);
            oacc[qb][mb] = mfma32(a, pk[kb][c], oacc[qb][mb]);
          }
    }
  }

  if (qw0 >= S) return;
  float* Oh = O + bh * (int64_t)S * D;
  float* Lh = LSE + bh * (int64_t)S;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const float inv = 1.0f / lt;
    const int query = qw0 + qb * 32 + c32;
    if (query < S) {
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = oacc[qb][mb][4 * j + r] * inv;
          *reinterpret_cast<f32x4*>(Oh + (int64_t)query * D + mb * 32 + 8 * j + 4 * h) = o;
        }
      if (h == 0) Lh[query] = (mrow[qb] + log2f(lt)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------ backward

// delta[i] = sum_d dO[i,d] * O[i,d] (float32), one row per d/8-lane group.
// O is the float32 forward output: rounding it to bf16 first would perturb
// delta by ~2^-9 |dO||O|, and dS = P (dP - delta) cancels for keys that
// dominate a row, which would amplify that error in dK and dQ.
template <typename T>
__global__ __launch_bounds__(256) void attn_delta(const float* __restrict__ O, const T* __restrict__ dO,
                                                  float* __restrict__ delta, int64_t rows, int d) {
  const int lpr = d / 8;
  const int rgs = 256 / lpr;
  const int lane = threadIdx.x % lpr;
  const int64_t row = (int64_t)blockIdx.x * rgs + threadIdx.x / lpr;
  float s = 0.f;
  if (row < rows) {
    float o[8], g[8];
    Row8<float>::load(O + row * d + 8 * lane, o);
    Row8<T>::load(dO + row * d + 8 * lane, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += o[e] * g[e];
  }
  for (int off = lpr >> 1; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && lane == 0) delta[row] = s;
}

template <int D>
struct BwdKVCfg {
  static constexpr int kWaves = 4;
  static constexpr int kKW = 32;            // keys per wave
  static constexpr int kKB = kWaves * kKW;  // keys per workgroup
  static constexpr int kQT = 64;            // queries per tile
  static constexpr int kRS = D + 8;
  static constexpr int kTS = kQT + 4;
};

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_bf16(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    float* __restrict__ dK, float* __restrict__ dV, int S, float sl2, float scale) {
  using C = BwdKVCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[C::kQT * C::kRS];
  __shared__ __attribute__((aligned(16))) __bf16 sdO[C::kQT * C::kRS];
  __shared__ __attribute__((aligned(16))) __bf16 sQt[D * C::kTS];
  __shared__ __attribute__((aligned(16))) __bf16 sdOt[D * C::kTS];
  __shared__ float sL[C::kQT], sDl[C::kQT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int64_t bh = blockIdx.y;
  const int kb0 = blockIdx.x * C::kKB;
  const int kw0 = kb0 + wave * C::kKW;
  const int key = kw0 + c32;
  const int64_t off = bh * (int64_t)S * D;

  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    kreg[dc] = key < S ? *reinterpret_cast<const bf16x8*>(K + off + (int64_t)key * D + dc * 16 + 8 * h) : zero8();
    vreg[dc] = key < S ? *reinterpret_cast<const bf16x8*>(V + off + (int64_t)key * D + dc * 16 + 8 * h) : zero8();
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    dka[mb] = zero16();
    dva[mb] = zero16();
  }

  for (int q0 = (kb0 / C::kQT) * C::kQT; q0 < S; q0 += C::kQT) {
    __syncthreads();
    stage_rows<D, C::kQT, 256>(Q + off, S, q0, sQ, C::kRS, sQt, C::kTS, tid);
    stage_rows<D, C::kQT, 256>(dO + off, S, q0, sdO, C::kRS, sdOt, C::kTS, tid);
    if (tid < C::kQT) {
      const int q = q0 + tid;
      sL[tid] = q < S ? LSE[bh * (int64_t)S + q] * kLog2e : 0.f;
      sDl[tid] = q < S ? DELTA[bh * (int64_t)S + q] : 0.f;
    }
    __syncthreads();
    if (kw0 >= S || q0 + C::kQT - 1 < kw0) continue;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qbase = q0 + qs * 32;
      if (qbase + 31 < kw0) continue;
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const int o = (qs * 32 + c32) * C::kRS + dc * 16 + 8 * h;
        sacc = mfma32(*reinterpret_cast<const bf16x8*>(sQ + o), kreg[dc], sacc);
        dpacc = mfma32(*reinterpret_cast<const bf16x8*>(sdO + o), vreg[dc], dpacc);
      }
      bf16x8 pch[2], dsch[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = qs * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        const int query = q0 + qi;
        const float p = (key <= query && query < S) ? fexp2(sacc[i] * sl2 - sL[qi]) : 0.f;
        const float ds = p * (dpacc[i] - sDl[qi]);
        pch[i >> 3][i & 7] = static_cast<__bf16>(p);
        dsch[i >> 3][i & 7] = static_cast<__bf16>(ds);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          const int col = qs * 32 + 16 * c + 4 * h;
          dva[mb] = mfma32(load_tr(sdOt, C::kTS, mb * 32 + c32, col), pch[c], dva[mb]);
          dka[mb] = mfma32(load_tr(sQt, C::kTS, mb * 32 + c32, col), dsch[c], dka[mb]);
        }
    }
  }
  if (key >= S) return;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 a, b;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = dka[mb][4 * j + r] * scale;
        b[r] = dva[mb][4 * j + r];
      }
      const int64_t o = off + (int64_t)key * D + mb * 32 + 8 * j + 4 * h;
      *reinterpret_cast<f32x4*>(dK + o) = a;
      *reinterpret_cast<f32x4*>(dV + o) = b;
    }
}

template <int D>
struct BwdQCfg {
  static constexpr int kWaves = 4;
  static constexpr int kQW = 32;
  static constexpr int kQB = kWaves * kQW;
  static constexpr int kKT = 64;
  static constexpr int kRS = D + 8;
  static constexpr int kTS = kKT + 4;
};

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    float* __restrict__ dQ, int S, float sl2, float scale) {
  using C = BwdQCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[C::kKT * C::kRS];
  __shared__ __attribute__((aligned(16))) __bf16 sV[C::kKT * C::kRS];
  __shared__ __attribute__((aligned(16))) __bf16 sKt[D * C::kTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int64_t bh = blockIdx.y;
  const int qblk = gridDim.x - 1 - blockIdx.x;
  const int q0 = qblk * C::kQB;
  const int qw0 = q0 + wave * C::kQW;
  const int query = qw0 + c32;
  const int64_t off = bh * (int64_t)S * D;

  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    qreg[dc] = query < S ? *reinterpret_cast<const bf16x8*>(Q + off + (int64_t)query * D + dc * 16 + 8 * h) : zero8();
    doreg[dc] = query < S ? *reinterpret_cast<const bf16x8*>(dO + off + (int64_t)query * D + dc * 16 + 8 * h) : zero8();
  }
  const float lse2 = query < S ? LSE[bh * (int64_t)S + query] * kLog2e : 0.f;
  const float dl = query < S ? DELTA[bh * (int64_t)S + query] : 0.f;
  f32x16 dqa[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) dqa[mb] = zero16();

  const int kend = min(S, q0 + C::kQB);
  for (int k0 = 0; k0 < kend; k0 += C::kKT) {
    __syncthreads();
    stage_rows<D, C::kKT, 256>(K + off, S, k0, sK, C::kRS, sKt, C::kTS, tid);
    stage_rows<D, C::kKT, 256>(V + off, S, k0, sV, C::kRS, nullptr, 0, tid);
    __syncthreads();
    if (qw0 >= S || k0 > qw0 + C::kQW - 1) continue;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kbase = k0 + kb * 32;
      if (kbase > qw0 + 31) continue;
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const int o = (kb * 32 + c32) * C::kRS + dc * 16 + 8 * h;
        sacc = mfma32(*reinterpret_cast<const bf16x8*>(sK + o), qreg[dc], sacc);
        dpacc = mfma32(*reinterpret_cast<const bf16x8*>(sV + o), doreg[dc], dpacc);
      }
      bf16x8 dsch[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + 8 * (i >> 2) + 4 * h + (i & 3);
        const float p = key <= query ? fexp2(sacc[i] * sl2 - lse2) : 0.f;
        dsch[i >> 3][i & 7] = static_cast<__bf16>(p * (dpacc[i] - dl));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
          dqa[mb] = mfma32(load_tr(sKt, C::kTS, mb * 32 + c32, kb * 32 + 16 * c + 4 * h), dsch[c],
                           dqa[mb]);
    }
  }
  if (query >= S) return;
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = dqa[mb][4 * j + r] * scale;
      *reinterpret_cast<f32x4*>(dQ + off + (int64_t)query * D + mb * 32 + 8 * j + 4 * h) = a;
    }
}

}  // namespace

// fp32 paths live in attention_f32.hip
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int64_t S, int d, int64_t BH, hipStream_t st);
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* lse,
                               const float* delta, const float* dout, float* dq, float* dk,
                               float* dv, int64_t S, int d, int64_t BH, hipStream_t st,
                               hipEvent_t* ev);

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int64_t S, int d, int dtype, int64_t BH, hipStream_t st) {
  if (S == 0) return hipSuccess;
  if (dtype == 0)
    return launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                               static_cast<const float*>(v), o, lse, S, d, BH, st);
  const float sl2 = kLog2e / sqrtf((float)d);
  const auto Q = static_cast<const __bf16*>(q);
  const auto K = static_cast<const __bf16*>(k);
  const auto V = static_cast<const __bf16*>(v);
  if (d == 64) {
    const dim3 grid((unsigned)((S + FwdCfg<64>::kQB - 1) / FwdCfg<64>::kQB), (unsigned)BH);
    attn_fwd_bf16<64><<<grid, 128, 0, st>>>(Q, K, V, o, lse, (int)S, sl2);
  } else {
    const dim3 grid((unsigned)((S + FwdCfg<128>::kQB - 1) / FwdCfg<128>::kQB), (unsigned)BH);
    attn_fwd_bf16<128><<<grid, 128, 0, st>>>(Q, K, V, o, lse, (int)S, sl2);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* delta, int64_t S, int d, int dtype, int64_t BH,
                           hipStream_t st, hipEvent_t* ev) {
  if (S == 0) return hipSuccess;
  const int64_t rows = S * BH;
  const int rgs = 256 / (d / 8);
  const unsigned dgrid = (unsigned)((rows + rgs - 1) / rgs);
  const bool f32 = dtype == 0;
  if (f32) attn_delta<float><<<dgrid, 256, 0, st>>>(o, static_cast<const float*>(dout), delta, rows, d);
  else attn_delta<__bf16><<<dgrid, 256, 0, st>>>(o, static_cast<const __bf16*>(dout), delta, rows, d);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[0], st);
  if (e != hipSuccess) return e;
  if (f32) {
    e = launch_attn_bwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                            static_cast<const float*>(v), lse, delta,
                            static_cast<const float*>(dout), dq, dk, dv, S, d, BH, st, ev);
    return e;
  }
  const float scale = 1.0f / sqrtf((float)d);
  const float sl2 = kLog2e * scale;
  const auto Q = static_cast<const __bf16*>(q);
  const auto K = static_cast<const __bf16*>(k);
  const auto V = static_cast<const __bf16*>(v);
  const auto G = static_cast<const __bf16*>(dout);
  if (d == 64) {
    const dim3 g1((unsigned)((S + BwdKVCfg<64>::kKB - 1) / BwdKVCfg<64>::kKB), (unsigned)BH);
    attn_bwd_dkdv_bf16<64><<<g1, 256, 0, st>>>(Q, K, V, G, lse, delta, dk, dv, (int)S, sl2, scale);
  } else {
    const dim3 g1((unsigned)((S + BwdKVCfg<128>::kKB - 1) / BwdKVCfg<128>::kKB), (unsigned)BH);
    attn_bwd_dkdv_bf16<128><<<g1, 256, 0, st>>>(Q, K, V, G, lse, delta, dk, dv, (int)S, sl2, scale);
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
  if (e != hipSuccess) return e;
  if (d == 64) {
    const dim3 g2((unsigned)((S + BwdQCfg<64>::kQB - 1) / BwdQCfg<64>::kQB), (unsigned)BH);
    attn_bwd_dq_bf16<64><<<g2, 256, 0, st>>>(Q, K, V, G, lse, delta, dq, (int)S, sl2, scale);
  } else {
    const dim3 g2((unsigned)((S + BwdQCfg<128>::kQB - 1) / BwdQCfg<128>::kQB), (unsigned)BH);
    attn_bwd_dq_bf16<128><<<g2, 256, 0, st>>>(Q, K, V, G, lse, delta, dq, (int)S, sl2, scale);
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  return e;
}

}  // namespace lh

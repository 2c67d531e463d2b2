// Causal attention for float32 inputs on the vector ALUs (the fp32 storage
// type; the bf16 path uses the matrix cores).  Four lanes share one row, each
// holding d/4 of its elements; keys (or queries) are staged 64 rows at a time
// in LDS.  The forward keeps a running max and normaliser per query (online
// softmax); the backward recomputes probabilities from the stored
// log-sum-exp in a key-major pass (dK, dV) and a query-major pass (dQ), so no
// atomics are needed.
//
// Precision: scores q.k, dP = dO.v and every accumulation are float64, and
// each exponential takes a float32 argument formed in float64 (s - max,
// s - lse).  A float32 dot product of large, heavy-tailed rows is off by
// ~1e-5 in absolute terms, a different amount for every key; exponentiated,
// that is a 1e-5 relative error in each weight, which dQ and dK sum over
// up to S keys.  On this path float64 costs about what float32 does per
// operation (no packed float32).
#include "kernels.h"

namespace lh {

namespace {

constexpr int kRows = 64;  // rows per workgroup and per LDS tile

template <int D>
__device__ __forceinline__ double dot4(const float (&a)[D / 4], const float* b) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) s = fma((double)a[e], (double)b[e], s);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  return s;
}

template <int D>
__device__ __forceinline__ void stage(float* dst, const float* src, int S, int r0, int tid) {
  for (int i = tid; i < kRows * D; i += 256) {
    const int r = i / D;
    dst[i] = r0 + r < S ? src[(int64_t)(r0 + r) * D + (i % D)] : 0.f;
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                    const float* __restrict__ V, float* __restrict__ O,
                                                    float* __restrict__ LSE, int S, double scale) {
  __shared__ float sK[kRows * D], sV[kRows * D];
  const int tid = threadIdx.x, sub = tid & 3;
  const int64_t off = blockIdx.y * (int64_t)S * D;
  const int query = blockIdx.x * kRows + tid / 4;
  float q[D / 4];
  double o[D / 4];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) {
    q[e] = query < S ? Q[off + (int64_t)query * D + sub * (D / 4) + e] : 0.f;
    o[e] = 0.0;
  }
  double m = -1e300, l = 0.0;
  const int kend = min(S, (int)(blockIdx.x + 1) * kRows);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    __syncthreads();
    stage<D>(sK, K + off, S, k0, tid);
    stage<D>(sV, V + off, S, k0, tid);
    __syncthreads();
    for (int j = 0; j < kRows; ++j) {
      const double s = dot4<D>(q, sK + j * D + sub * (D / 4)) * scale;
      if (k0 + j > query) continue;
      const double mn = fmax(m, s);
      const double alpha = expf((float)(m - mn));
      const double p = expf((float)(s - mn));
      l = l * alpha + p;
#pragma unroll
      for (int e = 0; e < D / 4; ++e) o[e] = o[e] * alpha + p * (double)sV[j * D + sub * (D / 4) + e];
      m = mn;
    }
  }
  if (query >= S) return;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) O[off + (int64_t)query * D + sub * (D / 4) + e] = (float)(o[e] / l);
  if (sub == 0) LSE[blockIdx.y * (int64_t)S + query] = (float)(m + log(l));
}

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ dO,
                                                         const float* __restrict__ LSE,
                                                         const float* __restrict__ DELTA,
                                                         float* __restrict__ dK, float* __restrict__ dV,
                                                         int S, double scale) {
  __shared__ float sQ[kRows * D], sG[kRows * D], sL[kRows], sDl[kRows];
  const int tid = threadIdx.x, sub = tid & 3;
  const int64_t off = blockIdx.y * (int64_t)S * D;
  const int key = blockIdx.x * kRows + tid / 4;
  float k[D / 4], v[D / 4];
  double dk[D / 4], dv[D / 4];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) {
    k[e] = key < S ? K[off + (int64_t)key * D + sub * (D / 4) + e] : 0.f;
    v[e] = key < S ? V[off + (int64_t)key * D + sub * (D / 4) + e] : 0.f;
    dk[e] = dv[e] = 0.0;
  }
  for (int q0 = blockIdx.x * kRows; q0 < S; q0 += kRows) {
    __syncthreads();
    stage<D>(sQ, Q + off, S, q0, tid);
    stage<D>(sG, dO + off, S, q0, tid);
    if (tid < kRows) {
      sL[tid] = q0 + tid < S ? LSE[blockIdx.y * (int64_t)S + q0 + tid] : 0.f;
      sDl[tid] = q0 + tid < S ? DELTA[blockIdx.y * (int64_t)S + q0 + tid] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < kRows; ++i) {
      const float* qi = sQ + i * D + sub * (D / 4);
      const float* gi = sG + i * D + sub * (D / 4);
      const double s = dot4<D>(k, qi) * scale;
      const double dp = dot4<D>(v, gi);
      const int query = q0 + i;
      if (query >= S || key > query) continue;
      const double p = expf((float)(s - (double)sL[i]));
      const double ds = p * (dp - (double)sDl[i]);
#pragma unroll
      for (int e = 0; e < D / 4; ++e) {
        dv[e] = fma(p, (double)gi[e], dv[e]);
        dk[e] = fma(ds, (double)qi[e], dk[e]);
      }
    }
  }
  if (key >= S) return;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) {
    dK[off + (int64_t)key * D + sub * (D / 4) + e] = (float)(dk[e] * scale);
    dV[off + (int64_t)key * D + sub * (D / 4) + e] = (float)dv[e];
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       const float* __restrict__ DELTA,
                                                       float* __restrict__ dQ, int S, double scale) {
  __shared__ float sK[kRows * D], sV[kRows * D];
  const int tid = threadIdx.x, sub = tid & 3;
  const int64_t off = blockIdx.y * (int64_t)S * D;
  const int query = blockIdx.x * kRows + tid / 4;
  float q[D / 4], g[D / 4];
  double dq[D / 4];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) {
    q[e] = query < S ? Q[off + (int64_t)query * D + sub * (D / 4) + e] : 0.f;
    g[e] = query < S ? dO[off + (int64_t)query * D + sub * (D / 4) + e] : 0.f;
    dq[e] = 0.0;
  }
  const double lse = query < S ? LSE[blockIdx.y * (int64_t)S + query] : 0.f;
  const double dl = query < S ? DELTA[blockIdx.y * (int64_t)S + query] : 0.f;
  const int kend = min(S, (int)(blockIdx.x + 1) * kRows);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    __syncthreads();
    stage<D>(sK, K + off, S, k0, tid);
    stage<D>(sV, V + off, S, k0, tid);
    __syncthreads();
    for (int j = 0; j < kRows; ++j) {
      const float* kj = sK + j * D + sub * (D / 4);
      const double s = dot4<D>(q, kj) * scale;
      const double dp = dot4<D>(g, sV + j * D + sub * (D / 4));
      if (k0 + j > query) continue;
      const double ds = (double)expf((float)(s - lse)) * (dp - dl);
#pragma unroll
      for (int e = 0; e < D / 4; ++e) dq[e] = fma(ds, (double)kj[e], dq[e]);
    }
  }
  if (query >= S) return;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) dQ[off + (int64_t)query * D + sub * (D / 4) + e] = (float)(dq[e] * scale);
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int64_t S, int d, int64_t BH, hipStream_t st) {
  const dim3 grid((unsigned)((S + kRows - 1) / kRows), (unsigned)BH);
  const double scale = 1.0 / sqrt((double)d);
  if (d == 64) attn_fwd_f32<64><<<grid, 256, 0, st>>>(q, k, v, o, lse, (int)S, scale);
  else attn_fwd_f32<128><<<grid, 256, 0, st>>>(q, k, v, o, lse, (int)S, scale);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* lse,
                               const float* delta, const float* dout, float* dq, float* dk,
                               float* dv, int64_t S, int d, int64_t BH, hipStream_t st,
                               hipEvent_t* ev) {
  const dim3 grid((unsigned)((S + kRows - 1) / kRows), (unsigned)BH);
  const double scale = 1.0 / sqrt((double)d);
  if (d == 64) attn_bwd_dkdv_f32<64><<<grid, 256, 0, st>>>(q, k, v, dout, lse, delta, dk, dv, (int)S, scale);
  else attn_bwd_dkdv_f32<128><<<grid, 256, 0, st>>>(q, k, v, dout, lse, delta, dk, dv, (int)S, scale);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
  if (e != hipSuccess) return e;
  if (d == 64) attn_bwd_dq_f32<64><<<grid, 256, 0, st>>>(q, k, v, dout, lse, delta, dq, (int)S, scale);
  else attn_bwd_dq_f32<128><<<grid, 256, 0, st>>>(q, k, v, dout, lse, delta, dq, (int)S, scale);
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  return e;
}

}  // namespace lh

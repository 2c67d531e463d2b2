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

// x from the lane of this quad that the DPP quad permutation Ctl names
// (0xB1: lane ^ 1, 0x4E: lane ^ 2), both 32-bit halves moved in registers.
template <int Ctl>
__device__ __forceinline__ double quad_swap(double x) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), Ctl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), Ctl, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// q.k of one row: each of the row's four lanes (an aligned quad, all active
// together) sums its d/4 products, then the four partial sums are added.
template <int D>
__device__ __forceinline__ double dot4(const float (&a)[D / 4], const float* b) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) s = fma((double)a[e], (double)b[e], s);
  s += quad_swap<0xB1>(s);
  s += quad_swap<0x4E>(s);
  return s;
}

// Rows [r0, r0 + kRows) of two [S][D] tensors into LDS (rows >= S as
// zeros): 16-byte loads, every one of both tiles issued before the first LDS
// store, so a pair of tiles costs one memory latency rather than one per
// element.
template <int D>
__device__ __forceinline__ void stage(float* dst0, const float* src0, float* dst1, const float* src1,
                                      int S, int r0, int tid) {
  constexpr int kPer = kRows * D / 4 / 256;  // 16-byte chunks per thread and tile
  float4 v[2][kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = tid + k * 256;  // chunk of the tile: row c / (D / 4)
    const int r = c / (D / 4);
    const int64_t o = (int64_t)min(r0 + r, S - 1) * D;  // clamped: never read past the end
    const bool in = r0 + r < S;
    v[0][k] = reinterpret_cast<const float4*>(src0 + o)[c % (D / 4)];
    v[1][k] = reinterpret_cast<const float4*>(src1 + o)[c % (D / 4)];
    if (!in) v[0][k] = v[1][k] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    reinterpret_cast<float4*>(dst0)[tid + k * 256] = v[0][k];
    reinterpret_cast<float4*>(dst1)[tid + k * 256] = v[1][k];
  }
}

// This lane's quarter of a row (d/4 consecutive floats, 16-byte loads; src
// must point into the tensor), replaced by zeros when !ok (a row past the
// end: callers pass the last row's address then).
template <int N>
__device__ __forceinline__ void load_quarter(const float* src, bool ok, float (&x)[N]) {
  static_assert(N % 4 == 0, "whole 16-byte chunks");
  float4 v[N / 4];
#pragma unroll
  for (int i = 0; i < N / 4; ++i) v[i] = reinterpret_cast<const float4*>(src)[i];  // src is a valid row
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    if (!ok) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    x[4 * i] = v[i].x;
    x[4 * i + 1] = v[i].y;
    x[4 * i + 2] = v[i].z;
    x[4 * i + 3] = v[i].w;
  }
}

// Forward: a query's keys are split over kSplit lane groups (key j of a tile
// goes to group j mod kSplit), each with its own running max, normaliser and
// output; the groups of a query sit 4 lanes apart in one wave and are merged
// with butterfly shuffles at the end.  Splitting the keys gives a workgroup
// 256 / (4 kSplit) queries, so short sequences still spread over many
// workgroups and each lane's dependent chain is kSplit times shorter.
constexpr int kSplit = 16;

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                    const float* __restrict__ V, float* __restrict__ O,
                                                    float* __restrict__ LSE, int S, double scale) {
  constexpr int kQ = 256 / (4 * kSplit);  // queries per workgroup
  __shared__ float sK[kRows * D], sV[kRows * D];
  const int tid = threadIdx.x, sub = tid & 3, grp = (tid >> 2) % kSplit;
  const int64_t off = blockIdx.y * (int64_t)S * D;
  const int query = blockIdx.x * kQ + tid / (4 * kSplit);
  float q[D / 4];
  double o[D / 4];
  load_quarter(Q + off + (int64_t)min(query, S - 1) * D + sub * (D / 4), query < S, q);
#pragma unroll
  for (int e = 0; e < D / 4; ++e) o[e] = 0.0;
  double m = -1e300, l = 0.0;
  const int kend = min(S, (int)(blockIdx.x + 1) * kQ);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    __syncthreads();
    stage<D>(sK, K + off, sV, V + off, S, k0, tid);
    __syncthreads();
    // the group's keys of this tile: scores first (independent), then one
    // update of the running maximum, then the weights (independent)
    constexpr int kJ = kRows / kSplit;
    double sc[kJ];
    double mt = m;
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int j = jj * kSplit + grp;
      sc[jj] = dot4<D>(q, sK + j * D + sub * (D / 4)) * scale;
      if (k0 + j <= query) mt = fmax(mt, sc[jj]);
    }
    if (mt > m) {
      const double alpha = expf((float)(m - mt));
      l *= alpha;
#pragma unroll
      for (int e = 0; e < D / 4; ++e) o[e] *= alpha;
      m = mt;
    }
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int j = jj * kSplit + grp;
      if (k0 + j > query) continue;
      const double p = expf((float)(sc[jj] - m));
      l += p;
#pragma unroll
      for (int e = 0; e < D / 4; ++e) o[e] += p * (double)sV[j * D + sub * (D / 4) + e];
    }
  }
  // merge the key groups of each query (lanes 4, 8, 16, 32 apart); a group that
  // saw no key has l = 0 and o = 0, and its weight underflows to 0
#pragma unroll
  for (int w = 4; w < 4 * kSplit; w <<= 1) {
    const double mo = __shfl_xor(m, w), lo = __shfl_xor(l, w);
    const double mn = fmax(m, mo);
    const double a = expf((float)(m - mn)), b = expf((float)(mo - mn));
    l = l * a + lo * b;
#pragma unroll
    for (int e = 0; e < D / 4; ++e) o[e] = o[e] * a + __shfl_xor(o[e], w) * b;
    m = mn;
  }
  if (query >= S || grp != 0) return;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) O[off + (int64_t)query * D + sub * (D / 4) + e] = (float)(o[e] / l);
  if (sub == 0) LSE[blockIdx.y * (int64_t)S + query] = (float)(m + log(l));
}

// Backward passes: a row's work is split over kSplit lane groups as in the
// forward (item j of a tile goes to group j mod kSplit), so that a short
// sequence still yields many workgroups; the groups' float64 sums are added
// by butterfly shuffles at the end.  A lane takes a few items of a tile at
// a time, their dot products independent of each other.  (Two heads of 512
// rows: dK/dV 200 -> 31 us, dQ 163 -> 26 us against one lane group per row;
// 4 groups give 86 and 61 us, and 16 groups stay ahead at 4,096 rows.)
template <int D>
struct BwdCfg {
  static constexpr int kRowsPerBlock = 256 / (4 * kSplit);
  static constexpr int kItems = kRows / kSplit;   // items of a tile per lane group
  static constexpr int kUdq = D == 64 ? 4 : 2;    // items at a time: dQ pass
  static constexpr int kUdkdv = D == 64 ? 2 : 1;  // dK/dV pass (two sums per key)
  static_assert(kItems % kUdq == 0 && kItems % kUdkdv == 0, "whole steps per tile");
};

template <int N>
__device__ __forceinline__ void sum_groups(double (&x)[N]) {
#pragma unroll
  for (int w = 4; w < 4 * kSplit; w <<= 1) {
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] += __shfl_xor(x[e], w);
  }
}

// dK, dV: a workgroup owns kRowsPerBlock keys and walks the queries from its
// first key to the end; a probability P = exp(s - lse) of query i and key j
// adds P dO_i to dV_j and P (dP - delta_i) q_i to dK_j (scaled once at the
// end).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ dO,
                                                         const float* __restrict__ LSE,
                                                         const float* __restrict__ DELTA,
                                                         float* __restrict__ dK, float* __restrict__ dV,
                                                         int S, double scale) {
  using C = BwdCfg<D>;
  __shared__ float sQ[kRows * D], sG[kRows * D], sL[kRows], sDl[kRows];
  const int tid = threadIdx.x, sub = tid & 3, grp = (tid >> 2) % kSplit;
  const int64_t off = blockIdx.y * (int64_t)S * D;
  const int key0 = blockIdx.x * C::kRowsPerBlock;
  const int key = key0 + tid / (4 * kSplit);
  float k[D / 4], v[D / 4];
  double dk[D / 4], dv[D / 4];
  const int64_t krow = off + (int64_t)min(key, S - 1) * D + sub * (D / 4);
  load_quarter(K + krow, key < S, k);
  load_quarter(V + krow, key < S, v);
#pragma unroll
  for (int e = 0; e < D / 4; ++e) dk[e] = dv[e] = 0.0;
  for (int q0 = key0; q0 < S; q0 += kRows) {
    __syncthreads();
    stage<D>(sQ, Q + off, sG, dO + off, S, q0, tid);
    if (tid < kRows) {
      sL[tid] = q0 + tid < S ? LSE[blockIdx.y * (int64_t)S + q0 + tid] : 0.f;
      sDl[tid] = q0 + tid < S ? DELTA[blockIdx.y * (int64_t)S + q0 + tid] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < C::kItems; ii += C::kUdkdv) {
      double s[C::kUdkdv], dp[C::kUdkdv];
#pragma unroll
      for (int u = 0; u < C::kUdkdv; ++u) {
        const int i = (ii + u) * kSplit + grp;
        s[u] = dot4<D>(k, sQ + i * D + sub * (D / 4)) * scale;
        dp[u] = dot4<D>(v, sG + i * D + sub * (D / 4));
      }
#pragma unroll
      for (int u = 0; u < C::kUdkdv; ++u) {
        const int i = (ii + u) * kSplit + grp;
        const int query = q0 + i;
        if (query >= S || key > query) continue;
        const float* qi = sQ + i * D + sub * (D / 4);
        const float* gi = sG + i * D + sub * (D / 4);
        const double p = expf((float)(s[u] - (double)sL[i]));
        const double ds = p * (dp[u] - (double)sDl[i]);
#pragma unroll
        for (int e = 0; e < D / 4; ++e) {
          dv[e] = fma(p, (double)gi[e], dv[e]);
          dk[e] = fma(ds, (double)qi[e], dk[e]);
        }
      }
    }
  }
  sum_groups(dk);
  sum_groups(dv);
  if (key >= S || grp != 0) return;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) {
    dK[off + (int64_t)key * D + sub * (D / 4) + e] = (float)(dk[e] * scale);
    dV[off + (int64_t)key * D + sub * (D / 4) + e] = (float)dv[e];
  }
}

// dQ: a workgroup owns kRowsPerBlock queries and walks the keys up to its
// last query; dQ_i sums P (dP - delta_i) k_j (scaled once at the end).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       const float* __restrict__ DELTA,
                                                       float* __restrict__ dQ, int S, double scale) {
  using C = BwdCfg<D>;
  __shared__ float sK[kRows * D], sV[kRows * D];
  const int tid = threadIdx.x, sub = tid & 3, grp = (tid >> 2) % kSplit;
  const int64_t off = blockIdx.y * (int64_t)S * D;
  const int query = blockIdx.x * C::kRowsPerBlock + tid / (4 * kSplit);
  float q[D / 4], g[D / 4];
  double dq[D / 4];
  const int64_t qrow = off + (int64_t)min(query, S - 1) * D + sub * (D / 4);
  load_quarter(Q + qrow, query < S, q);
  load_quarter(dO + qrow, query < S, g);
#pragma unroll
  for (int e = 0; e < D / 4; ++e) dq[e] = 0.0;
  const double lse = query < S ? LSE[blockIdx.y * (int64_t)S + query] : 0.f;
  const double dl = query < S ? DELTA[blockIdx.y * (int64_t)S + query] : 0.f;
  const int kend = min(S, (int)(blockIdx.x + 1) * C::kRowsPerBlock);
  for (int k0 = 0; k0 < kend; k0 += kRows) {
    __syncthreads();
    stage<D>(sK, K + off, sV, V + off, S, k0, tid);
    __syncthreads();
    for (int jj = 0; jj < C::kItems; jj += C::kUdq) {
      double s[C::kUdq], dp[C::kUdq];
#pragma unroll
      for (int u = 0; u < C::kUdq; ++u) {
        const int j = (jj + u) * kSplit + grp;
        s[u] = dot4<D>(q, sK + j * D + sub * (D / 4)) * scale;
        dp[u] = dot4<D>(g, sV + j * D + sub * (D / 4));
      }
#pragma unroll
      for (int u = 0; u < C::kUdq; ++u) {
        const int j = (jj + u) * kSplit + grp;
        if (k0 + j > query) continue;
        const float* kj = sK + j * D + sub * (D / 4);
        const double ds = (double)expf((float)(s[u] - lse)) * (dp[u] - dl);
#pragma unroll
        for (int e = 0; e < D / 4; ++e) dq[e] = fma(ds, (double)kj[e], dq[e]);
      }
    }
  }
  sum_groups(dq);
  if (query >= S || grp != 0) return;
#pragma unroll
  for (int e = 0; e < D / 4; ++e) dQ[off + (int64_t)query * D + sub * (D / 4) + e] = (float)(dq[e] * scale);
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int64_t S, int d, int64_t BH, hipStream_t st) {
  constexpr int kQ = 256 / (4 * kSplit);
  const dim3 grid((unsigned)((S + kQ - 1) / kQ), (unsigned)BH);
  const double scale = 1.0 / sqrt((double)d);
  if (d == 64) attn_fwd_f32<64><<<grid, 256, 0, st>>>(q, k, v, o, lse, (int)S, scale);
  else attn_fwd_f32<128><<<grid, 256, 0, st>>>(q, k, v, o, lse, (int)S, scale);
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_passes(const float* q, const float* k, const float* v, const float* lse,
                             const float* delta, const float* dout, float* dq, float* dk, float* dv,
                             int64_t S, int64_t BH, hipStream_t st, hipEvent_t* ev) {
  using C = BwdCfg<D>;
  const dim3 grid((unsigned)((S + C::kRowsPerBlock - 1) / C::kRowsPerBlock), (unsigned)BH);
  const double scale = 1.0 / sqrt((double)D);
  attn_bwd_dkdv_f32<D><<<grid, 256, 0, st>>>(q, k, v, dout, lse, delta, dk, dv, (int)S, scale);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
  if (e != hipSuccess) return e;
  attn_bwd_dq_f32<D><<<grid, 256, 0, st>>>(q, k, v, dout, lse, delta, dq, (int)S, scale);
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  return e;
}

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* lse,
                               const float* delta, const float* dout, float* dq, float* dk,
                               float* dv, int64_t S, int d, int64_t BH, hipStream_t st,
                               hipEvent_t* ev) {
  return d == 64 ? bwd_passes<64>(q, k, v, lse, delta, dout, dq, dk, dv, S, BH, st, ev)
                 : bwd_passes<128>(q, k, v, lse, delta, dout, dq, dk, dv, S, BH, st, ev);
}

}  // namespace lh

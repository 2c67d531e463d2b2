// Causal gather (gist.science technical summary §2.C; bitsgeniais post,
// phase 3): the selected candidates plus the whole coarsest level form the
// subsequence, ordered by (end token, level) ascending, where entry (l, j)
// ends at token (j+1)*p^l - 1.
//
// No sort is needed: the position of an entry is the number of chosen entries
// with a smaller key, summed level by level.  For level m that count is the
// number of chosen level-m entries with index below a bound that follows from
// the key comparison:
//   m <  l :  i < (j+1) * p^(l-m)          (end <= own end; lower level first)
//   m == l :  i < j
//   m >  l :  i < floor(end / p^m)         (end strictly before own end)
// Chosen candidates of a level are a contiguous, sorted run of `sel` (which
// is in ascending flat order), so each count is a difference of two ranks in
// `sel`; the coarsest level is chosen whole, so its count is the bound
// itself.
//
// One launch.  A block places 64 positions.  Its threads rank the level
// starts of `sel` once, then take one (entry, level) pair each, so the
// dependent loads of the rank searches run as short chains in parallel.  A
// rank search narrows to a window of `stride` entries with samples of `sel`
// staged in LDS (every stride-th entry, as dense as 2,048 samples allow: all
// of `sel` up to 2,048 candidates, every 4th at 7,808), then quarters that
// window in global memory (three pivots per round trip; `sel` is small and
// stays cached; no round trip for windows of up to 16) and counts the last
// <= 16 entries directly.  The source rows are loaded before
// the searches (they follow from the entries alone) and stored after them.
// The same block writes pos for the flat range from after the previous
// block's last entry to its own last entry (to C for the last block; the
// whole candidate range split evenly when K = 0): -1 everywhere first, then,
// after those stores have completed and a barrier, the positions of its
// entries.
#include <algorithm>

#include "kernels.h"

namespace lh {

namespace {

constexpr int kEntries = 64;      // subsequence positions per block
constexpr int kThreads = 256;     // four (entry, level) pairs per entry at a time
constexpr int kMaxSamples = 2048; // staged samples of sel
#ifndef LH_GATHER_MINSTRIDE
#define LH_GATHER_MINSTRIDE 1
#endif

struct Ranker {
  const int32_t* a;      // sorted ascending, n entries
  const int32_t* samp;   // LDS: samp[i] = a[i * stride], i < ns
  int32_t n, ns, stride;

  // number of entries of a below key
  __device__ __forceinline__ int32_t rank(int32_t key) const {
    // window from the samples: the first sample not below key
    int32_t l = 0, h = ns;
    while (l < h) {
      const int32_t mid = (l + h) >> 1;
      if (samp[mid] < key) l = mid + 1;
      else h = mid;
    }
    if (l == 0) return 0;            // a[0] >= key
    int32_t lo = (l - 1) * stride + 1;  // a[lo - 1] < key
    int32_t hi = min(l * stride, n);    // a[hi] >= key (or the end)
    // quarter the window: pivots lo + q, lo + 2q, lo + 3q < hi, all loaded at once
    while (hi - lo > 16) {
      const int32_t q = (hi - lo + 3) >> 2;
      const int32_t v1 = a[lo + q], v2 = a[lo + 2 * q], v3 = a[lo + 3 * q];
      if (v3 < key) {
        lo = lo + 3 * q + 1;
      } else if (v2 < key) {
        hi = lo + 3 * q;
        lo = lo + 2 * q + 1;
      } else if (v1 < key) {
        hi = lo + 2 * q;
        lo = lo + q + 1;
      } else {
        hi = lo + q;
      }
    }
    int32_t r = lo;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (lo + i < hi && a[lo + i] < key) ++r;
    return r;
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const int32_t* sel, const void* q, const void* k, const void* v, Lay lq, const void* pq,
    const void* pk, const void* pv, int32_t* sub_idx, int32_t* pos, void* qs, void* ks, void* vs,
    Geo g, int32_t stride, int32_t ns) {
  __shared__ int32_t samp[kMaxSamples];
  __shared__ int32_t s_base[kMaxLevels], s_pw[kMaxLevels], s_seg[kMaxLevels];
  __shared__ int32_t s_raw[kEntries];   // sel entries of this block (candidate blocks)
  __shared__ int32_t s_f[kEntries], s_l[kEntries], s_j[kEntries], s_cnt[kEntries];
  __shared__ int32_t s_pos[kEntries];
  const int64_t bh = blockIdx.y;
  const int32_t* sl = sel + bh * g.K;   // never dereferenced when K == 0
  int32_t* ph = pos + bh * g.M;
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.x * kEntries;
  const int32_t n = i0 < g.K ? (int32_t)min<int64_t>(kEntries, g.K - i0) : 0;
  const Ranker r{sl, samp, g.K, ns, stride};

  {  // every sample load of a thread in flight before its first LDS store
    constexpr int kPer = kMaxSamples / kThreads;
    int32_t sv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kThreads;
      sv[k] = i < ns ? sl[(int64_t)i * stride] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (tid + k * kThreads < ns) samp[tid + k * kThreads] = sv[k];
  }
  if (tid < g.L) {
    s_base[tid] = g.base[tid];
    s_pw[tid] = g.pw[tid];
  }
  if (tid < n) s_raw[tid] = sl[i0 + tid];
  __syncthreads();

  // the entries (flat index, level, index in level, coarsest count); the
  // rank of every level start in sel
  if (tid < kEntries) {
    const int64_t idx = i0 + tid;
    int32_t f = -1, l = 0, j = 0, cnt = 0;
    if (idx < g.S) {
      f = idx < g.K ? s_raw[tid] : s_base[g.L - 1] + (int32_t)(idx - g.K);
      if (f >= 0 && f < g.M) {
        while (l + 1 < g.L && f >= s_base[l + 1]) ++l;
        j = f - s_base[l];
        const int64_t end = (int64_t)(j + 1) * s_pw[l] - 1;
        cnt = l == g.L - 1 ? j : (int32_t)(end / s_pw[g.L - 1]);
      } else {
        f = -1;  // a malformed selection leaves the slot unplaced
      }
    }
    s_f[tid] = f;
    s_l[tid] = l;
    s_j[tid] = j;
    s_cnt[tid] = cnt;
  } else if (tid - kEntries < g.L - 1) {
    s_seg[tid - kEntries] = r.rank(s_base[tid - kEntries]);
  }
  __syncthreads();

  // Row copies: 16-byte chunks c -> (entry, tensor, chunk), chunks of one row
  // on consecutive lanes.  The source row follows from the entry alone, so
  // the first kPre chunks of every thread are loaded now and stored once the
  // positions are known: the loads overlap the rank searches.
  constexpr int es = sizeof(T);
  const int cpr = g.d * es / 16;  // chunks per row
  const int total = kEntries * 3 * cpr;
  auto src_of = [&](int e, int t) -> const f32x4* {
    const int32_t l = s_l[e];
    const void* base = l == 0 ? (t == 0 ? q : (t == 1 ? k : v)) : (t == 0 ? pq : (t == 1 ? pk : pv));
    const int64_t el = l == 0 ? lq.head(bh) + s_j[e] * lq.sn
                              : (bh * (int64_t)(g.M - g.N) + (s_f[e] - g.N)) * g.d;
    return reinterpret_cast<const f32x4*>(static_cast<const char*>(base) + el * es);
  };
  auto dst_of = [&](int t, int32_t p) -> f32x4* {
    void* base = t == 0 ? qs : (t == 1 ? ks : vs);
    return reinterpret_cast<f32x4*>(static_cast<char*>(base) + (bh * g.S + p) * g.d * es);
  };
  constexpr int kPre = 12;
  f32x4 pre[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int c = tid + u * kThreads;
    if (c >= total) break;
    const int e = c / (3 * cpr), rem = c % (3 * cpr);
    if (s_f[e] >= 0) pre[u] = src_of(e, rem / cpr)[rem % cpr];
  }

  // -1 over this block's flat range (stores only; they overlap the searches)
  {
    int64_t a = 0, b = 0;
    if (g.K == 0) {
      const int64_t per = ((int64_t)g.C + gridDim.x - 1) / gridDim.x;
      a = (int64_t)blockIdx.x * per;
      b = min(a + per, (int64_t)g.C);
    } else if (n > 0) {
      a = max(i0 == 0 ? 0 : sl[i0 - 1] + 1, 0);
      b = i0 + n == g.K ? (int64_t)g.C : min(s_raw[n - 1], g.C - 1);  // last entry: placed below
    }
    for (int64_t x = a + tid; x < b; x += kThreads) ph[x] = -1;
  }

  // counts of levels 0..L-2, one (entry, level) pair per thread
  {
    const int e = tid % kEntries;
    const int32_t f = s_f[e];
    if (f >= 0) {
      const int32_t l = s_l[e], j = s_j[e];
      const int64_t end = (int64_t)(j + 1) * s_pw[l] - 1;
      int32_t acc = 0;
      for (int m = tid / kEntries; m < g.L - 1; m += kThreads / kEntries) {
        int64_t bound;
        if (m < l) bound = (int64_t)(j + 1) * s_pw[l - m];
        else if (m == l) bound = j;
        else bound = end / s_pw[m];
        acc += r.rank(s_base[m] + (int32_t)bound) - s_seg[m];
      }
      if (acc) atomicAdd(&s_cnt[e], acc);
    }
  }
  // the -1 stores above have completed before any thread of the block
  // overwrites a slot of its range with a position
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (tid < kEntries) {
    const int32_t f = s_f[tid];
    int32_t p = -1;
    if (f >= 0) {
      // always true for a valid selection; an unsorted one could give any count
      if (s_cnt[tid] >= 0 && s_cnt[tid] < g.S) {
        p = s_cnt[tid];
        sub_idx[bh * g.S + p] = f;
      }
      ph[f] = p;
    }
    s_pos[tid] = p;
  }
  __syncthreads();

  // store the preloaded chunks, then copy the rest with kU loads in flight
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int c = tid + u * kThreads;
    if (c >= total) break;
    const int e = c / (3 * cpr), rem = c % (3 * cpr);
    const int32_t p = s_pos[e];
    if (p >= 0) dst_of(rem / cpr, p)[rem % cpr] = pre[u];
  }
  constexpr int kU = 4;
  for (int c0 = tid + kPre * kThreads; c0 < total; c0 += kU * kThreads) {
    f32x4 val[kU];
    f32x4* to[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      to[u] = nullptr;
      const int c = c0 + u * kThreads;
      if (c >= total) continue;
      const int e = c / (3 * cpr), rem = c % (3 * cpr);
      const int32_t p = s_pos[e];
      if (p < 0) continue;
      val[u] = src_of(e, rem / cpr)[rem % cpr];
      to[u] = dst_of(rem / cpr, p) + rem % cpr;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (to[u]) *to[u] = val[u];
  }
}

}  // namespace

hipError_t launch_gather(const int32_t* sel, const void* const qkv[3], const Lay& lq,
                         const void* const pyr[3], int32_t* sub_idx, int32_t* pos,
                         void* const sub[3], const Geo& g, int dtype, int64_t BH, hipStream_t st) {
  if (g.S == 0) return hipSuccess;
  // sample stride: the smallest that keeps at most kMaxSamples samples (1,
  // all of sel in LDS, up to 2,048 candidates), at least LH_GATHER_MINSTRIDE
  const int64_t K = g.K;
  const int64_t stride = std::max<int64_t>(LH_GATHER_MINSTRIDE, (K + kMaxSamples - 1) / kMaxSamples);
  const int32_t ns = (int32_t)((K + stride - 1) / stride);
  const dim3 grid((unsigned)((g.S + kEntries - 1) / kEntries), (unsigned)BH);
  if (dtype == 1)
    gather_kernel<__bf16><<<grid, kThreads, 0, st>>>(sel, qkv[0], qkv[1], qkv[2], lq, pyr[0], pyr[1],
                                                     pyr[2], sub_idx, pos, sub[0], sub[1], sub[2],
                                                     g, (int32_t)stride, ns);
  else
    gather_kernel<float><<<grid, kThreads, 0, st>>>(sel, qkv[0], qkv[1], qkv[2], lq, pyr[0], pyr[1],
                                                    pyr[2], sub_idx, pos, sub[0], sub[1], sub[2],
                                                    g, (int32_t)stride, ns);
  return hipGetLastError();
}

}  // namespace lh

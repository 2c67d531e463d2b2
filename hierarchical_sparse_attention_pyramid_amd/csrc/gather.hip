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
// is in ascending flat order), so each count is one binary search; the
// coarsest level is chosen whole, so its count is the bound itself.
#include "kernels.h"

namespace lh {

namespace {

constexpr int kEntries = 64;   // entries placed per block

__global__ void fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < n; k += stride) p[k] = v;
}

// first index in sorted a[lo, hi) with a[idx] >= key
__device__ __forceinline__ int32_t lower_bound(const int32_t* a, int32_t lo, int32_t hi,
                                               int32_t key) {
  while (lo < hi) {
    const int32_t mid = lo + ((hi - lo) >> 1);
    if (a[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

template <typename T>
__global__ __launch_bounds__(256) void gather_place(const int32_t* sel, const void* q, const void* k,
                                                    const void* v, const void* pq, const void* pk,
                                                    const void* pv, int32_t* sub_idx, int32_t* pos,
                                                    void* qs, void* ks, void* vs, Geo g) {
  __shared__ int32_t seg[kMaxLevels + 1];
  __shared__ int32_t s_pos[kEntries];
  __shared__ int64_t s_src[kEntries];   // source row: token (>= 0) or -(pyramid row) - 1
  const int64_t bh = blockIdx.y;
  const int32_t* sl = sel + bh * g.K;
  const int tid = threadIdx.x;
  if (tid < g.L - 1) seg[tid] = lower_bound(sl, 0, g.K, g.base[tid]);
  if (tid == 0) seg[g.L - 1] = g.K;
  __syncthreads();

  if (tid < kEntries) {
    const int64_t idx = (int64_t)blockIdx.x * kEntries + tid;
    s_pos[tid] = -1;
    const int32_t f = idx >= g.S ? -1 : (idx < g.K ? sl[idx] : g.base[g.L - 1] + (int32_t)(idx - g.K));
    if (f >= 0 && f < g.M) {  // a malformed selection leaves the slot unwritten
      int l = 0;
      while (l + 1 < g.L && f >= g.base[l + 1]) ++l;
      const int32_t j = f - g.base[l];
      const int64_t end = (int64_t)(j + 1) * g.pw[l] - 1;
      int64_t p = 0;
      for (int m = 0; m < g.L; ++m) {
        int64_t bound;
        if (m < l) bound = (int64_t)(j + 1) * g.pw[l - m];
        else if (m == l) bound = j;
        else bound = end / g.pw[m];
        if (m == g.L - 1) {
          p += bound;
        } else {
          p += lower_bound(sl, seg[m], seg[m + 1], g.base[m] + (int32_t)bound) - seg[m];
        }
      }
      if (p < g.S) {  // always true for a valid selection; never write past S
        s_pos[tid] = (int32_t)p;
        sub_idx[bh * g.S + p] = f;
        pos[bh * g.M + f] = (int32_t)p;
        s_src[tid] = l == 0 ? (int64_t)j : -(int64_t)(f - g.N) - 1;
      }
    }
  }
  __syncthreads();

  // copy rows: 16-byte chunks, (q, k, v) x kEntries rows
  constexpr int es = sizeof(T);
  const int cpr = g.d * es / 16;  // chunks per row
  const void* lv0[3] = {q, k, v};
  const void* pyr[3] = {pq, pk, pv};
  void* dst[3] = {qs, ks, vs};
  const int total = kEntries * 3 * cpr;
  for (int c = tid; c < total; c += blockDim.x) {
    const int e = c / (3 * cpr);
    const int rem = c % (3 * cpr);
    const int t = rem / cpr, ch = rem % cpr;
    const int32_t p = s_pos[e];
    if (p < 0) continue;
    const int64_t srow = s_src[e];
    const char* src = srow >= 0
        ? static_cast<const char*>(lv0[t]) + ((bh * g.N + srow) * g.d) * es
        : static_cast<const char*>(pyr[t]) + ((bh * (int64_t)(g.M - g.N) + (-srow - 1)) * g.d) * es;
    char* d = static_cast<char*>(dst[t]) + ((bh * g.S + p) * g.d) * es;
    reinterpret_cast<f32x4*>(d)[ch] = reinterpret_cast<const f32x4*>(src)[ch];
  }
}

}  // namespace

hipError_t launch_gather(const int32_t* sel, const void* const qkv[3], const void* const pyr[3],
                         int32_t* sub_idx, int32_t* pos, void* const sub[3], const Geo& g,
                         int dtype, int64_t BH, hipStream_t st) {
  const int64_t npos = BH * (int64_t)g.M;
  const int64_t fblocks = (npos + 255) / 256 < 4096 ? (npos + 255) / 256 : 4096;
  fill_i32<<<(unsigned)fblocks, 256, 0, st>>>(pos, npos, -1);
  const dim3 grid((unsigned)((g.S + kEntries - 1) / kEntries), (unsigned)BH);
  if (dtype == 1)
    gather_place<__bf16><<<grid, 256, 0, st>>>(sel, qkv[0], qkv[1], qkv[2], pyr[0], pyr[1], pyr[2],
                                               sub_idx, pos, sub[0], sub[1], sub[2], g);
  else
    gather_place<float><<<grid, 256, 0, st>>>(sel, qkv[0], qkv[1], qkv[2], pyr[0], pyr[1], pyr[2],
                                              sub_idx, pos, sub[0], sub[1], sub[2], g);
  return hipGetLastError();
}

}  // namespace lh

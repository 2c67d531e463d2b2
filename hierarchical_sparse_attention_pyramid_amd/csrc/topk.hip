// Joint top-K over pyramid levels 0..L-2 (gist.science technical summary
// §2.B; bitsgeniais post, phase 2): the K candidates first under the strict
// order (score descending, flat index ascending), written in ascending flat
// order.
//
// The gist.science summary (§2.B) and the bitsgeniais post (phase 2) name a
// fused chunked-bitonic top-K kernel; the operating points they report
// select k = 1536 candidates.  Here K reaches 32K out of 1.4M candidates per
// head, so the selection is an exact radix select on the float32 score bits
// instead (scores are non-negative, so their bit patterns order like the
// values; other bit patterns rank by their unsigned value).  It finds the
// score T of the K-th candidate and how many candidates equal to T are
// still needed (`need`), then keeps every candidate above T and the first
// `need` equal to T in flat order.  Integer work only: one deterministic
// answer.
//
// On this GPU a dependent kernel launch costs about 4-5 us whatever its
// size, so the design minimises launches rather than bytes:
//
//  * C <= 16384 candidates per head: one workgroup per head holds all of
//    its scores in LDS and runs three histogram passes (11 + 11 + 10 bits)
//    and the ordered compaction there: one launch, no workspace.
//  * larger heads: two 16-bit digits, three launches, and no separate
//    counting pass.
//      h0: histogram of the top 16 bits (per workgroup a direct-mapped LDS
//          table of packed 16-bit counters for the few coarse bins -- top 8
//          bits -- that its slices touch, then integer atomics into the
//          head's global coarse and fine -- top 16 bits -- histograms);
//      h1: every workgroup picks the pass-0 bin P0 from those histograms;
//          then, per 4096-candidate slice, it counts the candidates above
//          P0 and counting-sorts the ones inside P0 by bits 15..8 into a
//          per-slice record (offsets E and the low 16 bits of each), adding
//          the per-bin totals to the head's pass-1 coarse histogram;
//      w:  each workgroup picks T from the pass-1 coarse histogram and the
//          records' entries in the chosen coarse bin (usually a handful),
//          counts the candidates its earlier slices select from the
//          records alone (the slices' totals above P0, E, and those few
//          entries), and compacts its own slices in flat order.
//    The global histograms start each call at zero (a small clearing
//    kernel).  In lh_forward the pooling kernel that writes the scores also
//    does h0's counting (hist0.h), so the top-K stage itself is h1 and w.
#include "hist0.h"
#include "kernels.h"

namespace lh {

namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 4096;              // candidates per slice
constexpr int kPer = kSlice / kThreads;   // candidates per thread and slice
constexpr int kSmallThreads = 1024;
constexpr int kMaxSub = 15;               // slices per h0 workgroup: its LDS counters are 16-bit
#ifndef LH_TOPK_WG
#define LH_TOPK_WG 2048
#endif

// Workspace of the large-head path, per head (uint32 words):
//   [0, 8)                     header: P0 (pass-0 bin), rem0 (still needed inside it)
//   [kC0, kC0 + 256)           pass-0 coarse histogram (score bits 31..24)
//   [kF0, kF0 + 65536)         pass-0 fine histogram (score bits 31..16)
//   [kC1, kC1 + 256)           pass-1 coarse histogram (bits 15..8 of the candidates in P0)
//   [kSliceBase + s * kSliceWords, ...) record of slice s:
//       +0 candidates above P0, +1 candidates inside P0 (n),
//       +2 E[256] (uint16): entries whose bits 15..8 exceed b start at E[b],
//       +130 entries[4096] (uint16): low 16 bits, grouped by bits 15..8, descending.
// Words [kHdr, kZeroEnd) must be zero when h0 starts.
constexpr int kHdr = kTopkC0;
constexpr int kC0 = kTopkC0;
constexpr int kF0 = kTopkF0;
static_assert(kF0 == kC0 + 256, "pass-0 histogram layout");
constexpr int kC1 = kF0 + 65536;
constexpr int kZeroEnd = kC1 + 256;
constexpr int kSliceBase = (kZeroEnd + 63) / 64 * 64;
constexpr int kRecE = 2;
constexpr int kRecEnt = 2 + 128;
constexpr int kSliceWords = kRecEnt + kSlice / 2;

__device__ __forceinline__ uint32_t* head_ws(void* ws, int64_t bh, int64_t stride) {
  return static_cast<uint32_t*>(ws) + bh * stride;
}
__device__ __forceinline__ uint32_t* slice_rec(uint32_t* w, int s) {
  return w + kSliceBase + (int64_t)s * kSliceWords;
}

// Exclusive prefix sum over the NT threads of a block (in thread order);
// `sh` holds NT / 64 words.  Two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    if (k < wv) before += sh[k];
    total += sh[k];
  }
  __syncthreads();
  return before + x - v;
}

// Descending pick over 256 bins held one per thread (thread t holds bin
// 255 - t, count c): the bin holding the rem-th largest candidate and how
// many of that bin are still needed.  Same result in every thread.
__device__ __forceinline__ void pick256(uint32_t c, uint32_t rem, uint32_t* sh, uint32_t* res,
                                        uint32_t& bin, uint32_t& rem_out) {
  if (threadIdx.x == 0) {  // kept if no bin holds it (rem beyond the total: not for valid K)
    res[0] = 0;
    res[1] = rem;
  }
  uint32_t total;
  const uint32_t before = block_excl_scan<kThreads>(c, sh, total);  // its barriers order res
  if (before < rem && rem <= before + c) {
    res[0] = 255 - threadIdx.x;
    res[1] = rem - before;
  }
  __syncthreads();
  bin = res[0];
  rem_out = res[1];
  __syncthreads();  // res may be reused
}

// Candidates i0 + r * 256 + t of a slice (lane-consecutive loads); past C: 0.
__device__ __forceinline__ void load_slice(const float* s, int i0, int C, uint32_t (&u)[kPer]) {
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = i0 + r * kThreads + (int)threadIdx.x;
    u[r] = i < C ? __float_as_uint(s[i]) : 0u;
  }
}

// ---------------------------------------------------------------------------
// Small heads: everything in one workgroup's LDS.
constexpr int kSmallC = 16384;

__global__ __launch_bounds__(kSmallThreads) void topk_small(const float* score, int32_t* sel,
                                                            int32_t M, int32_t C, int32_t K) {
  constexpr int NT = kSmallThreads;
  __shared__ uint32_t keys[kSmallC];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh[NT / 64];
  __shared__ uint32_t res[2];
  const int64_t bh = blockIdx.x;
  const float* s = score + bh * M;
  for (int i = threadIdx.x; i < C; i += NT) keys[i] = __float_as_uint(s[i]);
  uint32_t prefix = 0, rem = (uint32_t)K;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbits = pass == 2 ? 10 : 11;
    const int nb = 1 << nbits;
    const int hi = shift + nbits;
    for (int b = threadIdx.x; b < 2048; b += NT) hist[b] = 0;
    __syncthreads();  // also publishes keys (first pass)
    for (int i = threadIdx.x; i < C; i += NT) {
      const uint32_t u = keys[i];
      if (hi >= 32 || ((u ^ prefix) >> hi) == 0u) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    if (threadIdx.x == 0) {
      res[0] = prefix;
      res[1] = rem;
    }
    __syncthreads();
    // thread t owns bins nb-1-t*per .. nb-per-t*per (descending)
    const int per = nb / NT;
    uint32_t cnt[2] = {0u, 0u};
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < per) cnt[j] = hist[nb - 1 - ((int)threadIdx.x * per + j)];
      local += cnt[j];
    }
    uint32_t total;
    const uint32_t before = block_excl_scan<NT>(local, sh, total);
    if (before < rem && rem <= before + local) {
      uint32_t cum = before;
      for (int j = 0; j < per; ++j) {
        const uint32_t c = cnt[j];
        if (cum + c >= rem) {
          res[0] = prefix | ((uint32_t)(nb - 1 - ((int)threadIdx.x * per + j)) << shift);
          res[1] = rem - cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    prefix = res[0];
    rem = res[1];
    __syncthreads();
  }
  const uint32_t T = prefix, need = rem;
  // ordered compaction: thread t owns the candidates t*E .. t*E + E - 1
  const int E = (C + NT - 1) / NT;  // <= 16
  const int first = (int)threadIdx.x * E;
  const int cnt = max(0, min(E, C - first));
  uint32_t neq = 0;
  for (int r = 0; r < cnt; ++r) neq += keys[first + r] == T ? 1u : 0u;
  uint32_t total;
  uint32_t eqr = block_excl_scan<NT>(neq, sh, total);
  uint32_t take = 0, ntake = 0;
  for (int r = 0; r < cnt; ++r) {
    const uint32_t u = keys[first + r];
    const bool is_eq = u == T;
    const bool t = u > T || (is_eq && eqr < need);
    eqr += is_eq ? 1u : 0u;
    take |= (t ? 1u : 0u) << r;
    ntake += t ? 1u : 0u;
  }
  uint32_t o = block_excl_scan<NT>(ntake, sh, total);
  int32_t* out = sel + bh * K;
  for (int r = 0; r < cnt; ++r) {
    if ((take >> r) & 1u) {
      if (o < (uint32_t)K) out[o] = first + r;  // bound: never past K
      ++o;
    }
  }
}

// ---------------------------------------------------------------------------
// Large heads.

// Clears words [kHdr, kZeroEnd) of every head (lh_topk only; in lh_forward
// the pooling kernel does it).
// workgroups per head of topk_zero: about one 16-byte store per thread
constexpr int kZeroBlocks = ((kZeroEnd - kHdr) / 4 + kThreads - 1) / kThreads;

__global__ __launch_bounds__(kThreads) void topk_zero(void* ws, int64_t stride) {
  constexpr int kVec = (kZeroEnd - kHdr) / 4;
  uint4* z = reinterpret_cast<uint4*>(head_ws(ws, blockIdx.y, stride) + kHdr);
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < kVec; i += gridDim.x * kThreads)
    z[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Pass 0: histogram of bits 31..16 over slices [s0, s1) of one head, in the
// LDS table of hist0.h (the slice loop needs no barrier).
__global__ __launch_bounds__(kThreads) void topk_h0(const float* score, void* ws, int64_t stride,
                                                    int32_t M, int32_t C, int32_t nsl, int32_t nsub) {
  __shared__ Hist0Lds hl;
  const int64_t bh = blockIdx.y;
  uint32_t* w = head_ws(ws, bh, stride);
  const float* s = score + bh * M;
  const int t = threadIdx.x;
  const int s0 = blockIdx.x * nsub, s1 = min(s0 + nsub, nsl);
  uint32_t u[kPer];
  if (s0 < s1) load_slice(s, s0 * kSlice, C, u);
  hist0_init(hl);
  __syncthreads();
  for (int sl = s0; sl < s1; ++sl) {
    const int i0 = sl * kSlice;
    uint32_t nx[kPer];
    const bool more = sl + 1 < s1;
    if (more) load_slice(s, (sl + 1) * kSlice, C, nx);
#pragma unroll
    for (int r = 0; r < kPer; ++r)
      if (i0 + r * kThreads + t < C) hist0_add(hl, u[r], w);
    if (more) {
#pragma unroll
      for (int r = 0; r < kPer; ++r) u[r] = nx[r];
    }
  }
  __syncthreads();
  hist0_flush(hl, w);
}

// Pick of pass 0, then the per-slice records and the pass-1 coarse histogram.
__global__ __launch_bounds__(kThreads) void topk_h1(const float* score, void* ws, int64_t stride,
                                                    int32_t M, int32_t C, int32_t K, int32_t nsl,
                                                    int32_t nsub) {
  __shared__ uint32_t sh[kThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t cnt[256], cur[256];
  const int64_t bh = blockIdx.y;
  uint32_t* w = head_ws(ws, bh, stride);
  const float* s = score + bh * M;
  const int s0 = blockIdx.x * nsub, s1 = min(s0 + nsub, nsl);
  uint32_t u[kPer];
  if (s0 < s1) load_slice(s, s0 * kSlice, C, u);  // overlaps the pick's loads
  const int t = threadIdx.x;
  uint32_t cb, r1, fb, rem0;
  pick256(w[kC0 + 255 - t], (uint32_t)K, sh, res, cb, r1);
  pick256(w[kF0 + (cb << 8) + 255 - t], r1, sh, res, fb, rem0);
  const uint32_t P0 = (cb << 8) | fb;
  if (blockIdx.x == 0 && t == 0) {
    w[0] = P0;
    w[1] = rem0;
  }
  for (int sl = s0; sl < s1; ++sl) {
    const int i0 = sl * kSlice;
    cnt[t] = 0u;
    __syncthreads();
    uint32_t gt = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if (i0 + r * kThreads + t < C) {
        const uint32_t k16 = u[r] >> 16;
        gt += k16 > P0 ? 1u : 0u;
        if (k16 == P0) atomicAdd(&cnt[(u[r] >> 8) & 255u], 1u);
      }
    }
    __syncthreads();
    uint32_t* rec = slice_rec(w, sl);
    const uint32_t c = cnt[255 - t];
    uint32_t n;
    const uint32_t before = block_excl_scan<kThreads>(c, sh, n);  // entries above bin 255 - t
    reinterpret_cast<uint16_t*>(rec + kRecE)[255 - t] = (uint16_t)before;
    cur[255 - t] = before;
    if (c) atomicAdd(&w[kC1 + 255 - t], c);
    uint32_t gtot;
    block_excl_scan<kThreads>(gt, sh, gtot);  // its barriers also publish cur
    if (t == 0) {
      rec[0] = gtot;
      rec[1] = n;
    }
    uint16_t* ent = reinterpret_cast<uint16_t*>(rec + kRecEnt);
    uint32_t nx[kPer];
    const bool more = sl + 1 < s1;
    if (more) load_slice(s, (sl + 1) * kSlice, C, nx);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if (i0 + r * kThreads + t < C && (u[r] >> 16) == P0) {
        const uint32_t slot = atomicAdd(&cur[(u[r] >> 8) & 255u], 1u);
        ent[slot] = (uint16_t)(u[r] & 0xFFFFu);
      }
    }
    if (more) {
#pragma unroll
      for (int r = 0; r < kPer; ++r) u[r] = nx[r];
    }
    __syncthreads();  // cnt and cur are rewritten by the next slice
  }
}

// Pick of T, offsets from the earlier slices' records, ordered compaction of
// this workgroup's slices [s0, s1).
__global__ __launch_bounds__(kThreads) void topk_w(const float* score, int32_t* sel, void* ws,
                                                   int64_t stride, int32_t M, int32_t C, int32_t K,
                                                   int32_t nsl, int32_t spw) {
  constexpr int kList = 2048;  // earlier slices' entries of the chosen coarse bin kept in LDS
  __shared__ uint32_t sh[kThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t fh[256];
  __shared__ uint8_t early[kList];
  __shared__ uint32_t nearly;
  __shared__ uint4 tile[kSlice / 4];  // a slice's score bits in flat order
  const int64_t bh = blockIdx.y;
  const int s0 = blockIdx.x * spw, s1 = min(s0 + spw, nsl);
  if (s0 >= s1) return;  // uniform per workgroup
  uint32_t* w = head_ws(ws, bh, stride);
  const float* s = score + bh * M;
  int32_t* out = sel + bh * K;
  const int t = threadIdx.x;
  uint32_t v[kPer];
  load_slice(s, s0 * kSlice, C, v);  // the first own slice, ahead of the picks
  const uint32_t P0 = w[0], rem0 = w[1];
  fh[t] = 0u;
  if (t == 0) nearly = 0u;
  uint32_t thi, r1, tlo, need;
  pick256(w[kC1 + 255 - t], rem0, sh, res, thi, r1);  // its barriers publish fh, nearly
  // one pass over every slice's record: fine counts of the entries in coarse
  // bin thi; for the slices before s0 also the candidates above that bin and
  // (in LDS) those entries' low bytes
  uint32_t gt_part = 0;
  for (int q = t; q < nsl; q += kThreads) {
    const uint32_t* rec = slice_rec(w, q);
    const uint16_t* E = reinterpret_cast<const uint16_t*>(rec + kRecE);
    const uint16_t* ent = reinterpret_cast<const uint16_t*>(rec + kRecEnt);
    const uint32_t lo = E[thi], hi = thi > 0 ? E[thi - 1] : rec[1];
    if (q < s0) gt_part += rec[0] + lo;
    for (uint32_t i = lo; i < hi; ++i) {
      const uint32_t x = ent[i] & 255u;
      atomicAdd(&fh[x], 1u);
      if (q < s0) {
        const uint32_t j = atomicAdd(&nearly, 1u);
        if (j < kList) early[j] = (uint8_t)x;
      }
    }
  }
  __syncthreads();
  pick256(fh[255 - t], r1, sh, res, tlo, need);
  const uint32_t T = (P0 << 16) | (thi << 8) | tlo;
  uint32_t eq_part = 0;
  if (nearly <= kList) {
    for (uint32_t i = t; i < nearly; i += kThreads) {
      const uint32_t x = early[i];
      gt_part += x > tlo ? 1u : 0u;
      eq_part += x == tlo ? 1u : 0u;
    }
  } else {  // more than the LDS list holds (many equal scores): read them again
    for (int q = t; q < s0; q += kThreads) {
      const uint32_t* rec = slice_rec(w, q);
      const uint16_t* E = reinterpret_cast<const uint16_t*>(rec + kRecE);
      const uint16_t* ent = reinterpret_cast<const uint16_t*>(rec + kRecEnt);
      const uint32_t lo = E[thi], hi = thi > 0 ? E[thi - 1] : rec[1];
      for (uint32_t i = lo; i < hi; ++i) {
        const uint32_t x = ent[i] & 255u;
        gt_part += x > tlo ? 1u : 0u;
        eq_part += x == tlo ? 1u : 0u;
      }
    }
  }
  uint32_t gtb, eqb;
  block_excl_scan<kThreads>(gt_part, sh, gtb);
  block_excl_scan<kThreads>(eq_part, sh, eqb);
  uint32_t off = gtb + (eqb < need ? eqb : need);
  for (int sl = s0; sl < s1; ++sl) {
    const int i0 = sl * kSlice;
    const int first = i0 + t * kPer;
    const int cnt = max(0, min(kPer, C - first));
    if (sl > s0) load_slice(s, i0, C, v);
    {
      uint32_t* t32 = reinterpret_cast<uint32_t*>(tile);
#pragma unroll
      for (int r = 0; r < kPer; ++r) t32[r * kThreads + t] = v[r];
    }
    __syncthreads();
    uint32_t u[kPer];
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const uint4 x = tile[t * (kPer / 4) + q];
      u[4 * q] = x.x;
      u[4 * q + 1] = x.y;
      u[4 * q + 2] = x.z;
      u[4 * q + 3] = x.w;
    }
    uint32_t neq = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) neq += (r < cnt && u[r] == T) ? 1u : 0u;
    uint32_t eq_slice;
    uint32_t eqr = eqb + block_excl_scan<kThreads>(neq, sh, eq_slice);
    uint32_t take = 0, ntake = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const bool valid = r < cnt;
      const bool is_eq = valid && u[r] == T;
      const bool tk = (valid && u[r] > T) || (is_eq && eqr < need);
      eqr += is_eq ? 1u : 0u;
      take |= (tk ? 1u : 0u) << r;
      ntake += tk ? 1u : 0u;
    }
    uint32_t take_slice;
    uint32_t o = off + block_excl_scan<kThreads>(ntake, sh, take_slice);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      if ((take >> r) & 1u) {
        if (o < (uint32_t)K) out[o] = first + r;  // bound: never past K
        ++o;
      }
    }
    eqb += eq_slice;
    off += take_slice;
    // the scans' barriers keep the tile alive until every thread has read it
  }
}

int64_t nslices(int64_t C) { return (C + kSlice - 1) / kSlice; }

int64_t head_stride(int64_t C) {
  return (kSliceBase + nslices(C) * kSliceWords + 63) / 64 * 64;
}

}  // namespace

bool topk_small_path(int64_t C) { return C <= kSmallC; }

size_t topk_ws_bytes(int64_t BH, int64_t C) {
  return topk_small_path(C) ? 0 : (size_t)BH * (size_t)head_stride(C) * sizeof(uint32_t);
}

int64_t topk_hist_stride(int64_t C) { return topk_small_path(C) ? 0 : head_stride(C); }

hipError_t launch_topk_zero(void* ws, int64_t C, int64_t BH, hipStream_t st) {
  if (topk_small_path(C)) return hipSuccess;
  topk_zero<<<dim3(kZeroBlocks, (unsigned)BH), kThreads, 0, st>>>(ws, head_stride(C));
  return hipGetLastError();
}

hipError_t launch_topk(const float* score, int32_t* sel, void* ws, const Geo& g, int64_t BH,
                       bool counted, hipStream_t st) {
  if (g.K == 0) return hipSuccess;
  if (topk_small_path(g.C)) {
    topk_small<<<(unsigned)BH, kSmallThreads, 0, st>>>(score, sel, g.M, g.C, g.K);
    return hipGetLastError();
  }
  const int64_t stride = head_stride(g.C);
  const int64_t nsl = nslices(g.C);
  // workgroups of one slice each, up to about LH_TOPK_WG in all (the
  // kernels are bound by per-slice latency, not bandwidth); h0 takes at most
  // kMaxSub slices per workgroup (16-bit LDS counters)
  const int64_t want = std::max<int64_t>(1, (LH_TOPK_WG + BH - 1) / BH);
  if (!counted) {
    topk_zero<<<dim3(kZeroBlocks, (unsigned)BH), kThreads, 0, st>>>(ws, stride);
    const int64_t hb0 =
        std::min<int64_t>(nsl, std::max<int64_t>(want, (nsl + kMaxSub - 1) / kMaxSub));
    const int64_t nsub0 = (nsl + hb0 - 1) / hb0;
    topk_h0<<<dim3((unsigned)((nsl + nsub0 - 1) / nsub0), (unsigned)BH), kThreads, 0, st>>>(
        score, ws, stride, g.M, g.C, (int32_t)nsl, (int32_t)nsub0);
  }
  const int64_t hb1 = std::min<int64_t>(nsl, want);
  const int64_t nsub1 = (nsl + hb1 - 1) / hb1;
  topk_h1<<<dim3((unsigned)((nsl + nsub1 - 1) / nsub1), (unsigned)BH), kThreads, 0, st>>>(
      score, ws, stride, g.M, g.C, g.K, (int32_t)nsl, (int32_t)nsub1);
  const int64_t wb = std::min<int64_t>(nsl, want);
  const int64_t spw = (nsl + wb - 1) / wb;
  const dim3 wgrid((unsigned)((nsl + spw - 1) / spw), (unsigned)BH);
  topk_w<<<wgrid, kThreads, 0, st>>>(score, sel, ws, stride, g.M, g.C, g.K, (int32_t)nsl,
                                     (int32_t)spw);
  return hipGetLastError();
}

}  // namespace lh

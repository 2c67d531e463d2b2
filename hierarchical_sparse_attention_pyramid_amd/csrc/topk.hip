// Joint top-K over pyramid levels 0..L-2 (gist.science technical summary
// §2.B; bitsgeniais post, phase 2): the K candidates first under the strict
// order (score descending, flat index ascending), written in ascending flat
// order.
//
// The gist.science summary (§2.B) and the bitsgeniais post (phase 2) name a
// fused chunked-bitonic top-K kernel; the operating points they report
// select k = 1536 candidates.  Here K reaches 32K out of 1.4M candidates per
// head, so the selection is an exact radix select instead:
//   1. three histogram passes over the float32 score bits (11 + 11 + 10
//      bits; scores are non-negative, so their bit patterns order like the
//      values) find the score T of the K-th candidate and how many
//      candidates equal to T are still needed;
//   2. an ordered stream compaction keeps every candidate above T and the
//      first `need` candidates equal to T in flat order.
// Both steps are exact integer work and give one deterministic answer.
//
// Workspace per head (uint32): four (prefix, remaining) pairs, one per pick
// ([0] from the init, [p + 1] after pass p), three histograms (one per
// pass), then two arrays of nblk block counters (candidates above and equal
// to the threshold).  Each pick (the bin holding the K-th candidate) is
// computed at the start of the launch that needs it, by every block of that
// launch from the finished histogram, and block 0 records it for the launches
// after: a "last block finishes the pass" scheme would need a device-scope
// fence in every block, which on a multi-XCD GPU (one L2 per XCD) costs more
// than the redundant pick.  Each block of the compaction sums the counters
// of the blocks before it itself.
#include "kernels.h"

namespace lh {

namespace {

constexpr int kBins = 2048;
constexpr int kSlice = 4096;  // candidates per block
constexpr int kThreads = 256;
constexpr int kHead = 8 + 3 * kBins;  // words before the block counters
#ifndef LH_TOPK_HIST_BLOCKS
#define LH_TOPK_HIST_BLOCKS 64
#endif
constexpr int64_t kHistBlocks = LH_TOPK_HIST_BLOCKS;

__device__ __forceinline__ uint32_t* head_ws(void* ws, int64_t bh, int64_t nblk) {
  return static_cast<uint32_t*>(ws) + bh * (kHead + 2 * nblk);
}
__device__ __forceinline__ uint32_t* hist_of(uint32_t* w, int pass) { return w + 8 + pass * kBins; }

__device__ __forceinline__ void pass_bits(int pass, int& shift, int& nbits) {
  shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  nbits = pass == 2 ? 10 : 11;
}

__global__ __launch_bounds__(kThreads) void topk_init(void* ws, int64_t nblk, int32_t K) {
  uint32_t* w = head_ws(ws, blockIdx.x, nblk);
  for (int b = threadIdx.x; b < 3 * kBins; b += kThreads) w[8 + b] = 0;
  if (threadIdx.x == 0) {
    w[0] = 0;           // threshold prefix
    w[1] = (uint32_t)K; // candidates still to take at or below the prefix
  }
}

// Exclusive prefix sum over the 256 threads of a block (in thread order).
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
  for (int k = 0; k < kThreads / 64; ++k) {
    if (k < wv) before += sh[k];
    total += sh[k];
  }
  __syncthreads();
  return before + x - v;
}

// Pick of pass `pass`: the bin of that pass's histogram holding the K-th
// candidate narrows the prefix.  Every thread of the block returns the new
// (prefix, remaining); block 0 also records it as pair pass + 1.
__device__ void pick(uint32_t* w, int pass, uint32_t& prefix_out, uint32_t& rem_out) {
  __shared__ uint32_t sh[kThreads / 64];
  __shared__ uint32_t res[2];
  int shift, nbits;
  pass_bits(pass, shift, nbits);
  const int nb = 1 << nbits;
  const int per = nb / kThreads;
  const uint32_t* hist = hist_of(w, pass);
  const uint32_t remaining = w[2 * pass + 1];
  const uint32_t prefix = w[2 * pass];
  if (threadIdx.x == 0) {  // overwritten by the thread that finds the bin
    res[0] = prefix;
    res[1] = remaining;
  }
  // thread t owns bins nb-1-(t*per) down to nb-1-(t*per+per-1): descending;
  // their counts stay in registers (one round of independent loads)
  constexpr int kMaxPer = kBins / kThreads;
  uint32_t cnt[kMaxPer];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    cnt[j] = j < per ? hist[nb - 1 - (threadIdx.x * per + j)] : 0u;
    local += cnt[j];
  }
  uint32_t total;
  const uint32_t before = block_excl_scan(local, sh, total);
  if (before < remaining && remaining <= before + local) {
    uint32_t cum = before;
    for (int j = 0; j < per; ++j) {
      const int b = nb - 1 - (threadIdx.x * per + j);
      const uint32_t c = cnt[j];
      if (cum + c >= remaining) {
        res[0] = prefix | ((uint32_t)b << shift);
        res[1] = remaining - cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  prefix_out = res[0];
  rem_out = res[1];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    w[2 * pass + 2] = prefix_out;
    w[2 * pass + 3] = rem_out;
  }
}

// This thread's candidates of the block's slice (i0 + tid + 256 r), loaded
// at once; positions past C read as 0 and are excluded by the callers' bounds
// tests.
__device__ __forceinline__ void load_slice(const float* s, int i0, int C, uint32_t (&u)[kSlice / kThreads]) {
#pragma unroll
  for (int r = 0; r < kSlice / kThreads; ++r) {
    const int i = i0 + r * kThreads + (int)threadIdx.x;
    u[r] = i < C ? __float_as_uint(s[i]) : 0u;
  }
}

// Histogram pass `pass` over `nsub` consecutive slices (LDS bins, then
// integer atomics into the head's histogram of that pass), after the pick of
// the pass before.  The first slice's scores are loaded before the pick, so
// the two latencies overlap, and each next slice is loaded while the current
// one is binned.  Several slices per block keep the number of blocks (each
// clears, flushes and picks over the whole bin range) low on long inputs.
__global__ __launch_bounds__(kThreads) void topk_hist(const float* score, void* ws, int64_t nblk,
                                                      int32_t M, int32_t C, int pass, int nsub) {
  constexpr int kPer = kSlice / kThreads;
  __shared__ uint32_t h[kBins];
  const int64_t bh = blockIdx.y;
  uint32_t* w = head_ws(ws, bh, nblk);
  int shift, nbits;
  pass_bits(pass, shift, nbits);
  const uint32_t mask = (1u << nbits) - 1u;
  const int hi = shift + nbits;
  const float* s = score + bh * M;
  const int b0 = blockIdx.x * nsub;  // first slice
  uint32_t u[kPer];
  load_slice(s, b0 * kSlice, C, u);
  for (int b = threadIdx.x; b < kBins; b += kThreads) h[b] = 0;
  uint32_t prefix = 0, rem;
  if (pass > 0) pick(w, pass - 1, prefix, rem);  // its barriers also order the zeroing
  else __syncthreads();
  auto bin = [&](int i0) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const bool valid = i0 + r * kThreads + (int)threadIdx.x < C;
      if (valid && (hi >= 32 || ((u[r] ^ prefix) >> hi) == 0u)) atomicAdd(&h[(u[r] >> shift) & mask], 1u);
    }
  };
  if (nsub == 1) {
    bin(b0 * kSlice);
  } else {
    for (int j = 0; j < nsub; ++j) {
      const int i0 = (b0 + j) * kSlice;
      if (i0 >= C) break;
      uint32_t nx[kPer];
      const bool more = j + 1 < nsub && i0 + kSlice < C;
      if (more) load_slice(s, i0 + kSlice, C, nx);
      bin(i0);
      if (more) {
#pragma unroll
        for (int r = 0; r < kPer; ++r) u[r] = nx[r];
      }
    }
  }
  __syncthreads();
  uint32_t* g = hist_of(w, pass);
  for (int b = threadIdx.x; b < kBins; b += kThreads)
    if (h[b]) atomicAdd(&g[b], h[b]);
}

// Last pick, then per-block counts of candidates above and equal to the
// threshold (scores loaded before the pick, as in the histogram passes).
__global__ __launch_bounds__(kThreads) void topk_count(const float* score, void* ws, int64_t nblk,
                                                       int32_t M, int32_t C) {
  constexpr int kPer = kSlice / kThreads;
  __shared__ uint32_t sh[kThreads / 64];
  const int64_t bh = blockIdx.y;
  uint32_t* w = head_ws(ws, bh, nblk);
  const int i0 = blockIdx.x * kSlice;
  uint32_t u[kPer];
  load_slice(score + bh * M, i0, C, u);
  uint32_t T, need;
  pick(w, 2, T, need);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const bool valid = i0 + r * kThreads + (int)threadIdx.x < C;
    gt += (valid && u[r] > T) ? 1u : 0u;
    eq += (valid && u[r] == T) ? 1u : 0u;
  }
  uint32_t tg, te;
  block_excl_scan(gt, sh, tg);
  block_excl_scan(eq, sh, te);
  if (threadIdx.x == 0) {
    uint32_t* blk = w + kHead;
    blk[blockIdx.x] = tg;
    blk[nblk + blockIdx.x] = te;
  }
}

// Ordered compaction of one block's slice: thread t owns the contiguous
// candidates i0 + 16t .. i0 + 16t + 15, so two block scans (equal-to-T ranks,
// then output offsets) order the whole slice.  The slice's first output
// position follows from the earlier slices' counts alone: every candidate
// above T is taken, and candidates equal to T are taken in flat order until
// `need` of them are in, so the earlier slices took GT + min(EQ, need) of
// them (GT, EQ: their counts above and equal to T).
__global__ __launch_bounds__(kThreads) void topk_write(const float* score, int32_t* sel, void* ws,
                                                       int64_t nblk, int32_t M, int32_t C,
                                                       int32_t K) {
  constexpr int kPer = kSlice / kThreads;
  __shared__ uint32_t sh[kThreads / 64];
  __shared__ uint4 tile[kSlice / 4];  // the slice's score bits, in flat order
  const int64_t bh = blockIdx.y;
  const uint32_t* w = head_ws(ws, bh, nblk);
  int32_t* out = sel + bh * K;
  const int i0 = blockIdx.x * kSlice;
  const int i1 = min(i0 + kSlice, C);
  const int first = i0 + threadIdx.x * kPer;
  const int cnt = max(0, min(kPer, i1 - first));  // valid candidates of this thread
  {
    // coalesced loads (lane-consecutive), then through LDS to the thread
    // that owns them; loaded first: independent of the counters below
    uint32_t v[kPer];
    load_slice(score + bh * M, i0, C, v);
    uint32_t* t32 = reinterpret_cast<uint32_t*>(tile);
#pragma unroll
    for (int r = 0; r < kPer; ++r) t32[r * kThreads + threadIdx.x] = v[r];
  }
  const uint32_t T = w[6], need = w[7];  // the last pick's pair
  const uint32_t* blk = w + kHead;
  uint32_t gt_part = 0, eq_part = 0;  // this thread's share of the earlier slices' counts
  for (int64_t b = threadIdx.x; b < blockIdx.x; b += kThreads) {
    gt_part += blk[b];
    eq_part += blk[nblk + b];
  }
  uint32_t total;
  block_excl_scan(gt_part, sh, total);  // its barriers also publish the tile
  const uint32_t gt_before = total;
  block_excl_scan(eq_part, sh, total);
  const uint32_t eqb = total;  // candidates equal to T in the earlier slices
  const uint32_t off = gt_before + (eqb < need ? eqb : need);
  uint32_t u[kPer];
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const uint4 x = tile[threadIdx.x * (kPer / 4) + q];
    u[4 * q] = x.x;
    u[4 * q + 1] = x.y;
    u[4 * q + 2] = x.z;
    u[4 * q + 3] = x.w;
  }
  uint32_t neq = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) neq += (r < cnt && u[r] == T) ? 1u : 0u;
  uint32_t eqr = eqb + block_excl_scan(neq, sh, total);  // equal candidates before this thread
  uint32_t take = 0, ntake = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const bool valid = r < cnt;
    const bool is_eq = valid && u[r] == T;
    const bool t = (valid && u[r] > T) || (is_eq && eqr < need);
    eqr += is_eq ? 1u : 0u;
    take |= (t ? 1u : 0u) << r;
    ntake += t ? 1u : 0u;
  }
  uint32_t o = off + block_excl_scan(ntake, sh, total);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if ((take >> r) & 1u) {
      if (o < (uint32_t)K) out[o] = first + r;  // bound: never past K
      ++o;
    }
  }
}

}  // namespace

int64_t topk_blocks(int64_t C) { return (C + kSlice - 1) / kSlice; }

size_t topk_ws_bytes(int64_t BH, int64_t C) {
  return (size_t)BH * (size_t)(kHead + 2 * topk_blocks(C)) * sizeof(uint32_t);
}

hipError_t launch_topk(const float* score, int32_t* sel, void* ws, const Geo& g, int64_t BH,
                       hipStream_t st) {
  if (g.K == 0) return hipSuccess;
  const int64_t nblk = topk_blocks(g.C);
  const dim3 grid((unsigned)nblk, (unsigned)BH);
  topk_init<<<(unsigned)BH, kThreads, 0, st>>>(ws, nblk, g.K);
  // at most kHistBlocks histogram blocks per head
  const int nsub = (int)((nblk + kHistBlocks - 1) / kHistBlocks);
  const dim3 hgrid((unsigned)((nblk + nsub - 1) / nsub), (unsigned)BH);
  for (int pass = 0; pass < 3; ++pass)
    topk_hist<<<hgrid, kThreads, 0, st>>>(score, ws, nblk, g.M, g.C, pass, nsub);
  topk_count<<<grid, kThreads, 0, st>>>(score, ws, nblk, g.M, g.C);
  topk_write<<<grid, kThreads, 0, st>>>(score, sel, ws, nblk, g.M, g.C, g.K);
  return hipGetLastError();
}

}  // namespace lh

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
// Workspace per head (uint32): [0] threshold prefix, [1] remaining count,
// [2..3] unused, [4..4+2048) histogram, then two arrays of nblk block
// counters (candidates above and equal to the threshold).  The bin pick is
// a separate one-block-per-head launch: a "last block finishes the pass"
// scheme would need a device-scope fence in every block, which on a
// multi-XCD GPU (one L2 per XCD) costs more than a launch.  Each block of the
// compaction sums the counters of the blocks before it itself.
#include "kernels.h"

namespace lh {

namespace {

constexpr int kBins = 2048;
constexpr int kSlice = 4096;  // candidates per block
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t* head_ws(void* ws, int64_t bh, int64_t nblk) {
  return static_cast<uint32_t*>(ws) + bh * (4 + kBins + 2 * nblk);
}

__device__ __forceinline__ void pass_bits(int pass, int& shift, int& nbits) {
  shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
  nbits = pass == 2 ? 10 : 11;
}

__global__ __launch_bounds__(kThreads) void topk_init(void* ws, int64_t nblk, int32_t K) {
  uint32_t* w = head_ws(ws, blockIdx.x, nblk);
  for (int b = threadIdx.x; b < kBins; b += kThreads) w[4 + b] = 0;
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

// Histogram pass `pass` over this block's slice (LDS bins, then integer
// atomics into the head's histogram).
__global__ __launch_bounds__(kThreads) void topk_hist(const float* score, void* ws, int64_t nblk,
                                                      int32_t M, int32_t C, int pass) {
  __shared__ uint32_t h[kBins];
  const int64_t bh = blockIdx.y;
  uint32_t* w = head_ws(ws, bh, nblk);
  int shift, nbits;
  pass_bits(pass, shift, nbits);
  const uint32_t mask = (1u << nbits) - 1u;
  const int hi = shift + nbits;
  for (int b = threadIdx.x; b < kBins; b += kThreads) h[b] = 0;
  __syncthreads();
  const uint32_t prefix = w[0];
  const float* s = score + bh * M;
  const int i0 = blockIdx.x * kSlice;
  const int i1 = min(i0 + kSlice, C);
  for (int i = i0 + threadIdx.x; i < i1; i += kThreads) {
    const uint32_t u = __float_as_uint(s[i]);
    if (hi >= 32 || ((u ^ prefix) >> hi) == 0u) atomicAdd(&h[(u >> shift) & mask], 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kThreads)
    if (h[b]) atomicAdd(&w[4 + b], h[b]);
}

// One block per head: pick the bin holding the K-th candidate, narrow the
// prefix, clear the histogram for the next pass.
__global__ __launch_bounds__(kThreads) void topk_pick(void* ws, int64_t nblk, int pass) {
  __shared__ uint32_t sh[kThreads / 64];
  uint32_t* w = head_ws(ws, blockIdx.x, nblk);
  int shift, nbits;
  pass_bits(pass, shift, nbits);
  const int nb = 1 << nbits;
  const int per = nb / kThreads;
  const uint32_t remaining = w[1];
  const uint32_t prefix = w[0];
  // thread t owns bins nb-1-(t*per) down to nb-1-(t*per+per-1): descending
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) local += w[4 + nb - 1 - (threadIdx.x * per + j)];
  uint32_t total;
  const uint32_t before = block_excl_scan(local, sh, total);
  if (before < remaining && remaining <= before + local) {
    uint32_t cum = before;
    for (int j = 0; j < per; ++j) {
      const int b = nb - 1 - (threadIdx.x * per + j);
      const uint32_t c = w[4 + b];
      if (cum + c >= remaining) {
        w[0] = prefix | ((uint32_t)b << shift);
        w[1] = remaining - cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kThreads) w[4 + b] = 0;
}

// Per-block counts of candidates above and equal to the threshold.
__global__ __launch_bounds__(kThreads) void topk_count(const float* score, void* ws, int64_t nblk,
                                                       int32_t M, int32_t C) {
  __shared__ uint32_t sh[kThreads / 64];
  const int64_t bh = blockIdx.y;
  uint32_t* w = head_ws(ws, bh, nblk);
  const uint32_t T = w[0];
  const float* s = score + bh * M;
  const int i0 = blockIdx.x * kSlice;
  const int i1 = min(i0 + kSlice, C);
  uint32_t gt = 0, eq = 0;
  for (int i = i0 + threadIdx.x; i < i1; i += kThreads) {
    const uint32_t u = __float_as_uint(s[i]);
    gt += u > T;
    eq += u == T;
  }
  uint32_t tg, te;
  block_excl_scan(gt, sh, tg);
  block_excl_scan(eq, sh, te);
  if (threadIdx.x == 0) {
    uint32_t* blk = w + 4 + kBins;
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
  const int64_t bh = blockIdx.y;
  const uint32_t* w = head_ws(ws, bh, nblk);
  const uint32_t T = w[0], need = w[1];
  const uint32_t* blk = w + 4 + kBins;
  uint32_t gt_part = 0, eq_part = 0;  // this thread's share of the earlier slices' counts
  for (int64_t b = threadIdx.x; b < blockIdx.x; b += kThreads) {
    gt_part += blk[b];
    eq_part += blk[nblk + b];
  }
  uint32_t total;
  block_excl_scan(gt_part, sh, total);
  const uint32_t gt_before = total;
  block_excl_scan(eq_part, sh, total);
  const uint32_t eqb = total;  // candidates equal to T in the earlier slices
  const uint32_t off = gt_before + (eqb < need ? eqb : need);
  const float* s = score + bh * M;
  int32_t* out = sel + bh * K;
  const int i1 = min((int)(blockIdx.x + 1) * kSlice, C);
  const int first = blockIdx.x * kSlice + threadIdx.x * kPer;
  const int cnt = max(0, min(kPer, i1 - first));  // valid candidates of this thread
  uint32_t u[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) u[r] = r < cnt ? __float_as_uint(s[first + r]) : 0u;
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
  return (size_t)BH * (size_t)(4 + kBins + 2 * topk_blocks(C)) * sizeof(uint32_t);
}

hipError_t launch_topk(const float* score, int32_t* sel, void* ws, const Geo& g, int64_t BH,
                       hipStream_t st) {
  if (g.K == 0) return hipSuccess;
  const int64_t nblk = topk_blocks(g.C);
  const dim3 grid((unsigned)nblk, (unsigned)BH);
  topk_init<<<(unsigned)BH, kThreads, 0, st>>>(ws, nblk, g.K);
  for (int pass = 0; pass < 3; ++pass) {
    topk_hist<<<grid, kThreads, 0, st>>>(score, ws, nblk, g.M, g.C, pass);
    topk_pick<<<(unsigned)BH, kThreads, 0, st>>>(ws, nblk, pass);
  }
  topk_count<<<grid, kThreads, 0, st>>>(score, ws, nblk, g.M, g.C);
  topk_write<<<grid, kThreads, 0, st>>>(score, sel, ws, nblk, g.M, g.C, g.K);
  return hipGetLastError();
}

}  // namespace lh

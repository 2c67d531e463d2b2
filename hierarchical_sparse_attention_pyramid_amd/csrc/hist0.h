// First histogram pass of the large-head top-K (score bits 31..16), shared by
// the top-K's own pass-0 kernel and the pooling kernel, which counts the
// candidate scores it writes (so that lh_forward needs no separate pass over
// the scores).
//
// A workgroup counts into a direct-mapped LDS table: coarse bin c (score
// bits 31..24) counts in slot c % kHistSlots, which the first candidate of
// that bin claims with a compare-and-swap of the slot's tag; a candidate
// whose slot another coarse bin holds goes straight to the global
// histograms.  The scores of one layer span a few adjacent coarse bins, so
// collisions are rare.  Fine counters are 16-bit halves of LDS words, so a
// workgroup counts at most 65535 candidates.  The flush adds each pair of
// adjacent fine bins with one 64-bit atomic (the global fine histogram is
// read as 32-bit counts; a pair's low count never carries into the high one)
// and each claimed slot's total to the coarse histogram.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

// Per-head top-K workspace words (uint32) that hold the pass-0 histograms.
constexpr int kTopkC0 = 8;                  // coarse histogram, 256 words
constexpr int kTopkF0 = kTopkC0 + 256;      // fine histogram, 65536 words

constexpr int kHistSlots = 16;
constexpr uint32_t kHistFree = 0xFFFFFFFFu;

struct Hist0Lds {
  uint32_t lf[kHistSlots * 128];  // bin f of slot k: half f & 1 of word k*128 + (f & 255) / 2
  uint32_t tag[kHistSlots];       // coarse bin counted in each slot, or kHistFree
  uint32_t lc[kHistSlots];        // per-slot totals (flush)
};

// Every thread of the workgroup; a barrier must follow before any add.
__device__ __forceinline__ void hist0_init(Hist0Lds& h) {
  for (int i = threadIdx.x; i < kHistSlots * 32; i += blockDim.x)
    reinterpret_cast<uint4*>(h.lf)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < kHistSlots) {
    h.tag[threadIdx.x] = kHistFree;
    h.lc[threadIdx.x] = 0u;
  }
}

// One candidate with score bits u; w: the head's top-K workspace.
__device__ __forceinline__ void hist0_add(Hist0Lds& h, uint32_t u, uint32_t* w) {
  const uint32_t f = u >> 16, c = f >> 8, k = c % kHistSlots;
  uint32_t tg = h.tag[k];
  if (tg == kHistFree) {
    const uint32_t old = atomicCAS(&h.tag[k], kHistFree, c);
    tg = old == kHistFree ? c : old;
  }
  if (tg == c) {
    atomicAdd(&h.lf[k * 128 + ((f & 255u) >> 1)], (f & 1u) ? 0x10000u : 1u);
  } else {  // the slot holds another coarse bin: straight to the global histograms
    atomicAdd(&w[kTopkF0 + f], 1u);
    atomicAdd(&w[kTopkC0 + c], 1u);
  }
}

// Every thread of the workgroup, after a barrier that follows the last add.
__device__ __forceinline__ void hist0_flush(Hist0Lds& h, uint32_t* w) {
  for (int i = threadIdx.x; i < kHistSlots * 128; i += blockDim.x) {
    const int k = i >> 7;
    const uint32_t v = h.lf[i];
    if (v) {
      const uint32_t lo = v & 0xFFFFu, hi = v >> 16;
      const uint32_t f = (h.tag[k] << 8) | ((uint32_t)(i & 127) << 1);
      atomicAdd(reinterpret_cast<unsigned long long*>(w + kTopkF0 + f),
                ((unsigned long long)hi << 32) | lo);
      atomicAdd(&h.lc[k], lo + hi);
    }
  }
  __syncthreads();
  if (threadIdx.x < kHistSlots && h.lc[threadIdx.x]) atomicAdd(&w[kTopkC0 + h.tag[threadIdx.x]], h.lc[threadIdx.x]);
}

}  // namespace lh

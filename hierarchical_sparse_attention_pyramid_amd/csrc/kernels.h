// Host-side launchers of the Lighthouse kernels (internal; the public API is
// include/lighthouse.h).  Every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

namespace lh {

// Maximum pyramid levels one pooling pass produces in registers.
constexpr int kStageLevels = 3;
// The token pass's workgroup may form up to kPoolLdsLevels further levels from
// its rows' top-level float32 sums in LDS (kPoolLdsFloats floats: entries x
// 3 tensors x d).
constexpr int kPoolLdsLevels = 3;
constexpr int kPoolLdsFloats = 6144;

struct PoolFwdArgs {
  const void* in[3];     // stage input: tokens (dtype, layout lin) or f32 sums [BH][in_rows][d]
  Lay lin;               // row layout of `in`
  void* pyr[3];          // pyramid rows [BH][M-N][d] (dtype); null = do not pool
  float* sums_out[3];    // f32 sums of this stage's top level [BH][out_rows][d], or null
  float* score;          // [BH][M] or null
  int64_t in_rows;       // rows per head of `in` (entries of level lvl0)
  int64_t out_rows;      // rows per head of sums_out
  int32_t lvl0;          // level of the input rows
  int32_t lam;           // levels produced: lvl0+1 .. lvl0+lam
  int32_t chunk;         // input rows per row group (a multiple of p^lam)
  int32_t xl;            // token pass: further levels lam+1 .. lam+xl formed in LDS
  // the large-head top-K's workspace (hist_stride words per head): every
  // candidate score written (flat index below C) is counted into its pass-0
  // histograms (hist0.h), which must be zero when the first pass starts;
  // null: no counting
  uint32_t* hist;
  int64_t hist_stride;
  Geo g;
};

struct PoolBwdArgs {
  const void* in;        // dout (dtype, layout lin) or f32 sums [BH][in_rows][d]
  Lay lin;               // row layout of `in`
  void* dos;             // [BH][S][d] (dtype)
  float* sums_out;       // [BH][out_rows][d] or null
  const int32_t* pos;    // [BH][M]
  int64_t in_rows, out_rows;  // virtual rows (see shift)
  int32_t lvl0, lam, chunk;
  int32_t xl;            // token pass: further levels lam+1 .. lam+xl formed in LDS
  int32_t shift;         // 0: span reading; 1: causal reading (virtual row u = token u - 1)
  Geo g;
};

struct BcastArgs {
  const float* src[3];   // [BH][S][d] float32
  void* out[3];          // [B,H,N,d] token tensors, layout lout
  Lay lout;
  const int32_t* pos;    // [BH][M]
  int32_t mean;          // 1: mean over contributors; 0: weight 1/p^level
  int32_t shift;         // 0: span reading; 1: causal reading (forward scatter only)
  Geo g;
};

hipError_t launch_pool_fwd(const PoolFwdArgs& a, int dtype, int64_t BH, bool first,
                           bool do_pool, bool do_score, hipStream_t st);
hipError_t launch_pool_bwd(const PoolBwdArgs& a, int dtype, int64_t BH, bool first,
                           hipStream_t st);
hipError_t launch_bcast(const BcastArgs& a, int dtype, int ntensors, int64_t BH, hipStream_t st);

// top-K
// Heads of at most 16384 candidates are selected in one workgroup's LDS (no
// workspace); larger ones use a workspace of topk_hist_stride(C) words per
// head, whose pass-0 histograms (hist0.h) start each selection at zero.
bool topk_small_path(int64_t C);
size_t topk_ws_bytes(int64_t BH, int64_t C);
int64_t topk_hist_stride(int64_t C);  // 0 on the small path
// clears the histograms (large heads; nothing on the small path)
hipError_t launch_topk_zero(void* ws, int64_t C, int64_t BH, hipStream_t st);
// counted: the caller cleared the histograms and counted pass 0 (the pooling
// kernel in lh_forward); else the clearing kernel and the pass-0 kernel run first
hipError_t launch_topk(const float* score, int32_t* sel, void* ws, const Geo& g, int64_t BH,
                       bool counted, hipStream_t st);

// gather
// q, k, v: token tensors of layout lq
hipError_t launch_gather(const int32_t* sel, const void* const q[3], const Lay& lq,
                         const void* const pyr[3], int32_t* sub_idx, int32_t* pos,
                         void* const qs[3], const Geo& g, int dtype, int64_t BH, hipStream_t st);

// attention
// Buffers of the forward's key-range split (bf16): chunk-0 partial outputs
// [BH][S][d] and lambdas [BH][S], float32.  The split runs only on causal
// grids too small to balance (see attn_fwd_bf16).
struct FwdSplitBufs {
  float* o;
  float* lam;
};
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int64_t S, int d, int dtype, int64_t BH, hipStream_t st,
                           const FwdSplitBufs* split = nullptr);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* delta, float* lse2, int64_t S, int d, int dtype, int64_t BH,
                           hipStream_t st, hipEvent_t* ev,  // ev: ends of rowsum, dK/dV, dQ
                           hipEvent_t dq_done = nullptr);   // bf16: recorded after the dQ pass

}  // namespace lh

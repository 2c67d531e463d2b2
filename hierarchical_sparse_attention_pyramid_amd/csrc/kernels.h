// Host-side launchers of the Lighthouse kernels (internal; the public API is
// include/lighthouse.h).  Every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace lh {

// Maximum pyramid levels one pooling pass produces in registers.
constexpr int kStageLevels = 3;

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
  Geo g;
};

struct PoolBwdArgs {
  const void* in;        // dout (dtype, layout lin) or f32 sums [BH][in_rows][d]
  Lay lin;               // row layout of `in`
  void* dos;             // [BH][S][d] (dtype)
  float* sums_out;       // [BH][out_rows][d] or null
  const int32_t* pos;    // [BH][M]
  int64_t in_rows, out_rows;
  int32_t lvl0, lam, chunk;
  Geo g;
};

struct BcastArgs {
  const float* src[3];   // [BH][S][d] float32
  void* out[3];          // [B,H,N,d] token tensors, layout lout
  Lay lout;
  const int32_t* pos;    // [BH][M]
  int32_t mean;          // 1: mean over contributors; 0: weight 1/p^level
  Geo g;
};

hipError_t launch_pool_fwd(const PoolFwdArgs& a, int dtype, int64_t BH, bool first,
                           bool do_pool, bool do_score, hipStream_t st);
hipError_t launch_pool_bwd(const PoolBwdArgs& a, int dtype, int64_t BH, bool first,
                           hipStream_t st);
hipError_t launch_bcast(const BcastArgs& a, int dtype, int ntensors, int64_t BH, hipStream_t st);

// top-K
int64_t topk_blocks(int64_t C);
size_t topk_ws_bytes(int64_t BH, int64_t C);
hipError_t launch_topk(const float* score, int32_t* sel, void* ws, const Geo& g, int64_t BH,
                       hipStream_t st);

// gather
// q, k, v: token tensors of layout lq
hipError_t launch_gather(const int32_t* sel, const void* const q[3], const Lay& lq,
                         const void* const pyr[3], int32_t* sub_idx, int32_t* pos,
                         void* const qs[3], const Geo& g, int dtype, int64_t BH, hipStream_t st);

// attention
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int64_t S, int d, int dtype, int64_t BH, hipStream_t st);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* delta, float* lse2, int64_t S, int d, int dtype, int64_t BH,
                           hipStream_t st, hipEvent_t* ev);  // ev: ends of rowsum, dK/dV, dQ

}  // namespace lh

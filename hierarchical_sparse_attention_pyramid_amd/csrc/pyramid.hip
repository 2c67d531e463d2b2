// Pooling kernels: the forward pyramid with fused scores, and the scatter
// backward, which is the same span reduction applied to dout / c_t.
//
// Symmetric average pooling follows the gist.science technical summary of
// the Lighthouse paper, §2.A (levels of p consecutive entries, level 0 =
// tokens) and the bitsgeniais post, phase 1.  Scores follow §2.B of the same
// summary and phase 2 of the post: an l2 norm of q and of k per token, coarse
// levels inheriting the max of their children.
//
// Mapping: a row of d elements is covered by d/8 lanes (8 elements each, one
// 16-byte bf16 or 32-byte fp32 access); a 256-thread block holds 256/(d/8)
// such row groups.  Each row group walks one chunk of consecutive input rows
// in order and keeps one running float32 sum per level in registers, so each
// input row is read exactly once and every level is produced in the same
// pass.  Deep pyramids use several passes: a pass hands the float32 sums of
// its top level to the next one.
#include "hist0.h"
#include "kernels.h"
#include "walk.h"

namespace lh {

namespace {

#ifndef LH_POOL_ROWS
#define LH_POOL_ROWS 4
#endif
#ifndef LH_POOL_NT
#define LH_POOL_NT 1
#endif
constexpr int kRowsInFlight = LH_POOL_ROWS;  // rows whose loads a row group issues together
constexpr bool kStream = LH_POOL_NT != 0;    // token rows are read once: streaming loads

// y[lane + k] for lanes of the same 16-lane DPP row (row_shl:k); used only
// where lane + k stays inside the lane's row group.
template <int K>
__device__ __forceinline__ float from_lane_plus(float y) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, y), 0x100 + K,
                                                            0xf, 0xf, true));
}

// ||x||_2 of a d-long row spread over `lpr` lanes (element 8*lane + e in
// x[e]), in the fixed float32 order: squares, then the halving tree
// y[i] += y[i + w/2] for w = d, d/2, ..., 2 (cross-lane strides d/2..8 first,
// then in-lane strides 4, 2, 1), then a correctly rounded square root.  No
// fused multiply-add, so the result is reproducible bit for bit.  The value
// is exact in the row group's first lane (the one that uses it); the
// cross-lane steps shift lanes down (DPP row_shl) toward that lane, so no
// LDS crossbar traffic is needed.
__device__ __forceinline__ float row_norm(const float (&x)[8], int lpr) {
#pragma clang fp contract(off)
  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = x[e] * x[e];
  if (lpr == 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = a[e] + from_lane_plus<8>(a[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = a[e] + from_lane_plus<4>(a[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = a[e] + from_lane_plus<2>(a[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = a[e] + from_lane_plus<1>(a[e]);
  const float b0 = a[0] + a[4], b1 = a[1] + a[5], b2 = a[2] + a[6], b3 = a[3] + a[7];
  const float c0 = b0 + b2, c1 = b1 + b3;
  return sqrtf(c0 + c1);  // correctly rounded on gfx950 (not __fsqrt_rn)
}

// Candidate scores one row group stages for the top-K's counting: its chunk
// (at most 64 rows) and the coarser entries completed in it.
constexpr int kStageCap = 128;

// One pass over the tensors listed in `tid` for the chunk of rows
// [r0, r0 + nrows) of head bh.  SCORE: 0 none, 1 norms (level 0 input),
// 2 max-pool of stored level-lvl0 scores.  stage (LDS, kStageCap words, or
// null): the row group's list of candidate score bits written, nst their
// count; they are counted after the pass, off the row loop.
template <typename Tin, typename Tout, int NT, int SCORE>
__device__ __forceinline__ void pool_pass(const PoolFwdArgs& a, const int (&tid)[NT],
                                          bool do_pool, int64_t bh, int64_t r0, int nrows,
                                          int lane, uint32_t* stage, int& nst) {
  const Geo& g = a.g;
  const int d = g.d;
  const int lpr = d / 8;
  const Tin* in[NT];
  Tout* pyr[NT];
  float* so[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    in[i] = a.in[tid[i]] ? static_cast<const Tin*>(a.in[tid[i]]) + a.lin.head(bh) + 8 * lane
                         : nullptr;  // score-only passes above level 0 read no rows
    pyr[i] = do_pool ? static_cast<Tout*>(a.pyr[tid[i]]) + bh * (int64_t)(g.M - g.N) * d + 8 * lane
                     : nullptr;
    so[i] = a.sums_out[tid[i]] ? a.sums_out[tid[i]] + bh * a.out_rows * d + 8 * lane : nullptr;
  }
  float* score = a.score ? a.score + bh * g.M : nullptr;

  float acc[kStageLevels][NT][8];
  float smax[kStageLevels];
  int cnt[kStageLevels];
#pragma unroll
  for (int l = 0; l < kStageLevels; ++l) {
    smax[l] = neg_inf();
    cnt[l] = 0;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[l][i][e] = 0.f;
  }

  for (int rb = 0; rb < nrows; rb += kRowsInFlight) {
    // issue the loads of up to kRowsInFlight rows before using any of them
    float xs[kRowsInFlight][NT][8];
    if (SCORE == 1 || do_pool) {
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int64_t row = r0 + min(rb + u, nrows - 1);
#pragma unroll
        for (int i = 0; i < NT; ++i)
          Row8<Tin>::template load<kStream>(in[i] + row * a.lin.sn, xs[u][i]);
      }
    }
    float sin[kRowsInFlight];
    if constexpr (SCORE == 2) {
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) sin[u] = score[g.base[a.lvl0] + r0 + min(rb + u, nrows - 1)];
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      if (rb + u >= nrows) break;
      const int64_t row = r0 + rb + u;
      float s = 0.f;
      if constexpr (SCORE == 1) {
        s = row_norm(xs[u][0], lpr) + row_norm(xs[u][1], lpr);
        if (lane == 0) {
          score[row] = s;
          if (stage != nullptr && row < g.C && nst < kStageCap) stage[nst++] = __float_as_uint(s);
        }
      } else if constexpr (SCORE == 2) {
        s = sin[u];
      }
      if (do_pool) {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[0][i][e] += xs[u][i][e];
      }
      if constexpr (SCORE != 0) smax[0] = fmaxf(smax[0], s);

#pragma unroll
      for (int l = 0; l < kStageLevels; ++l) {
        if (l >= a.lam) break;
        if (++cnt[l] < g.p) break;
        cnt[l] = 0;
        const int lev = a.lvl0 + l + 1;                       // level just completed
        const int64_t j = (row + 1) / g.pw[l + 1] - 1;        // its index in that level
        if (do_pool) {
#pragma unroll
          for (int i = 0; i < NT; ++i) {
            float m[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = acc[l][i][e] * g.inv_pw[lev];
            Row8<Tout>::template store<kStream>(pyr[i] + (int64_t)(g.base[lev] - g.N + j) * d, m);
          }
        }
        if constexpr (SCORE != 0) {
          if (lane == 0) {
            const int64_t flat = g.base[lev] + j;
            score[flat] = smax[l];
            if (stage != nullptr && flat < g.C && nst < kStageCap)
              stage[nst++] = __float_as_uint(smax[l]);
          }
        }
        if (l + 1 < kStageLevels && l + 1 < a.lam) {
          if (do_pool) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[(l + 1) % kStageLevels][i][e] += acc[l][i][e];
          }
          if constexpr (SCORE != 0)
            smax[(l + 1) % kStageLevels] = fmaxf(smax[(l + 1) % kStageLevels], smax[l]);
        } else if (do_pool && so[0] != nullptr) {
#pragma unroll
          for (int i = 0; i < NT; ++i) Row8<float>::store(so[i] + j * d, acc[l][i]);
        }
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[l][i][e] = 0.f;
        smax[l] = neg_inf();
      }
    }
  }
}

template <typename Tin, typename Tout, bool FIRST>
__global__ __launch_bounds__(256) void pool_fwd_kernel(PoolFwdArgs a, int do_pool, int do_score) {
  // the top-K's pass-0 counting (hist0.h) of the candidate scores written:
  // each row group lists them in LDS, and the workgroup counts the lists
  // after the row walk
  __shared__ Hist0Lds hl;
  __shared__ uint32_t stage[32 * kStageCap];
  __shared__ int nstage[32];
  const bool count = a.hist != nullptr && do_score;  // uniform
  const int lpr = a.g.d / 8;
  const int rgs = 256 / lpr;
  const int rg = threadIdx.x / lpr, lane = threadIdx.x % lpr;
  const int64_t bh = blockIdx.y;
  int nst = 0;
  if (count) hist0_init(hl);
  const int64_t nchunks = (a.in_rows + a.chunk - 1) / a.chunk;
  const int64_t c = (int64_t)blockIdx.x * rgs + rg;
  if (c < nchunks) {
    const int64_t r0 = c * a.chunk;
    const int nrows = (int)min((int64_t)a.chunk, a.in_rows - r0);
    constexpr int kScore = FIRST ? 1 : 2;
    // pass 1: q and k (with the scores); pass 2: v (two passes keep fewer
    // rows' accumulators live in registers than one pass over all three)
    const int qk[2] = {0, 1};
    if (do_score) {
      pool_pass<Tin, Tout, 2, kScore>(a, qk, do_pool != 0, bh, r0, nrows, lane,
                                      count ? stage + rg * kStageCap : nullptr, nst);
    } else if (do_pool) {
      pool_pass<Tin, Tout, 2, 0>(a, qk, true, bh, r0, nrows, lane, nullptr, nst);
    }
    if (do_pool) {
      const int vv[1] = {2};
      pool_pass<Tin, Tout, 1, 0>(a, vv, true, bh, r0, nrows, lane, nullptr, nst);
    }
  }
  if (count) {  // every thread of the workgroup reaches these barriers
    if (lane == 0) nstage[rg] = nst;
    __syncthreads();
    uint32_t* hw = a.hist + bh * a.hist_stride;
    for (int i = threadIdx.x; i < rgs * kStageCap; i += 256) {
      const int r = i / kStageCap, j = i % kStageCap;
      if (j < nstage[r]) hist0_add(hl, stage[i], hw);
    }
    __syncthreads();
    hist0_flush(hl, hw);
  }
}

// Scatter backward: dos[pos(e)] = sum over the tokens t that entry e feeds
// of dout[t] / c_t (0 for a token that nothing feeds).  Same row-group walk
// as the forward; only selected entries are written.  The causal reading
// (shift = 1: entry (l, j) feeds the p^l tokens from its end token on) is
// the span reduction over virtual rows u = t + 1, with positions looked up
// as vpos(l, J) = pos(l, J - 1) and the rows padded with zeros to
// N + p^(L-1), so that the windows of every level's last entry complete.  On the token pass, c_t (the number of selected ancestors of
// t) comes from an ancestor walk that keeps per-level counts.  The positions
// the workgroup needs (its rows' own, the levels it writes and, on the token
// pass, every ancestor level) are first staged in LDS in one coalesced
// burst, so that no load of a row group waits on a position load.
constexpr int kBwdPosCache = 4608;  // ints: workgroup rows + their ancestors (p >= 2)

template <typename Tin, typename Tout, bool FIRST, int SH>
__global__ __launch_bounds__(256) void pool_bwd_kernel(PoolBwdArgs a) {
  const Geo& g = a.g;
  const int d = g.d;
  const int lpr = d / 8;
  const int rgs = 256 / lpr;
  const int rg = threadIdx.x / lpr, lane = threadIdx.x % lpr;
  const int64_t bh = blockIdx.y;
  const int64_t nchunks = (a.in_rows + a.chunk - 1) / a.chunk;
  const int64_t c = (int64_t)blockIdx.x * rgs + rg;
  const int32_t* pos = a.pos + bh * g.M;
  // position of virtual entry j of level l (-1: outside the level or not selected)
  auto vpos = [&](int l, int32_t j) {
    if constexpr (SH == 0) {
      return pos[g.base[l] + j];
    } else {
      const int32_t jj = j - SH;
      return jj >= 0 && jj < g.nlev[l] ? pos[g.base[l] + jj] : -1;
    }
  };

  // ---- stage positions: rows [B0, B0 + BT) of level lvl0 (token pass), then
  // the entries of every level above lvl0 that these rows belong to
  __shared__ int32_t sp[kBwdPosCache];
  __shared__ int32_t soff[kMaxLevels], sjlo[kMaxLevels];
  const int64_t B0 = (int64_t)blockIdx.x * rgs * a.chunk;
  const int64_t BT = min((int64_t)rgs * a.chunk, a.in_rows - B0);
  int off = 0;
  if (FIRST) {
    for (int i = threadIdx.x; i < BT; i += 256) sp[i] = vpos(0, (int32_t)(B0 + i));
    off = (int)BT;
  }
  const int ltop = FIRST ? g.L : min(g.L, a.lvl0 + a.lam + 1);  // levels whose positions are read
  for (int l = a.lvl0 + 1; l < ltop; ++l) {
    const int32_t f = g.pw[l] / g.pw[a.lvl0];  // rows of level lvl0 per entry of level l
    const int32_t jlo = (int32_t)(B0 / f);
    const int32_t jhi = (int32_t)((B0 + BT - 1) / f);
    if (threadIdx.x == 0) {
      soff[l] = off;
      sjlo[l] = jlo;
    }
    for (int i = threadIdx.x; i <= jhi - jlo; i += 256) sp[off + i] = vpos(l, jlo + i);
    off += jhi - jlo + 1;
  }
  __syncthreads();
  if (c >= nchunks) return;  // no barrier below
  auto posf = [&](int l, int32_t j) { return sp[soff[l] + (j - sjlo[l])]; };

  const int64_t r0 = c * a.chunk;
  const int nrows = (int)min((int64_t)a.chunk, a.in_rows - r0);
  const Tin* in = static_cast<const Tin*>(a.in) + a.lin.head(bh) + 8 * lane;
  Tout* dos = static_cast<Tout*>(a.dos) + bh * (int64_t)g.S * d + 8 * lane;
  float* so = a.sums_out ? a.sums_out + bh * a.out_rows * d + 8 * lane : nullptr;

  float acc[kStageLevels][8];
  int cnt[kStageLevels];
#pragma unroll
  for (int l = 0; l < kStageLevels; ++l) {
    cnt[l] = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;
  }
  // c_t on the token pass.  p a power of two >= 4 and a chunk of 2^lc
  // aligned rows with 3 log2(p) >= lc: levels with p^l >= 2^lc give the same
  // count to all rows of the chunk (counted once here) and at most two inner
  // levels vary per row.  Otherwise: the ancestor walk of counts.
  const int lc = 31 - __builtin_clz((unsigned)a.chunk);
  const bool fastc = FIRST && g.log2p >= 2 && (1 << lc) == a.chunk && 3 * g.log2p >= lc;
  int cnt_outer = 0;
  if (fastc) {
    for (int l = 1; l < g.L; ++l)
      if (g.log2p * l >= lc) cnt_outer += posf(l, (int32_t)(r0 >> (g.log2p * l))) >= 0;
  }
  AncestorWalk<0, 1> walk;
  for (int rb = 0; rb < nrows; rb += kRowsInFlight) {
    float xs[kRowsInFlight][8];
    int32_t pt[kRowsInFlight];
    bool inside[kRowsInFlight];  // causal: the virtual row is a token
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int64_t row = r0 + min(rb + u, nrows - 1);
      if constexpr (FIRST && SH != 0) {
        // token row of virtual row `row`, clamped into the tokens so that the
        // load needs no branch; rows outside get weight 0 below
        const int64_t t = row - SH;
        inside[u] = t >= 0 && t < g.N;
        const int64_t tc = t < 0 ? 0 : (t < g.N ? t : g.N - 1);
        Row8<Tin>::template load<kStream>(in + tc * a.lin.sn, xs[u]);
      } else {
        inside[u] = true;
        Row8<Tin>::template load<kStream>(in + row * a.lin.sn, xs[u]);
      }
      if constexpr (FIRST) pt[u] = sp[row - B0];
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      if (rb + u >= nrows) break;
      const int64_t row = r0 + rb + u;
      if constexpr (FIRST) {
        int ct = (pt[u] >= 0 ? 1 : 0);
        if (fastc) {
          ct += cnt_outer;
#pragma unroll
          for (int l = 1; l <= 2; ++l)
            if (l < g.L && g.log2p * l < lc) ct += posf(l, (int32_t)(row >> (g.log2p * l))) >= 0;
        } else {
          walk.advance((int32_t)row, posf, nullptr, g, true, lane);
          ct += walk.cnt[1];
        }
        // span reading: every token has a contributor; causal: 0 for an unfed
        // token and for the virtual rows that are no token
        const float rc =
            SH == 0 || (ct > 0 && inside[u]) ? 1.0f / static_cast<float>(ct) : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[u][e] *= rc;
        if (pt[u] >= 0) Row8<Tout>::store(dos + (int64_t)pt[u] * d, xs[u]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[0][e] += xs[u][e];
#pragma unroll
      for (int l = 0; l < kStageLevels; ++l) {
        if (l >= a.lam) break;
        if (++cnt[l] < g.p) break;
        cnt[l] = 0;
        const int lev = a.lvl0 + l + 1;
        const int64_t j = (row + 1) / g.pw[l + 1] - 1;
        const int32_t pe = posf(lev, (int32_t)j);
        if (pe >= 0) Row8<Tout>::store(dos + (int64_t)pe * d, acc[l]);
        if (l + 1 < kStageLevels && l + 1 < a.lam) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[(l + 1) % kStageLevels][e] += acc[l][e];
        } else if (so != nullptr) {
          Row8<float>::store(so + j * d, acc[l]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;
      }
    }
  }
}

dim3 pool_grid(int64_t in_rows, int chunk, int d, int64_t BH) {
  const int rgs = 256 / (d / 8);
  const int64_t nchunks = (in_rows + chunk - 1) / chunk;
  return dim3((unsigned)((nchunks + rgs - 1) / rgs), (unsigned)BH);
}

}  // namespace

hipError_t launch_pool_fwd(const PoolFwdArgs& a, int dtype, int64_t BH, bool first,
                           bool do_pool, bool do_score, hipStream_t st) {
  const dim3 grid = pool_grid(a.in_rows, a.chunk, a.g.d, BH);
  const int dp = do_pool, ds = do_score;
  if (dtype == 1) {
    if (first) pool_fwd_kernel<__bf16, __bf16, true><<<grid, 256, 0, st>>>(a, dp, ds);
    else pool_fwd_kernel<float, __bf16, false><<<grid, 256, 0, st>>>(a, dp, ds);
  } else {
    if (first) pool_fwd_kernel<float, float, true><<<grid, 256, 0, st>>>(a, dp, ds);
    else pool_fwd_kernel<float, float, false><<<grid, 256, 0, st>>>(a, dp, ds);
  }
  return hipGetLastError();
}

hipError_t launch_pool_bwd(const PoolBwdArgs& a, int dtype, int64_t BH, bool first,
                           hipStream_t st) {
  const dim3 grid = pool_grid(a.in_rows, a.chunk, a.g.d, BH);
  // the shift is a template parameter: the span reading's kernels carry no
  // virtual-row bookkeeping at all
  if (dtype == 1) {
    if (first) {
      if (a.shift) pool_bwd_kernel<__bf16, __bf16, true, 1><<<grid, 256, 0, st>>>(a);
      else pool_bwd_kernel<__bf16, __bf16, true, 0><<<grid, 256, 0, st>>>(a);
    } else {
      if (a.shift) pool_bwd_kernel<float, __bf16, false, 1><<<grid, 256, 0, st>>>(a);
      else pool_bwd_kernel<float, __bf16, false, 0><<<grid, 256, 0, st>>>(a);
    }
  } else {
    if (first) {
      if (a.shift) pool_bwd_kernel<float, float, true, 1><<<grid, 256, 0, st>>>(a);
      else pool_bwd_kernel<float, float, true, 0><<<grid, 256, 0, st>>>(a);
    } else {
      if (a.shift) pool_bwd_kernel<float, float, false, 1><<<grid, 256, 0, st>>>(a);
      else pool_bwd_kernel<float, float, false, 0><<<grid, 256, 0, st>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace lh

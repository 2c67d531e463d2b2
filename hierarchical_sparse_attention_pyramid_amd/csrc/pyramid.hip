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
// in order and keeps one running float32 sum per level in registers (up to
// three levels), so each input row is read exactly once.  On the token pass
// the workgroup then forms the levels whose spans divide its rows from the
// row groups' top-level sums in LDS (p >= 4).  Deeper pyramids use further
// passes: a pass hands the float32 sums of its top level to the next one.
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
// xbuf / xsc (LDS, or null): with a.xl > 0 the top level's float32 sums
// [entry][tensor][d] and scores of the workgroup's entries (from index xe0
// of that level) go there instead of to sums_out.
template <typename Tin, typename Tout, int NT, int SCORE>
__device__ __forceinline__ void pool_pass(const PoolFwdArgs& a, const int (&tid)[NT],
                                          bool do_pool, int64_t bh, int64_t r0, int nrows,
                                          int lane, uint32_t* stage, int& nst, float* xbuf,
                                          float* xsc, int64_t xe0) {
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
        } else if (xbuf != nullptr) {
          const int64_t x = j - xe0;
          if (do_pool) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
              for (int e = 0; e < 8; ++e) xbuf[(x * 3 + tid[i]) * d + 8 * lane + e] = acc[l][i][e];
          }
          if constexpr (SCORE != 0) {
            if (lane == 0) xsc[x] = smax[l];
          }
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

// Levels lam+1 .. lam+xl of the token pass from the top register level's
// float32 sums and scores of the workgroup's E entries (index e0 on), staged
// in LDS by pool_pass: each new entry sums p consecutive ones in order (the
// same float32 additions a further pass over the stored sums makes) and
// takes the max of their scores.  Every thread calls it; at most one sum
// item (8 elements of one entry's tensor row) and one score per thread and
// level, which the plan guarantees (p >= 4, E x 3 x d <= kPoolLdsFloats).
template <typename Tout>
__device__ __forceinline__ void pool_lds_levels(const PoolFwdArgs& a, int64_t bh, int64_t E,
                                                int64_t e0, bool do_pool, bool do_score,
                                                float* xbuf, float* xsc, Hist0Lds* hl,
                                                uint32_t* hw) {
  const Geo& g = a.g;
  const int d = g.d, p = g.p, gpr = d / 8;
  const int t = threadIdx.x;
  for (int x = 1; x <= a.xl; ++x) {
    const int lev = a.lam + x;
    const int64_t En = E / p, j0 = e0 / p;
    float s[8];
    const bool item = do_pool && t < En * 3 * gpr;
    const int k = t / (3 * gpr), ten = (t / gpr) % 3, g8 = t % gpr;
    if (item) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = 0.f;
      for (int c = 0; c < p; ++c) {
        const float* src = xbuf + ((k * p + c) * 3 + ten) * d + 8 * g8;
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += src[e];
      }
    }
    const bool sc = do_score && t < En;
    float sm = neg_inf();
    if (sc)
      for (int c = 0; c < p; ++c) sm = fmaxf(sm, xsc[t * p + c]);
    __syncthreads();  // every read of the level below is done
    if (item) {
      const int64_t j = j0 + k;
      float m[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = s[e] * g.inv_pw[lev];
      Tout* pyr = static_cast<Tout*>(a.pyr[ten]) + bh * (int64_t)(g.M - g.N) * d;
      Row8<Tout>::template store<kStream>(pyr + (int64_t)(g.base[lev] - g.N + j) * d + 8 * g8, m);
      if (x < a.xl) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xbuf[(k * 3 + ten) * d + 8 * g8 + e] = s[e];
      } else if (a.sums_out[ten] != nullptr) {
        Row8<float>::store(a.sums_out[ten] + (bh * a.out_rows + j) * d + 8 * g8, s);
      }
    }
    if (sc) {
      const int64_t flat = g.base[lev] + j0 + t;
      a.score[bh * g.M + flat] = sm;
      if (hl != nullptr && flat < g.C) hist0_add(*hl, __float_as_uint(sm), hw);
      xsc[t] = sm;
    }
    __syncthreads();
    E = En;
    e0 = j0;
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
  __shared__ float xbuf[kPoolLdsFloats];
  __shared__ float xsc[kPoolLdsFloats / 192];
  const bool count = a.hist != nullptr && do_score;  // uniform
  const bool lds_levels = FIRST && a.xl > 0;         // uniform
  const int lpr = a.g.d / 8;
  const int rgs = 256 / lpr;
  const int rg = threadIdx.x / lpr, lane = threadIdx.x % lpr;
  const int64_t bh = blockIdx.y;
  const int64_t B0 = (int64_t)blockIdx.x * rgs * a.chunk;  // the workgroup's first row
  const int64_t xe0 = B0 / a.g.pw[a.lam];                  // its first top-level entry
  int nst = 0;
  if (count) hist0_init(hl);
  const int64_t nchunks = (a.in_rows + a.chunk - 1) / a.chunk;
  const int64_t c = (int64_t)blockIdx.x * rgs + rg;
  if (c < nchunks) {
    const int64_t r0 = c * a.chunk;
    const int nrows = (int)min((int64_t)a.chunk, a.in_rows - r0);
    constexpr int kScore = FIRST ? 1 : 2;
    float* xb = lds_levels ? xbuf : nullptr;
    float* xs = lds_levels ? xsc : nullptr;
    // pass 1: q and k (with the scores); pass 2: v (two passes keep fewer
    // rows' accumulators live in registers than one pass over all three)
    const int qk[2] = {0, 1};
    if (do_score) {
      pool_pass<Tin, Tout, 2, kScore>(a, qk, do_pool != 0, bh, r0, nrows, lane,
                                      count ? stage + rg * kStageCap : nullptr, nst, xb, xs, xe0);
    } else if (do_pool) {
      pool_pass<Tin, Tout, 2, 0>(a, qk, true, bh, r0, nrows, lane, nullptr, nst, xb, xs, xe0);
    }
    if (do_pool) {
      const int vv[1] = {2};
      pool_pass<Tin, Tout, 1, 0>(a, vv, true, bh, r0, nrows, lane, nullptr, nst, xb, xs, xe0);
    }
  }
  // every thread of the workgroup reaches the barriers below
  uint32_t* hw = count ? a.hist + bh * a.hist_stride : nullptr;
  if (count && lane == 0) nstage[rg] = nst;
  if (count || lds_levels) __syncthreads();
  if (count) {
    for (int i = threadIdx.x; i < rgs * kStageCap; i += 256) {
      const int r = i / kStageCap, j = i % kStageCap;
      if (j < nstage[r]) hist0_add(hl, stage[i], hw);
    }
  }
  if (lds_levels)
    pool_lds_levels<Tout>(a, bh, min((int64_t)rgs * a.chunk, a.in_rows - B0) / a.g.pw[a.lam], xe0,
                          do_pool != 0, do_score != 0, xbuf, xsc, count ? &hl : nullptr, hw);
  if (count) {
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
__global__ __launch_bounds__(256, (FIRST && sizeof(Tin) == 2) ? 5 : 1) void pool_bwd_kernel(PoolBwdArgs a) {
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
  auto posf = [&](int l, int32_t j) { return sp[soff[l] + (j - sjlo[l])]; };
  // token pass with a.xl > 0: the top register level's float32 sums of the
  // workgroup's entries (from xe0) are staged in LDS for the levels above
  __shared__ float xbuf[kPoolLdsFloats / 3];
  const bool lds_levels = FIRST && a.xl > 0;  // uniform
  const int64_t xe0 = B0 / g.pw[a.lam];
  if (c < nchunks) {
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
        } else if (lds_levels) {
#pragma unroll
          for (int e = 0; e < 8; ++e) xbuf[(j - xe0) * d + 8 * lane + e] = acc[l][e];
        } else if (so != nullptr) {
          Row8<float>::store(so + j * d, acc[l]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[l][e] = 0.f;
      }
    }
  }
  }  // c < nchunks
  if (!lds_levels) return;
  // levels lam+1 .. lam+xl: each entry sums p consecutive staged ones in order
  // (the float32 additions a further pass over stored sums makes); selected
  // entries are written to dos; the top one's sums go to sums_out.  At most
  // one 8-element item per thread and level (the plan guarantees it).
  __syncthreads();  // every staged sum is in LDS
  const int gpr = d / 8, t = threadIdx.x;
  int64_t E = BT / g.pw[a.lam], e0 = xe0;
  for (int x = 1; x <= a.xl; ++x) {
    const int lev = a.lam + x;
    const int64_t En = E / g.p, j0 = e0 / g.p;
    const bool item = t < En * gpr;
    const int k = t / gpr, g8 = t % gpr;
    float sx[8];
    if (item) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sx[e] = 0.f;
      for (int cc = 0; cc < g.p; ++cc) {
        const float* src = xbuf + (k * g.p + cc) * d + 8 * g8;
#pragma unroll
        for (int e = 0; e < 8; ++e) sx[e] += src[e];
      }
    }
    __syncthreads();  // every read of the level below is done
    if (item) {
      const int64_t j = j0 + k;
      const int32_t pe = posf(lev, (int32_t)j);
      if (pe >= 0)
        Row8<Tout>::store(static_cast<Tout*>(a.dos) + (bh * (int64_t)g.S + pe) * d + 8 * g8, sx);
      if (x < a.xl) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xbuf[k * d + 8 * g8 + e] = sx[e];
      } else if (a.sums_out != nullptr) {
        Row8<float>::store(a.sums_out + (bh * a.out_rows + j) * d + 8 * g8, sx);
      }
    }
    __syncthreads();
    E = En;
    e0 = j0;
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

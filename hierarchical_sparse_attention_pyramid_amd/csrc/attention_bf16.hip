// Causal flash-style attention on bf16 inputs with gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, float32 accumulation).  This is the "stock dense
// attention on the gathered subsequence" of the gist.science technical
// summary, §2.C, and, at S = N, the dense baseline.
//
// MFMA 32x32x16 operand layout (wave of 64 lanes, lane = 32*h + c):
//   A (32 x 16): lane holds row c, k = 8h .. 8h+7 (8 bf16)
//   B (16 x 32): lane holds column c, k = 8h .. 8h+7
//   D (32 x 32): lane holds column c, rows 8*(i/4) + 4h + (i%4), i = 0..15
// A contraction index may be permuted as long as A and B agree.  Chunk c of
// a D-layout block (elements 8c..8c+7) covers rows 16c + {4h..4h+3} and
// 16c + 8 + {4h..4h+3}; feeding it as a B operand therefore pairs with an A
// operand whose lane reads two runs of 4 consecutive rows of the transposed
// tile.  Those transposed tiles are staged in LDS.
//
// Forward: each wave owns 64 queries and computes S^T = K Q^T (keys x
// queries), so every lane holds one query column: the softmax statistics are
// per lane (one cross-half shuffle), and O^T = V^T P^T accumulates with P^T
// straight from registers.
// Backward: a key-block pass (dK, dV; keys stationary) and a query-block pass
// (dQ; queries stationary), both atomic-free, recomputing P from the stored
// log-sum-exp.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <vector>

#include "kernels.h"

// Forward tiling (queries per wave, waves per workgroup, minimum waves per
// SIMD the register budget must allow).
#ifndef LH_FWD64_QW
#define LH_FWD64_QW 32
#define LH_FWD64_WAVES 4
#define LH_FWD64_MINW 2
#endif
#ifndef LH_FWD128_QW
#define LH_FWD128_QW 32
#define LH_FWD128_WAVES 8
#define LH_FWD128_MINW 2
#endif
// Backward: waves per workgroup of the key-block (dK, dV) and query-block
// (dQ) passes; every wave owns 32 keys or 32 queries.  d = 64 key-block
// passes with at least LH_BKV64_WIDE_MIN workgroups of LH_BKV64_WIDE waves
// use those (wider workgroups share each staged query tile among more keys);
// smaller grids keep LH_BKV64_WAVES, so that enough workgroups exist.
#ifndef LH_BKV64_WIDE
#define LH_BKV64_WIDE 8
#define LH_BKV64_WIDE_MIN 256
#endif
#ifndef LH_BKV64_WAVES
#define LH_BKV64_WAVES 4
#define LH_BKV64_MINW 2
#define LH_BKV128_WAVES 8
#define LH_BKV128_MINW 1
#define LH_BKV128_VLDS 1
#define LH_BQ64_WAVES 4
#define LH_BQ128_WAVES 8
#define LH_BQ64_MINW 2
#define LH_BQ128_MINW 2
#endif

// Causal pairing per pass, off by default: measured neutral or slower in every
// pass (d = 128 key blocks at S = 16K, 32K and 34K: 1.4-9% slower paired).
#ifndef LH_PAIR_FWD
#define LH_PAIR_FWD 0
#endif
#ifndef LH_PAIR_BKV64
#define LH_PAIR_BKV64 0
#endif
#ifndef LH_PAIR_BKV128
#define LH_PAIR_BKV128 0
#endif
#ifndef LH_PAIR_BQ
#define LH_PAIR_BQ 0
#endif

namespace lh {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<__bf16>(0.f);
  return z;
}

// max over lanes l and l ^ 32 (the two halves of a query column)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// acc + the sum of the eight bf16 values of v (two-element dot products with 1)
__device__ __forceinline__ float add_bf16x8(const bf16x8& v, float acc) {
  const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

// ------------------------------------------------------------------ tiles
//
// K/V/Q/dO tiles are staged row-major in LDS by direct global->LDS loads
// (global_load_lds, 16 bytes per lane: lane l of one instruction lands at
// byte 16*l of a 1 KB run).  Rows hold d/8 16-byte chunks whose order is
// XOR-swizzled per row, so that both the row reads of an MFMA A operand
// (16 rows, same chunk) and the transposed reads below hit distinct banks.
//
// Transposed operands come from ds_read_tr16_b64: within each 16-lane group,
// lane i receives element i%4 of the 8-byte reads of lanes i/4, 4+i/4, 8+i/4
// and 12+i/4.  Pointing lane j at row r0 + j/4, columns c0 + 4*(j%4) .. +3
// therefore hands lane i the four rows r0..r0+3 of column c0 + i.

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__host__ __device__ constexpr int swz(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

// byte offset of logical 16-byte chunk x of row r in a swizzled tile
template <int D>
__host__ __device__ constexpr int toff(int r, int x) {
  return r * (D * 2) + ((x ^ swz<D>(r)) << 4);
}

// swz is a permutation of the low row bits, so toff is linear over XOR:
// toff(rc ^ rl, xc ^ xl) = toff(rc, xc) ^ toff(rl, xl) whenever rc and rl
// (and xc and xl) occupy disjoint bits, and rows that are multiples of 16
// have swz = 0, so they only add r * 2D.  Every read address below is
// (lane part ^ chunk part) + row part: the lane part (with the tile's byte
// offset, a multiple of the tile size) is formed once per tile, the few
// distinct chunk parts cost one XOR each per tile, and the row part is an
// immediate offset of the LDS instruction.  Where registers are scarcest,
// kEach = true folds every part into one XOR per read instead, so that no
// per-tile chunk parts stay live.

// Buffer descriptor (raw, stride 0) of `bytes` bytes from p: loads at
// offsets >= bytes return zero.  The record count is an unsigned 32-bit
// field; the host keeps every head's S * d * 2 below 2^32 (M * d < 2^31).
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           __builtin_bit_cast(int, bytes), kBufWord3);
}

// Asynchronously copy rows [r0, r0 + R) of a [S][D] bf16 tensor into a
// swizzled LDS tile with direct buffer loads (16 bytes per lane; lane l of
// one instruction lands at byte 16*l of a 1 KB run).  The descriptor covers
// rows [r0, S), so rows >= S read as zero (they are masked or unused), and
// each instruction needs only a 32-bit lane offset.  Waves w = wave,
// wave + NW, ... of the workgroup split the instructions.
template <int D, int R, int NW>
__device__ __forceinline__ void load_tile(const __bf16* src, int S, int r0, __bf16* tile, int wave,
                                          int lane) {
  constexpr int kCPR = D / 8;
  constexpr int kInst = R * kCPR / 64;
  const int rows = S > r0 ? S - r0 : 0;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src + (int64_t)r0 * D, (uint32_t)rows * (uint32_t)(D * 2));
#pragma unroll
  for (int n = wave; n < kInst; n += NW) {
    const int p = n * 64 + lane;
    const int r = p / kCPR, pc = p % kCPR;
    const int x = pc ^ swz<D>(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + n * 512), 16,
                                             (r * D + x * 8) * 2, 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Row reads (A operand): lane (h, c) reads tile row rc + c, logical chunk
// 2*dc + h (rc a multiple of 32).
template <int D>
__device__ __forceinline__ uint32_t lane_rows(int lane) {
  return (uint32_t)(toff<D>(lane & 31, 0) ^ ((lane >> 5) << 4));
}

__device__ __forceinline__ bf16x8 lds_rows_at(const void* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(static_cast<const char*>(base) + off);
}
template <int D>
constexpr uint32_t cst_rows(int rc, int dc) {
  return (uint32_t)(rc * D * 2 + (dc << 5));
}
template <int D>
constexpr uint32_t cst_tr(int rc, int cb) {
  return (uint32_t)toff<D>(rc, cb >> 3);
}

template <int D, bool kEach = false>
__device__ __forceinline__ bf16x8 lds_rows(const void* base, uint32_t lane_t, int rc, int dc) {
  const char* b = static_cast<const char*>(base);
  if constexpr (kEach)
    return lds_rows_at(base, lane_t ^ cst_rows<D>(rc, dc));
  else
    return *reinterpret_cast<const bf16x8*>(b + (lane_t ^ (uint32_t)(dc << 5)) + rc * D * 2);
}

// Transposed reads (A operand from a row-major tile): lane l (group G = l/16,
// j = l%16, h = l/32) reads row rc + 4h + j/4 at columns cb + 16*(G&1) +
// 4*(j%4) .. +3; the result holds column cb + (l%32) of rows rc + 4h .. +3.
// Reads at rows rc and rc + 8 form one operand (rc a multiple of 16, cb of
// 32).
template <int D>
__device__ __forceinline__ uint32_t lane_tr(int lane) {
  const int j = lane & 15, G = lane >> 4;
  const int rl = 4 * (G >> 1) + (j >> 2);
  const int xl = 2 * (G & 1) + ((j & 3) >> 1);
  return (uint32_t)(toff<D>(rl, xl) + 8 * (j & 1));
}
template <int D, bool kEach = false>
__device__ __forceinline__ bf16x8 lds_tr8(const void* base, uint32_t lane_t, int rc, int cb) {
  const char* b = static_cast<const char*>(base);
  bf16x4 lo, hi;
  if constexpr (kEach) {
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b + (lane_t ^ cst_tr<D>(rc, cb))));
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(b + (lane_t ^ cst_tr<D>(rc + 8, cb))));
  } else {
    const char* br = b + rc * D * 2;
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(br + (lane_t ^ (uint32_t)toff<D>(0, cb >> 3))));
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(br + (lane_t ^ (uint32_t)toff<D>(8, cb >> 3))));
  }
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = lo[e];
    a[e + 4] = hi[e];
  }
  return a;
}

// ------------------------------------------------------------------ grid
//
// One-dimensional grids: workgroup p of T runs on XCD p % 8 (workgroups are
// handed to the eight XCDs round robin).  When the heads split evenly over
// the XCDs, workgroups are remapped so that every XCD owns BH/8 heads and
// walks their query blocks heaviest first (latest queries first, since a
// causal query block costs in proportion to its position), interleaving its
// heads.  Workgroups running together on an XCD then stream the same K/V
// tiles through that XCD's L2 instead of all heads' tiles.
__device__ __forceinline__ void map_block(int p, int T, int BH, int nqb, int& head, int& qblk) {
  if ((BH & 7) == 0) {
    const int x = p & 7, local = p >> 3;
    const int hpx = BH >> 3;
    head = x * hpx + local % hpx;
    qblk = nqb - 1 - local / hpx;
  } else {
    head = p % BH;
    qblk = nqb - 1 - p / BH;
  }
  (void)T;
}

// Causal pairing: block b costs in proportion to b + 1 (or to nb - b for key
// blocks), so a workgroup that runs blocks r and nb - 1 - r back to back does
// the same work as every other one.  Without pairing the heaviest blocks set
// the kernel's length while the light ones leave compute units idle at the
// end.  Small grids are not paired (halving them would leave units idle).
// Returns the workgroup's head and its one or two blocks in run order
// (`rank` counts from the heavy end: block nb - 1 - rank for query blocks).
struct Runs {
  int head, n, rank[2];
};

__device__ __forceinline__ Runs plan_runs(int p, int T, int nb, int paired) {
  Runs r;
  if (!paired) {
    int qblk;
    map_block(p, T, T / nb, nb, r.head, qblk);
    r.n = 1;
    r.rank[0] = nb - 1 - qblk;
    r.rank[1] = 0;
    return r;
  }
  const int np = (nb + 1) / 2;
  const int BH = T / np;
  int pair;
  if ((BH & 7) == 0) {
    const int x = p & 7, local = p >> 3, hpx = BH >> 3;
    r.head = x * hpx + local % hpx;
    pair = local / hpx;
  } else {
    r.head = p % BH;
    pair = p / BH;
  }
  r.rank[0] = pair;            // heavy: rank pair from the heavy end
  r.rank[1] = nb - 1 - pair;   // light partner
  r.n = r.rank[1] > r.rank[0] ? 2 : 1;
  return r;
}

// Number of workgroups of a (possibly paired) causal grid.
inline int64_t causal_grid(int64_t nb, int64_t BH, bool paired) {
  return (paired ? (nb + 1) / 2 : nb) * BH;
}

inline bool pair_blocks(int64_t nb, int64_t BH) { return nb * BH >= 1024 && nb >= 2; }

// ------------------------------------------------------------------ forward
//
// Online softmax with lazy rescaling: a row keeps its running maximum m
// until a tile raises it by more than 2^8 (in exp2 units); until then
// probabilities exp2(s - m) may exceed 1 by at most that factor, which
// float32 sums and bf16 operands hold exactly as well.  The decision is taken
// for the whole wave, so the rescale of the accumulators is a uniform branch
// that is skipped on almost every tile.

constexpr float kLazyRescale = 8.0f;

template <int D, int QW, int WAVES>
struct FwdCfg {
  static constexpr int kQW = QW;                 // queries per wave
  static constexpr int kNQB = QW / 32;           // 32-query blocks per wave
  static constexpr int kWaves = WAVES;
  static constexpr int kQB = WAVES * QW;         // queries per workgroup
  static constexpr int kKT = 64;                 // keys per tile
  static constexpr int kTile = kKT * D;          // elements per K or V tile
  static constexpr int kThreads = 64 * WAVES;
};

// Key-range split (FwdSplit::n > 0), for causal grids too small to balance:
// the heaviest query blocks (those with more key tiles than the mean load of
// a resident workgroup slot) each run as two workgroups, chunk 0 over the
// first half of the block's key tiles and chunk 1 over the rest (which holds
// the diagonal).  A chunk writes its partial result, the output normalised by
// its own sum and lambda = m + log2(sum) per query (chunk 1 into O and LSE,
// chunk 0 into the split buffers); attn_fwd_merge then combines the two:
//   w_c = exp2(lambda_c - max lambda), O = (w_0 y_0 + w_1 y_1) / (w_0 + w_1).
// order[] lists every head's work items (whole blocks and chunks) by
// decreasing number of key tiles; workgroups take them in that order.
constexpr int kSplitItems = 1024;
struct FwdSplit {
  float* o;      // [BH][S][D] chunk-0 partial outputs
  float* lam;    // [BH][S] chunk-0 lambda (log2 units)
  int32_t n;     // work items per head (0: no split)
  uint16_t order[kSplitItems];  // item = query block << 2 | kind (0 whole, 1 chunk 0, 2 chunk 1)
};

template <int D, int QW, int WAVES, int MINW>
__global__ __launch_bounds__(64 * WAVES, MINW) void attn_fwd_bf16(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int S, float sl2, int paired, FwdSplit sp) {
  using C = FwdCfg<D, QW, WAVES>;
  constexpr int NQB = C::kNQB;
  __shared__ __attribute__((aligned(1024))) __bf16 sKV[2][2][C::kTile];  // [buffer][K,V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h = lane >> 5, c32 = lane & 31;
  const uint32_t lrow = lane_rows<D>(lane), ltr = lane_tr<D>(lane);
  const int nqb = (S + C::kQB - 1) / C::kQB;
  const bool split = sp.n > 0;
  const Runs runs = plan_runs(blockIdx.x, gridDim.x, split ? sp.n : nqb, split ? 0 : paired);
  const int64_t bh = __builtin_amdgcn_readfirstlane(runs.head);
  for (int run = 0; run < runs.n; ++run) {
  if (run > 0) __syncthreads();  // every wave is done with the LDS tiles
  const int rank = __builtin_amdgcn_readfirstlane(runs.rank[run]);
  // split: the rank-th item of the list (kind 0 whole block, 1 chunk 0, 2 chunk 1)
  const int code = split ? (int)sp.order[rank] : 0;
  const int qblk = split ? code >> 2 : nqb - 1 - rank;
  const int kind = code & 3;
  const int q0 = qblk * C::kQB;
  const int qw0 = q0 + wave * C::kQW;
  const __bf16* Qh = Q + bh * (int64_t)S * D;
  const __bf16* Kh = K + bh * (int64_t)S * D;
  const __bf16* Vh = V + bh * (int64_t)S * D;

  const int kend = min(S, q0 + C::kQB);
  const int nall = (kend + C::kKT - 1) / C::kKT;
  const int kt0 = kind == 2 ? nall >> 1 : 0;        // this workgroup's key tiles
  const int ntiles = kind == 1 ? nall >> 1 : nall;  // [kt0, ntiles)
  if (kt0 < ntiles) {
    load_tile<D, C::kKT, WAVES>(Kh, S, kt0 * C::kKT, sKV[kt0 & 1][0], wave, lane);
    load_tile<D, C::kKT, WAVES>(Vh, S, kt0 * C::kKT, sKV[kt0 & 1][1], wave, lane);
  }

  bf16x8 qreg[NQB][D / 16];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = qw0 + qb * 32 + c32;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      qreg[qb][dc] = row < S ? *reinterpret_cast<const bf16x8*>(Qh + (int64_t)row * D + dc * 16 + 8 * h)
                             : zero8();
  }
  f32x16 oacc[NQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) oacc[qb][mb] = zero16();
  float mrow[NQB], lsum[NQB];   // running max (exp2 units) and sum per query
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    mrow[qb] = neg_inf();
    lsum[qb] = 0.f;
  }

  for (int kt = kt0; kt < ntiles; ++kt) {
    const int k0 = kt * C::kKT;
    wait_loads();
    __syncthreads();  // tile kt is in LDS; buffer (kt+1)&1 is free
    if (kt + 1 < ntiles) {
      load_tile<D, C::kKT, WAVES>(Kh, S, k0 + C::kKT, sKV[(kt + 1) & 1][0], wave, lane);
      load_tile<D, C::kKT, WAVES>(Vh, S, k0 + C::kKT, sKV[(kt + 1) & 1][1], wave, lane);
    }
    if (qw0 >= S || k0 > qw0 + C::kQW - 1) continue;  // nothing visible for this wave
    // lane parts of this tile's reads (K and V tiles of buffer kt & 1)
    const uint32_t kbo = (uint32_t)((kt & 1) * 2 * C::kTile * 2);
    const uint32_t lk = lrow ^ kbo;
    const uint32_t lv = ltr ^ (kbo + C::kTile * 2);

    // Issue every LDS read of this tile before the first MFMA that needs it
    // (the V^T operands do not depend on the scores, so their latency hides
    // under the QK^T products and the softmax); with two query blocks per
    // wave both use the same operands, which halves LDS traffic per product.
    bf16x8 kop[2][D / 16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) kop[kb][dc] = lds_rows<D>(sKV, lk, kb * 32, dc);
    bf16x8 vop[2][2][D / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
          vop[kb][c][mb] = lds_tr8<D>(sKV, lv, kb * 32 + 16 * c, mb * 32);

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qbase = qw0 + qb * 32;
      if (k0 > qbase + 31) continue;
      f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(kop[kb][dc], qreg[qb][dc], sacc[kb]);
      const int query = qbase + c32;
      float mx = neg_inf();   // max of raw scores (the scale is positive)
      if (k0 + C::kKT - 1 > qbase) {  // diagonal tile: causal mask
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key > query) sacc[kb][i] = neg_inf();
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      // This lane's half of the tile; the running maximum is shared by both
      // halves, so the exact column maximum is needed only to rescale.
      mx *= sl2;
      if (__any(mx > mrow[qb] + kLazyRescale)) {  // wave-uniform
        const float mnew = fmaxf(mrow[qb], max_halves(mx));
        const float alpha = fexp2(mrow[qb] - mnew);
        lsum[qb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) oacc[qb][mb] *= alpha;
        mrow[qb] = mnew;
      }
      const float nm = -mrow[qb];
      bf16x8 pk[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pk[kb][c][e] = static_cast<__bf16>(fexp2(__builtin_fmaf(sacc[kb][8 * c + e], sl2, nm)));
          // the normaliser sums the rounded weights the products use
          lsum[qb] = add_bf16x8(pk[kb][c], lsum[qb]);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb)
            oacc[qb][mb] = mfma32(vop[kb][c][mb], pk[kb][c], oacc[qb][mb]);
    }
  }

  float* Oh = O + bh * (int64_t)S * D;
  float* Lh = LSE + bh * (int64_t)S;
  if (qw0 < S) {
    // kind 1 writes to the split buffers; kinds 1 and 2 write partials
    float* dO_ = kind == 1 ? sp.o + bh * (int64_t)S * D : Oh;
    float* dL = kind == 1 ? sp.lam + bh * (int64_t)S : Lh;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float lt = lsum[qb] + __shfl_xor(lsum[qb], 32);
      // a chunk that saw none of the query's keys holds an empty partial
      const float inv = kind == 0 || lt > 0.f ? 1.0f / lt : 0.f;
      const float lam = kind == 0 || lt > 0.f ? mrow[qb] + log2f(lt) : neg_inf();
      const int query = qw0 + qb * 32 + c32;
      if (query < S) {
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = oacc[qb][mb][4 * j + r] * inv;
            *reinterpret_cast<f32x4*>(dO_ + (int64_t)query * D + mb * 32 + 8 * j + 4 * h) = o;
          }
        if (h == 0) dL[query] = kind == 0 ? lam * kLn2 : lam;
      }
    }
  }
  }  // run
}

// Combines the two chunks of every split query block (rows [r0, S) of each
// head, the blocks from the first split one on): chunk 0's partial from the
// split buffers, chunk 1's from O and LSE (lambda in log2 units), both
// written by attn_fwd_bf16; writes the final O and the natural-log LSE.
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_merge(float* __restrict__ O, float* __restrict__ LSE,
                                                      const float* __restrict__ P0,
                                                      const float* __restrict__ L0, int S, int r0) {
  constexpr int kLanes = D / 4, kRows = 256 / kLanes;
  const int64_t bh = blockIdx.y;
  const int row = r0 + (int)blockIdx.x * kRows + (int)threadIdx.x / kLanes;
  const int lane = threadIdx.x % kLanes;
  if (row >= S) return;
  const int64_t ri = bh * (int64_t)S + row;
  const float l0 = L0[ri], l1 = LSE[ri];
  const float lm = fmaxf(l0, l1);  // finite: one chunk holds the query's own key
  const float w0 = fexp2(l0 - lm), w1 = fexp2(l1 - lm);
  const float wt = w0 + w1;
  const float inv = 1.0f / wt;
  const int64_t at = ri * D + 4 * lane;
  const f32x4 y0 = *reinterpret_cast<const f32x4*>(P0 + at);
  const f32x4 y1 = *reinterpret_cast<const f32x4*>(O + at);
  f32x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = (w0 * y0[r] + w1 * y1[r]) * inv;
  *reinterpret_cast<f32x4*>(O + at) = o;
  if (lane == 0) LSE[ri] = (lm + log2f(wt)) * kLn2;
}

// ------------------------------------------------------------------ backward

// delta[i] = sum_d dO[i,d] * O[i,d], one row per d/8-lane group, for the
// float32 storage path (the bf16 path forms it in its dQ pass), accumulated
// in float64 like every dot product of that path (the backward subtracts
// delta from dP for each key).  O is the float32 forward output in both
// paths: rounding it to bf16 first would perturb delta by ~2^-9 |dO||O|, and
// dS = P (dP - delta) cancels for keys that dominate a row, which would
// amplify that error in dK and dQ.
__global__ __launch_bounds__(256) void attn_delta_f32(const float* __restrict__ O,
                                                      const float* __restrict__ dO,
                                                      float* __restrict__ delta, int64_t rows,
                                                      int d) {
  const int lpr = d / 8;
  const int rgs = 256 / lpr;
  const int lane = threadIdx.x % lpr;
  const int64_t row = (int64_t)blockIdx.x * rgs + threadIdx.x / lpr;
  double s = 0;
  if (row < rows) {
    float o[8], g[8];
    Row8<float>::load(O + row * d + 8 * lane, o);
    Row8<float>::load(dO + row * d + 8 * lane, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (double)o[e] * (double)g[e];
  }
  for (int off = lpr >> 1; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && lane == 0) delta[row] = (float)s;
}

// Stage 64 float32 values (lse or delta of a query tile) into LDS with one
// direct load (4 bytes per lane); rows >= S read as zero (masked queries).
__device__ __forceinline__ void load_vec64(const float* src, int S, int r0, float* dst, int lane) {
  const int rows = S > r0 ? S - r0 : 0;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(src + r0, (uint32_t)rows * 4u), (lds_void*)dst, 4, lane * 4, 0,
                                           0, 0);
}

// Key-block pass: each wave keeps 32 keys (K and V rows as MFMA B operands)
// and walks the query tiles from its block's diagonal to the end, producing
// dK and dV with no atomics.  Per 32-query slice:
//   S = Q K^T, dP = dO V^T         (A = Q / dO rows from LDS)
//   P = exp2(S*scale*log2e - lse*log2e), dS = P (dP - delta)
//   dV^T += dO^T P, dK^T += Q^T dS  (A = transposed reads of the Q / dO tiles)
template <int D, int WAVES>
struct BwdKVCfg {
  static constexpr int kKW = 32;
  static constexpr int kKB = WAVES * kKW;  // keys per workgroup
  static constexpr int kQT = 64;           // queries per tile
  static constexpr int kTile = kQT * D;
};

// P and dS of a 32-query x 32-key slice in B-operand chunks (key column per
// lane).  sL holds lse * log2(e), sD rowsum(dO*O) of the query tile.
template <bool kMask>
__device__ __forceinline__ void kv_weights(const f32x16& sacc, const f32x16& dpacc, const float* sL,
                                           const float* sD, int qs, int h, float sl2, int key,
                                           int q0, int S, bf16x8 (&pch)[2], bf16x8 (&dsch)[2]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int qi = qs * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
    float p = fexp2(__builtin_fmaf(sacc[i], sl2, -sL[qi]));
    if (kMask && (key > q0 + qi || q0 + qi >= S)) p = 0.f;
    pch[i >> 3][i & 7] = static_cast<__bf16>(p);
    dsch[i >> 3][i & 7] = static_cast<__bf16>(p * (dpacc[i] - sD[qi]));
  }
}

template <int D, int WAVES, int MINW>
__global__ __launch_bounds__(64 * WAVES, MINW) void attn_bwd_dkdv_bf16(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ DELTA,
    float* __restrict__ dK, float* __restrict__ dV, int S, float sl2, float scale, int paired) {
  using C = BwdKVCfg<D, WAVES>;
  // d = 128: the wave's 32 V rows live in LDS instead of registers (the
  // register file would otherwise spill); they are the B operand of dP.
  constexpr bool kVInLds = D == 128 && LH_BKV128_VLDS;
  constexpr bool kEach = D == 128;  // register budget: one XOR per LDS read
  // Q, dO, lse and rowsum tiles in two buffers each.  d = 64: every buffer
  // its own array and each tile step compiled for one parity, so that the
  // step's LDS reads need not wait for the next tile's direct loads (2-3%
  // faster).  d = 128: one array of all four tiles and one loop body, the
  // parity a run-time offset of the lane part of each read: there the
  // register file is full, and both the parity copies and a shared helper
  // for the slice code (as d = 64 uses) raise the spills from 23 to 39 or
  // more, which costs 10%, so that path keeps its own copy of the slices.
  constexpr bool kSplit = D == 64;
  constexpr int kT1 = kSplit ? C::kTile : 8, kQ1 = kSplit ? C::kQT : 1;
  __shared__ __attribute__((aligned(1024))) __bf16 sQ0[kSplit ? C::kTile : 4 * C::kTile];
  __shared__ __attribute__((aligned(1024))) __bf16 sG0[kT1];
  __shared__ __attribute__((aligned(1024))) __bf16 sQ1[kT1];
  __shared__ __attribute__((aligned(1024))) __bf16 sG1[kT1];
  __shared__ __attribute__((aligned(1024))) __bf16 sVw[kVInLds ? WAVES : 1][kVInLds ? 32 * D : 8];
  __shared__ float sL0[kSplit ? C::kQT : 4 * C::kQT], sD0[kQ1], sL1[kQ1], sD1[kQ1];
  // tiles of parity P: Q, dO, lse, rowsum
  auto tQ = [&](int P) __attribute__((always_inline)) { return kSplit ? (P ? sQ1 : sQ0) : sQ0 + 2 * P * C::kTile; };
  auto tG = [&](int P) __attribute__((always_inline)) { return kSplit ? (P ? sG1 : sG0) : sQ0 + (2 * P + 1) * C::kTile; };
  auto tL = [&](int P) __attribute__((always_inline)) { return kSplit ? (P ? sL1 : sL0) : sL0 + 2 * P * C::kQT; };
  auto tD = [&](int P) __attribute__((always_inline)) { return kSplit ? (P ? sD1 : sD0) : sL0 + (2 * P + 1) * C::kQT; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h = lane >> 5, c32 = lane & 31;
  const uint32_t lrow = lane_rows<D>(lane), ltr = lane_tr<D>(lane);
  const uint32_t lvw = lrow ^ (uint32_t)(kVInLds ? wave * 32 * D * 2 : 0);  // this wave's V rows
  const int nkb = (S + C::kKB - 1) / C::kKB;
  const Runs runs = plan_runs(blockIdx.x, gridDim.x, nkb, paired);
  const int64_t bh = __builtin_amdgcn_readfirstlane(runs.head);
  for (int run = 0; run < runs.n; ++run) {
  if (run > 0) __syncthreads();  // every wave is done with the LDS tiles
  const int kblk = __builtin_amdgcn_readfirstlane(runs.rank[run]);  // early keys (most queries) are the heavy end
  const int kb0 = kblk * C::kKB;
  const int kw0 = kb0 + wave * C::kKW;
  const int key = kw0 + c32;
  const int64_t off = bh * (int64_t)S * D;
  const float* lse_h = LSE2 + bh * (int64_t)S;
  const float* del_h = DELTA + bh * (int64_t)S;

  const int t0 = kb0 / C::kQT;
  const int ntiles = (S + C::kQT - 1) / C::kQT;
  auto issue = [&](int P, int t) __attribute__((always_inline)) {
    load_tile<D, C::kQT, WAVES>(Q + off, S, t * C::kQT, tQ(P), wave, lane);
    load_tile<D, C::kQT, WAVES>(dO + off, S, t * C::kQT, tG(P), wave, lane);
    if (wave == 0) load_vec64(lse_h, S, t * C::kQT, tL(P), lane);
    if (wave == WAVES - 1) load_vec64(del_h, S, t * C::kQT, tD(P), lane);
  };
  issue(0, t0);

  bf16x8 kreg[D / 16], vreg[kVInLds ? 1 : D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    kreg[dc] = key < S ? *reinterpret_cast<const bf16x8*>(K + off + (int64_t)key * D + dc * 16 + 8 * h) : zero8();
  if constexpr (kVInLds) {
    load_tile<D, 32, 1>(V + off, S, kw0, sVw[wave], 0, lane);  // landed by the first barrier
  } else {
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
      vreg[dc] = key < S ? *reinterpret_cast<const bf16x8*>(V + off + (int64_t)key * D + dc * 16 + 8 * h) : zero8();
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    dka[mb] = zero16();
    dva[mb] = zero16();
  }

  // d = 64: query tile t in the buffers of parity PAR = (t - t0) & 1
  auto tile_step = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    const __bf16* bQ = tQ(PAR);
    const __bf16* bG = tG(PAR);
    const float* sL = tL(PAR);
    const float* sD = tD(PAR);
    const int q0 = t * C::kQT;
    wait_loads();
    __syncthreads();
    if (t + 1 < ntiles) issue(1 - PAR, t + 1);
    if (kw0 >= S || q0 + C::kQT - 1 < kw0) return;
    const uint32_t lvt = lvw;
    const uint32_t lq = lrow, lg = lrow, tq = ltr, tg = ltr;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      // d = 128: keep the scheduler from hoisting the next slice's reads
      // (their registers would push live values out to scratch)
      if constexpr (kEach) __builtin_amdgcn_sched_barrier(0);
      const int qbase = q0 + qs * 32;
      if (qbase + 31 < kw0) continue;
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        sacc = mfma32(lds_rows<D, kEach>(bQ, lq, qs * 32, dc), kreg[dc], sacc);
        const bf16x8 vb = kVInLds ? lds_rows<D, kEach>(sVw, lvt, 0, dc) : vreg[kVInLds ? 0 : dc];
        dpacc = mfma32(lds_rows<D, kEach>(bG, lg, qs * 32, dc), vb, dpacc);
      }
      // Only a slice that meets the diagonal or the end of the sequence needs
      // masks (a wave-uniform branch keeps them off every other slice).
      bf16x8 pch[2], dsch[2];
      if (qbase < kw0 + 31 || q0 + C::kQT > S)
        kv_weights<true>(sacc, dpacc, sL, sD, qs, h, sl2, key, q0, S, pch, dsch);
      else
        kv_weights<false>(sacc, dpacc, sL, sD, qs, h, sl2, key, q0, S, pch, dsch);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          dva[mb] = mfma32(lds_tr8<D, kEach>(bG, tg, qs * 32 + 16 * c, mb * 32), pch[c], dva[mb]);
          dka[mb] = mfma32(lds_tr8<D, kEach>(bQ, tq, qs * 32 + 16 * c, mb * 32), dsch[c], dka[mb]);
        }
    }
  };
  if constexpr (kSplit) {
    for (int t = t0; t < ntiles; t += 2) {
      tile_step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < ntiles) tile_step(std::integral_constant<int, 1>{}, t + 1);
    }
  } else {  // d = 128
    for (int t = t0; t < ntiles; ++t) {
      const int buf = (t - t0) & 1;
      const int q0 = t * C::kQT;
      wait_loads();
      __syncthreads();
      if (t + 1 < ntiles) issue(buf ^ 1, t + 1);
      if (kw0 >= S || q0 + C::kQT - 1 < kw0) continue;
      const uint32_t tbo = (uint32_t)(buf * 2 * C::kTile * 2);  // Q tile; the dO tile follows
      const uint32_t lvt = lvw;
      const uint32_t lq = lrow ^ tbo, lg = lrow ^ (tbo + C::kTile * 2);
      const uint32_t tq = ltr ^ tbo, tg = ltr ^ (tbo + C::kTile * 2);
      const float* sL = tL(buf);
      const float* sD = tD(buf);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        // d = 128: keep the scheduler from hoisting the next slice's reads
        // (their registers would push live values out to scratch)
        if constexpr (kEach) __builtin_amdgcn_sched_barrier(0);
        const int qbase = q0 + qs * 32;
        if (qbase + 31 < kw0) continue;
        f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          sacc = mfma32(lds_rows<D, kEach>(sQ0, lq, qs * 32, dc), kreg[dc], sacc);
          const bf16x8 vb = kVInLds ? lds_rows<D, kEach>(sVw, lvt, 0, dc) : vreg[kVInLds ? 0 : dc];
          dpacc = mfma32(lds_rows<D, kEach>(sQ0, lg, qs * 32, dc), vb, dpacc);
        }
        // Only a slice that meets the diagonal or the end of the sequence needs
        // masks (a wave-uniform branch keeps them off every other slice).
        bf16x8 pch[2], dsch[2];
        if (qbase < kw0 + 31 || q0 + C::kQT > S)
          kv_weights<true>(sacc, dpacc, sL, sD, qs, h, sl2, key, q0, S, pch, dsch);
        else
          kv_weights<false>(sacc, dpacc, sL, sD, qs, h, sl2, key, q0, S, pch, dsch);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb) {
            dva[mb] = mfma32(lds_tr8<D, kEach>(sQ0, tg, qs * 32 + 16 * c, mb * 32), pch[c], dva[mb]);
            dka[mb] = mfma32(lds_tr8<D, kEach>(sQ0, tq, qs * 32 + 16 * c, mb * 32), dsch[c], dka[mb]);
          }
      }
    }
  }
  if (key < S) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 a, b;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = dka[mb][4 * j + r] * scale;
          b[r] = dva[mb][4 * j + r];
        }
        const int64_t o = off + (int64_t)key * D + mb * 32 + 8 * j + 4 * h;
        *reinterpret_cast<f32x4*>(dK + o) = a;
        *reinterpret_cast<f32x4*>(dV + o) = b;
      }
  }
  }  // run
}

// Query-block pass: each wave keeps 32 queries (Q and dO rows as B operands,
// lse and delta in registers) and walks the key tiles up to its diagonal:
//   S^T = K Q^T, dP^T = V dO^T      (A = K / V rows from LDS)
//   dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T (A = transposed reads of K)
// Every query belongs to one wave of this pass, so the pass also forms its
// delta = rowsum(dO*O) and lse*log2(e) and writes them for the key-block
// pass, which runs after it.
template <int D, int WAVES>
struct BwdQCfg {
  static constexpr int kQW = 32;
  static constexpr int kQB = WAVES * kQW;
  static constexpr int kKT = 64;
  static constexpr int kTile = kKT * D;
};

// dS^T of a 32-key x 32-query slice in B-operand chunks (query column per
// lane); lse2 = lse * log2(e) of the lane's query, and dpacc already holds
// dP^T - rowsum(dO*O) (its products accumulate onto -rowsum).
template <bool kMask>
__device__ __forceinline__ void q_weights(const f32x16& sacc, const f32x16& dpacc, float lse2,
                                          float sl2, int kbase, int h, int query,
                                          bf16x8 (&dsch)[2]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float p = fexp2(__builtin_fmaf(sacc[i], sl2, -lse2));
    if (kMask && kbase + 8 * (i >> 2) + 4 * h + (i & 3) > query) p = 0.f;
    dsch[i >> 3][i & 7] = static_cast<__bf16>(p * dpacc[i]);
  }
}

template <int D, int WAVES, int MINW>
__global__ __launch_bounds__(64 * WAVES, MINW) void attn_bwd_dq_bf16(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ LSE2, float* __restrict__ DELTA, float* __restrict__ dQ, int S, float sl2,
    float scale, int paired) {
  using C = BwdQCfg<D, WAVES>;
  // K and V tiles in two buffers each.  d = 64: every buffer its own array
  // and each tile step compiled for one parity (reads need not wait for the
  // loads); d = 128: one array and one loop body, the parity a run-time offset
  // of the lane part of each read (the register budget of the key-block
  // pass, kept alike here)
  constexpr bool kSplit = D == 64;
  constexpr int kT1 = kSplit ? C::kTile : 8;
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[kSplit ? C::kTile : 4 * C::kTile];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[kT1];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[kT1];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[kT1];
  auto tK = [&](int P) __attribute__((always_inline)) { return kSplit ? (P ? sK1 : sK0) : sK0 + 2 * P * C::kTile; };
  auto tV = [&](int P) __attribute__((always_inline)) { return kSplit ? (P ? sV1 : sV0) : sK0 + (2 * P + 1) * C::kTile; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int h = lane >> 5, c32 = lane & 31;
  const uint32_t lrow = lane_rows<D>(lane), ltr = lane_tr<D>(lane);
  const int nqb = (S + C::kQB - 1) / C::kQB;
  const Runs runs = plan_runs(blockIdx.x, gridDim.x, nqb, paired);
  const int64_t bh = __builtin_amdgcn_readfirstlane(runs.head);
  for (int run = 0; run < runs.n; ++run) {
  if (run > 0) __syncthreads();  // every wave is done with the LDS tiles
  const int qblk = nqb - 1 - __builtin_amdgcn_readfirstlane(runs.rank[run]);
  const int q0 = qblk * C::kQB;
  const int qw0 = q0 + wave * C::kQW;
  const int query = qw0 + c32;
  const int64_t off = bh * (int64_t)S * D;

  const int kend = min(S, q0 + C::kQB);
  const int ntiles = (kend + C::kKT - 1) / C::kKT;
  load_tile<D, C::kKT, WAVES>(K + off, S, 0, tK(0), wave, lane);
  load_tile<D, C::kKT, WAVES>(V + off, S, 0, tV(0), wave, lane);

  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    qreg[dc] = query < S ? *reinterpret_cast<const bf16x8*>(Q + off + (int64_t)query * D + dc * 16 + 8 * h) : zero8();
    doreg[dc] = query < S ? *reinterpret_cast<const bf16x8*>(dO + off + (int64_t)query * D + dc * 16 + 8 * h) : zero8();
  }
  // rowsum(dO*O) and lse*log2(e) of the lane's query, written for the
  // key-block pass that runs after this one: the two halves of the wave hold
  // the two halves of the query's dO row
  float dl = 0.f, lse2 = 0.f;
  if (query < S) {
    const float* orow = O + off + (int64_t)query * D + 8 * h;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(orow + dc * 16);
      const f32x4 b = *reinterpret_cast<const f32x4*>(orow + dc * 16 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dl = __builtin_fmaf((float)doreg[dc][e], a[e], dl);
        dl = __builtin_fmaf((float)doreg[dc][4 + e], b[e], dl);
      }
    }
    lse2 = LSE[bh * (int64_t)S + query] * kLog2e;
  }
  dl += __shfl_xor(dl, 32);
  if (query < S && h == 0) {
    DELTA[bh * (int64_t)S + query] = dl;
    LSE2[bh * (int64_t)S + query] = lse2;
  }
  f32x16 dqa[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) dqa[mb] = zero16();
  // the dP^T products start from -rowsum(dO*O) of the lane's query (the lane
  // is fixed for the whole pass), which saves a subtraction per weight
  f32x16 negdl;
#pragma unroll
  for (int i = 0; i < 16; ++i) negdl[i] = -dl;

  // key tile kt, held in the buffers of parity kt & 1 = PAR
  // d = 64: key tile kt in the buffers of parity PAR = kt & 1
  auto tile_step = [&](auto par, int kt) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    const __bf16* bK = tK(PAR);
    const __bf16* bV = tV(PAR);
    const int k0 = kt * C::kKT;
    wait_loads();
    __syncthreads();
    if (kt + 1 < ntiles) {
      load_tile<D, C::kKT, WAVES>(K + off, S, k0 + C::kKT, tK(1 - PAR), wave, lane);
      load_tile<D, C::kKT, WAVES>(V + off, S, k0 + C::kKT, tV(1 - PAR), wave, lane);
    }
    if (qw0 >= S || k0 > qw0 + C::kQW - 1) return;
    const uint32_t lk = lrow, lv = lrow, tk = ltr;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kbase = k0 + kb * 32;
      if (kbase > qw0 + 31) continue;
      f32x16 sacc = zero16(), dpacc = negdl;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        sacc = mfma32(lds_rows<D>(bK, lk, kb * 32, dc), qreg[dc], sacc);
        dpacc = mfma32(lds_rows<D>(bV, lv, kb * 32, dc), doreg[dc], dpacc);
      }
      bf16x8 dsch[2];
      if (kbase + 31 > qw0)  // diagonal slice (wave-uniform)
        q_weights<true>(sacc, dpacc, lse2, sl2, kbase, h, query, dsch);
      else
        q_weights<false>(sacc, dpacc, lse2, sl2, kbase, h, query, dsch);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
          dqa[mb] = mfma32(lds_tr8<D>(bK, tk, kb * 32 + 16 * c, mb * 32), dsch[c], dqa[mb]);
    }
  };
  if constexpr (kSplit) {
    for (int kt = 0; kt < ntiles; kt += 2) {
      tile_step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < ntiles) tile_step(std::integral_constant<int, 1>{}, kt + 1);
    }
  } else {  // d = 128
    for (int kt = 0; kt < ntiles; ++kt) {
      const int k0 = kt * C::kKT;
      wait_loads();
      __syncthreads();
      if (kt + 1 < ntiles) {
        load_tile<D, C::kKT, WAVES>(K + off, S, k0 + C::kKT, sK0 + 2 * ((kt + 1) & 1) * C::kTile, wave, lane);
        load_tile<D, C::kKT, WAVES>(V + off, S, k0 + C::kKT, sK0 + (2 * ((kt + 1) & 1) + 1) * C::kTile, wave, lane);
      }
      if (qw0 >= S || k0 > qw0 + C::kQW - 1) continue;
      const uint32_t kbo = (uint32_t)((kt & 1) * 2 * C::kTile * 2);  // K tile; the V tile follows
      const uint32_t lk = lrow ^ kbo, lv = lrow ^ (kbo + C::kTile * 2), tk = ltr ^ kbo;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kbase = k0 + kb * 32;
        if (kbase > qw0 + 31) continue;
        f32x16 sacc = zero16(), dpacc = negdl;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          sacc = mfma32(lds_rows<D>(sK0, lk, kb * 32, dc), qreg[dc], sacc);
          dpacc = mfma32(lds_rows<D>(sK0, lv, kb * 32, dc), doreg[dc], dpacc);
        }
        bf16x8 dsch[2];
        if (kbase + 31 > qw0)  // diagonal slice (wave-uniform)
          q_weights<true>(sacc, dpacc, lse2, sl2, kbase, h, query, dsch);
        else
          q_weights<false>(sacc, dpacc, lse2, sl2, kbase, h, query, dsch);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int mb = 0; mb < D / 32; ++mb)
            dqa[mb] = mfma32(lds_tr8<D>(sK0, tk, kb * 32 + 16 * c, mb * 32), dsch[c], dqa[mb]);
      }
    }
  }
  if (query < S) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = dqa[mb][4 * j + r] * scale;
        *reinterpret_cast<f32x4*>(dQ + off + (int64_t)query * D + mb * 32 + 8 * j + 4 * h) = a;
      }
  }
  }  // run
}

}  // namespace

// fp32 paths live in attention_f32.hip
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int64_t S, int d, int64_t BH, hipStream_t st);
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* lse,
                               const float* delta, const float* dout, float* dq, float* dk,
                               float* dv, int64_t S, int d, int64_t BH, hipStream_t st,
                               hipEvent_t* ev);

namespace {
// Workgroups of the forward kernel resident at once on the current device
// (compute units x workgroups per unit), looked up once per device.
template <typename Kern>
int64_t resident_slots(Kern kern, int threads) {
  static std::atomic<int64_t> cache[64];  // host threads may race to fill it: same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, 0) != hipSuccess)
      return 0;
    v = (int64_t)cus * per;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

#ifndef LH_FWD_SPLIT
#define LH_FWD_SPLIT 1
#endif

// The split plan of a causal forward grid that fits in one round of the
// resident workgroup slots (grids with more workgroups than slots balance
// well enough by themselves: at 16 heads of 8,192 rows, 1.33 workgroups per
// slot, the split measured 3% slower, while at 16 heads of 4,096 rows and
// d = 128, one workgroup per slot, the forward went 0.125 -> 0.108 ms).
// Blocks with more key tiles than the mean load per slot (total tiles /
// slots) run as two chunks.  Fills sp.n and sp.order (items by decreasing
// tiles, ties by block, then kind); returns the first split block (nb if none).
int64_t plan_split(int64_t S, int64_t nb, int qb, int64_t BH, int64_t slots, FwdSplit& sp) {
  sp.n = 0;
  if (!LH_FWD_SPLIT || slots <= 0 || nb < 2 || nb * BH > slots) return nb;
  auto tiles = [&](int64_t b) { return (std::min<int64_t>(S, (b + 1) * qb) + 63) / 64; };
  int64_t total = 0;
  for (int64_t b = 0; b < nb; ++b) total += tiles(b);
  const int64_t mean = (total * BH + slots - 1) / slots;
  int64_t b0 = nb;  // tiles(b) is nondecreasing: the split blocks are a suffix
  while (b0 > 0 && tiles(b0 - 1) > mean && tiles(b0 - 1) >= 2) --b0;
  if (b0 == nb || nb + (nb - b0) > kSplitItems || nb >= (1 << 14)) return nb;
  struct Item { int64_t w; int code; };
  std::vector<Item> it;
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t t = tiles(b);
    if (b < b0) {
      it.push_back({t, (int)(b << 2)});
    } else {
      it.push_back({t >> 1, (int)(b << 2 | 1)});
      it.push_back({t - (t >> 1), (int)(b << 2 | 2)});
    }
  }
  std::stable_sort(it.begin(), it.end(), [](const Item& x, const Item& y) {
    return x.w != y.w ? x.w > y.w : x.code > y.code;
  });
  sp.n = (int32_t)it.size();
  for (size_t i = 0; i < it.size(); ++i) sp.order[i] = (uint16_t)it[i].code;
  return b0;
}

template <int D, int QW, int WAVES, int MINW>
hipError_t fwd_bf16(const __bf16* Q, const __bf16* K, const __bf16* V, float* o, float* lse,
                    int64_t S, int64_t BH, float sl2, const FwdSplitBufs* sb, hipStream_t st) {
  using C = FwdCfg<D, QW, WAVES>;
  auto kern = attn_fwd_bf16<D, QW, WAVES, MINW>;
  const int64_t nb = (S + C::kQB - 1) / C::kQB;
  FwdSplit sp{};
  sp.o = sb ? sb->o : nullptr;
  sp.lam = sb ? sb->lam : nullptr;
  const int64_t b0 = sb ? plan_split(S, nb, C::kQB, BH, resident_slots(kern, C::kThreads), sp) : nb;
  const bool pr = sp.n == 0 && LH_PAIR_FWD && pair_blocks(nb, BH);
  const int64_t grid = sp.n > 0 ? sp.n * BH : causal_grid(nb, BH, pr);
  kern<<<dim3((unsigned)grid), C::kThreads, 0, st>>>(Q, K, V, o, lse, (int)S, sl2, pr ? 1 : 0, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.n == 0) return e;
  const int64_t r0 = b0 * C::kQB;  // first row of the split blocks
  constexpr int kRows = 256 / (D / 4);
  attn_fwd_merge<D><<<dim3((unsigned)((S - r0 + kRows - 1) / kRows), (unsigned)BH), 256, 0, st>>>(
      o, lse, sp.o, sp.lam, (int)S, (int)r0);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int64_t S, int d, int dtype, int64_t BH, hipStream_t st,
                           const FwdSplitBufs* split) {
  if (S == 0) return hipSuccess;
  if (dtype == 0)
    return launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                               static_cast<const float*>(v), o, lse, S, d, BH, st);
  const float sl2 = kLog2e / sqrtf((float)d);
  const auto Q = static_cast<const __bf16*>(q);
  const auto K = static_cast<const __bf16*>(k);
  const auto V = static_cast<const __bf16*>(v);
  if (d == 64)
    return fwd_bf16<64, LH_FWD64_QW, LH_FWD64_WAVES, LH_FWD64_MINW>(Q, K, V, o, lse, S, BH, sl2,
                                                                     split, st);
  return fwd_bf16<128, LH_FWD128_QW, LH_FWD128_WAVES, LH_FWD128_MINW>(Q, K, V, o, lse, S, BH, sl2,
                                                                       split, st);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* delta, float* lse2, int64_t S, int d, int dtype, int64_t BH,
                           hipStream_t st, hipEvent_t* ev, hipEvent_t dq_done) {
  if (S == 0) return dq_done ? hipEventRecord(dq_done, st) : hipSuccess;
  const int64_t rows = S * BH;
  const int rgs = 256 / (d / 8);
  const unsigned dgrid = (unsigned)((rows + rgs - 1) / rgs);
  // float32: rowsum kernel, key-block pass, query-block pass.  bf16: the
  // query-block pass forms the rowsum and lse*log2(e) and runs first.  ev[0],
  // ev[1], ev[2] mark the ends of the rowsum, dK/dV and dQ stages (for bf16
  // recorded in the order ev[0], ev[2], ev[1]; the rowsum stage is empty).
  const bool f32 = dtype == 0;
  if (f32)
    attn_delta_f32<<<dgrid, 256, 0, st>>>(o, static_cast<const float*>(dout), delta, rows, d);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[0], st);
  if (e != hipSuccess) return e;
  if (f32) {
    e = launch_attn_bwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                            static_cast<const float*>(v), lse, delta,
                            static_cast<const float*>(dout), dq, dk, dv, S, d, BH, st, ev);
    if (e == hipSuccess && dq_done) e = hipEventRecord(dq_done, st);  // dQ is the last pass
    return e;
  }
  const float scale = 1.0f / sqrtf((float)d);
  const float sl2 = kLog2e * scale;
  const auto Q = static_cast<const __bf16*>(q);
  const auto K = static_cast<const __bf16*>(k);
  const auto V = static_cast<const __bf16*>(v);
  const auto G = static_cast<const __bf16*>(dout);
  if (d == 64) {
    using C2 = BwdQCfg<64, LH_BQ64_WAVES>;
    const int64_t nb = (S + C2::kQB - 1) / C2::kQB;
    const bool pr = LH_PAIR_BQ && pair_blocks(nb, BH);
    attn_bwd_dq_bf16<64, LH_BQ64_WAVES, LH_BQ64_MINW>
        <<<dim3((unsigned)causal_grid(nb, BH, pr)), 64 * LH_BQ64_WAVES, 0, st>>>(
            Q, K, V, G, o, lse, lse2, delta, dq, (int)S, sl2, scale, pr ? 1 : 0);
  } else {
    using C2 = BwdQCfg<128, LH_BQ128_WAVES>;
    const int64_t nb = (S + C2::kQB - 1) / C2::kQB;
    const bool pr = LH_PAIR_BQ && pair_blocks(nb, BH);
    attn_bwd_dq_bf16<128, LH_BQ128_WAVES, LH_BQ128_MINW>
        <<<dim3((unsigned)causal_grid(nb, BH, pr)), 64 * LH_BQ128_WAVES, 0, st>>>(
            Q, K, V, G, o, lse, lse2, delta, dq, (int)S, sl2, scale, pr ? 1 : 0);
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], st);
  if (e == hipSuccess && dq_done) e = hipEventRecord(dq_done, st);
  if (e != hipSuccess) return e;
  if (d == 64) {
    auto dkdv64 = [&](auto waves) {
      constexpr int W = decltype(waves)::value;
      using C1 = BwdKVCfg<64, W>;
      const int64_t nb = (S + C1::kKB - 1) / C1::kKB;
      const bool pr = LH_PAIR_BKV64 && pair_blocks(nb, BH);
      attn_bwd_dkdv_bf16<64, W, LH_BKV64_MINW>
          <<<dim3((unsigned)causal_grid(nb, BH, pr)), 64 * W, 0, st>>>(
              Q, K, V, G, lse2, delta, dk, dv, (int)S, sl2, scale, pr ? 1 : 0);
    };
    const int64_t wide_kb = BwdKVCfg<64, LH_BKV64_WIDE>::kKB;
    if ((S + wide_kb - 1) / wide_kb * BH >= LH_BKV64_WIDE_MIN)
      dkdv64(std::integral_constant<int, LH_BKV64_WIDE>{});
    else
      dkdv64(std::integral_constant<int, LH_BKV64_WAVES>{});
  } else {
    using C1 = BwdKVCfg<128, LH_BKV128_WAVES>;
    const int64_t nb = (S + C1::kKB - 1) / C1::kKB;
    const bool pr = LH_PAIR_BKV128 && pair_blocks(nb, BH);
    attn_bwd_dkdv_bf16<128, LH_BKV128_WAVES, LH_BKV128_MINW>
        <<<dim3((unsigned)causal_grid(nb, BH, pr)), 64 * LH_BKV128_WAVES, 0, st>>>(
            Q, K, V, G, lse2, delta, dk, dv, (int)S, sl2, scale, pr ? 1 : 0);
  }
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[1], st);
  return e;
}

}  // namespace lh

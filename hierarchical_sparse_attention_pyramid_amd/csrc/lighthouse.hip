// C ABI of the Lighthouse library: host-side validation, buffer sizing and
// the launch sequences of the forward and backward passes.  See
// include/lighthouse.h for the contract of every entry point.
#include "lighthouse.h"

#include <algorithm>
#include <mutex>
#include <string>

#include "kernels.h"

// Scratch of lh_topk_noalloc: the top-K workspace in a fixed device array, so
// that the call allocates nothing.  Each device holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint32_t scratch[kNoAllocScratchBytes / sizeof(uint32_t)];

namespace {

thread_local std::string g_err;

lh_status fail(lh_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

lh_status hip_fail(hipError_t e, const char* where) {
  return fail(LH_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Stage {
  int lvl0, lam, chunk;
  int xl;  // token pass: levels above lvl0 + lam formed in the workgroup through LDS
  int64_t rows_in, rows_out;      // forward pooling: rows per head
  int64_t brows_in, brows_out;    // scatter backward: virtual rows per head
  int out_buf;  // 0 = A, 1 = B, -1 = no f32 sums written
};

struct Plan {
  lh::Geo g;
  lh::Lay tin, tout;  // token tensors: q, k, v, dq, dk, dv / out, dout
  int64_t B, H, BH;
  int dtype;
  int sh;  // scatter reading: 0 span, 1 causal (virtual token u = t + 1)
  size_t es;
  lh_sizes sz;
  int nstages;
  Stage st[lh::kMaxLevels];
  size_t sums_rows[2];  // rows per head of the A / B f32 sum buffers
};

#ifndef LH_POOL_TOKCHUNK
#define LH_POOL_TOKCHUNK 64
#endif
// A pooling workgroup covers at most 32 row groups x 64 rows; the backward
// pooling kernel stages those rows' positions and their ancestors' (at most
// as many again for p >= 2, plus one per level) in a fixed LDS cache sized
// for that bound.
static_assert(LH_POOL_TOKCHUNK <= 64, "token chunks above 64 rows overflow the position cache");

// token-pass row groups below which the chunks shrink: 32 per compute unit
constexpr int64_t kPoolRowGroupsWanted = 256 * 32;

int lam_max(int p) {
  int lam = 1;
  int64_t pw = p;
  while (lam < lh::kStageLevels && pw * p <= LH_POOL_TOKCHUNK) {
    pw *= p;
    ++lam;
  }
  return lam;
}

// Layout of the token tensors from optional element strides (all zero: the
// packed [B,H,N,d] layout).  Rows must start on 16-byte boundaries and no two
// elements of different (b, h, n) may share an address; the stride of a
// dimension of extent 1 is ignored.
lh_status token_layout(const lh_shape* s, const int64_t (&st)[3], const char* what,
                       lh::Lay& out) {
  if (st[0] == 0 && st[1] == 0 && st[2] == 0) {
    out = lh::packed_lay(s->H, s->N, s->d);
    return LH_OK;
  }
  const int64_t es = s->dtype == LH_BF16 ? 2 : 4;
  const int64_t ext[3] = {s->B, s->H, s->N};
  int order[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i) {
    if (ext[i] == 1) continue;  // index always 0: the stride is never used
    if (st[i] < 1 || st[i] > (int64_t(1) << 40))
      return fail(LH_EINVAL, std::string(what) + " strides must be positive (or all zero)");
    if ((st[i] * es) % 16)
      return fail(LH_EINVAL, std::string(what) + " strides must be multiples of 16 bytes");
  }
  std::sort(order, order + 3, [&](int a, int b) { return st[a] < st[b]; });
  int64_t span = s->d;  // elements covered by the smaller dimensions
  for (int k = 0; k < 3; ++k) {
    const int i = order[k];
    if (ext[i] == 1) continue;
    if (st[i] < span)
      return fail(LH_EINVAL, std::string(what) + " strides make rows overlap");
    span = st[i] * (ext[i] - 1) + span;
  }
  out = lh::Lay{ext[0] == 1 ? 0 : st[0], ext[1] == 1 ? 0 : st[1], ext[2] == 1 ? 0 : st[2],
                (int32_t)s->H};
  return LH_OK;
}

lh_status make_plan(const lh_shape* s, Plan& P) {
  g_err.clear();
  if (!s) return fail(LH_EINVAL, "shape is null");
  if (s->B < 1 || s->H < 1 || s->N < 1 || s->d < 1)
    return fail(LH_EINVAL, "B, H, N and d must be positive");
  if (s->dtype != LH_FP32 && s->dtype != LH_BF16) return fail(LH_EINVAL, "unknown dtype");
  if (s->scatter != LH_SCATTER_SPAN && s->scatter != LH_SCATTER_CAUSAL)
    return fail(LH_EINVAL, "unknown scatter reading");
  if (s->p < 2) return fail(LH_EINVAL, "pooling factor p must be >= 2");
  if (s->p > 64) return fail(LH_EUNSUPPORTED, "pooling factor p > 64 is not supported");
  if (s->L < 1) return fail(LH_EINVAL, "L must be >= 1");
  if (s->L > lh::kMaxLevels) return fail(LH_EUNSUPPORTED, "L > 16 levels is not supported");
  if (s->d != 64 && s->d != 128) return fail(LH_EUNSUPPORTED, "head dim must be 64 or 128");
  lh::Geo& g = P.g;
  int64_t pw = 1, M = 0;
  for (int l = 0; l < s->L; ++l) {
    if (l > 0) {
      if (pw > s->N / s->p) return fail(LH_EINVAL, "N must be divisible by p^(L-1)");
      pw *= s->p;
    }
    if (s->N % pw) return fail(LH_EINVAL, "N must be divisible by p^(L-1)");
    g.pw[l] = (int32_t)pw;
    g.inv_pw[l] = (float)(1.0 / (double)pw);
    g.nlev[l] = (int32_t)(s->N / pw);
    g.base[l] = (int32_t)M;
    M += s->N / pw;
  }
  for (int l = s->L; l < lh::kMaxLevels; ++l) {
    g.pw[l] = 0;
    g.inv_pw[l] = 0.f;
    g.nlev[l] = 0;
    g.base[l] = (int32_t)M;
  }
  const int64_t nc = s->N / pw;
  const int64_t BH = s->B * s->H;
  // 32-bit indexing: flat entries of all heads, and one head's M * d
  // elements (so that S * d * 2 bytes, a buffer-descriptor record count in
  // the attention kernels, stays below 2^32)
  if (BH * M >= (int64_t(1) << 31))
    return fail(LH_EUNSUPPORTED, "B*H*M must stay below 2^31");
  if (M * s->d >= (int64_t(1) << 31))
    return fail(LH_EUNSUPPORTED, "M*d must stay below 2^31");
  if (BH > 65535)  // the per-head kernels put B*H on the grid's y dimension
    return fail(LH_EUNSUPPORTED, "B*H above 65535 is not supported");
  if (s->S < nc || s->S > M)
    return fail(LH_EINVAL, "S must satisfy N/p^(L-1) <= S <= M (number of pyramid entries)");
  if (s->H >= (int64_t(1) << 31)) return fail(LH_EUNSUPPORTED, "H must stay below 2^31");
  lh_status ls;
  if ((ls = token_layout(s, s->qkv_stride, "qkv", P.tin)) != LH_OK) return ls;
  if ((ls = token_layout(s, s->out_stride, "out", P.tout)) != LH_OK) return ls;
  g.N = (int32_t)s->N;
  g.d = (int32_t)s->d;
  g.p = s->p;
  g.L = s->L;
  g.M = (int32_t)M;
  g.S = (int32_t)s->S;
  g.n_coarse = (int32_t)nc;
  g.C = (int32_t)(M - nc);
  g.K = (int32_t)(s->S - nc);
  g.log2p = -1;
  for (int b = 0; b < 31; ++b)
    if ((1 << b) == s->p) g.log2p = b;
  P.B = s->B;
  P.H = s->H;
  P.BH = BH;
  P.dtype = s->dtype;
  P.es = s->dtype == LH_BF16 ? 2 : 4;
  // with one level both readings feed token t from entry t alone: run the span form
  P.sh = s->scatter == LH_SCATTER_CAUSAL && s->L > 1 ? 1 : 0;
  // the causal scatter backward pools N + p^(L-1) virtual rows (see pyramid.hip)
  const int64_t nvb = s->N + (P.sh ? pw : 0);

  // pooling passes
  P.nstages = 0;
  P.sums_rows[0] = P.sums_rows[1] = 0;
  if (s->L == 1) {
    // scores only, no level to form: chunks shrink like the token passes'
    // below, down to one row
    int chunk = LH_POOL_TOKCHUNK;
    while (chunk > 1 && BH * (s->N / chunk) < kPoolRowGroupsWanted) chunk /= 2;
    P.st[P.nstages++] = Stage{0, 0, chunk, 0, s->N, s->N, nvb, nvb, -1};
  } else {
    const int lm = lam_max(s->p);
    int lvl = 0;
    while (lvl < s->L - 1) {
      const int lam = std::min(s->L - 1 - lvl, lm);
      int64_t plam = 1;
      for (int i = 0; i < lam; ++i) plam *= s->p;
      // token passes walk 64-row chunks, unless that leaves fewer than
      // about 32 row groups per compute unit (short sequences, few heads):
      // then shorter chunks, down to one span of the pass's top level, so
      // that more row groups share the rows; upper passes see p^lvl times
      // fewer rows and take one span per row group
      int64_t rep = lvl == 0 ? std::max<int64_t>(1, LH_POOL_TOKCHUNK / plam) : 1;
      while (rep > 1 && BH * (s->N / (plam * rep)) < kPoolRowGroupsWanted) rep /= 2;
      // The token pass's workgroup covers rgs * chunk consecutive rows; the
      // levels whose spans divide that (at most kPoolLdsLevels more, p >= 4,
      // with the top register level's float32 sums of the workgroup in at
      // most kPoolLdsFloats) are formed from those sums in LDS instead of by
      // a further pass.
      int xl = 0;
      if (lvl == 0 && s->p >= 4) {
        const int64_t span = (int64_t)(256 / (s->d / 8)) * plam * rep;
        int64_t pe = plam;
        if ((span / plam) * 3 * s->d <= lh::kPoolLdsFloats)
          while (xl < lh::kPoolLdsLevels && lvl + lam + xl < s->L - 1 && span % (pe * s->p) == 0) {
            pe *= s->p;
            ++xl;
          }
      }
      int64_t ptop = plam;
      for (int i = 0; i < xl; ++i) ptop *= s->p;
      const int64_t rows_in = s->N / g.pw[lvl];
      const int64_t brows_in = nvb / g.pw[lvl];
      Stage t{lvl, lam, (int)(plam * rep), xl, rows_in, rows_in / ptop, brows_in, brows_in / ptop, -1};
      P.st[P.nstages++] = t;
      lvl += lam + xl;
    }
    for (int k = 0; k + 1 < P.nstages; ++k) {
      P.st[k].out_buf = k % 2;
      P.sums_rows[k % 2] = std::max<size_t>(
          P.sums_rows[k % 2], (size_t)std::max(P.st[k].rows_out, P.st[k].brows_out));
    }
  }

  lh_sizes& z = P.sz;
  const size_t e = P.es, d = (size_t)s->d;
  z.M = M;
  z.C = M - nc;
  z.K = s->S - nc;
  z.n_coarse = nc;
  z.bytes_qkv = (size_t)BH * s->N * d * e;
  z.bytes_pyramid = (size_t)BH * (M - s->N) * d * e;
  z.bytes_score = (size_t)BH * M * 4;
  z.bytes_sel = (size_t)BH * z.K * 4;
  z.bytes_sub_idx = (size_t)BH * s->S * 4;
  z.bytes_pos = (size_t)BH * M * 4;
  z.bytes_sub = (size_t)BH * s->S * d * e;
  z.bytes_sub_f32 = (size_t)BH * s->S * d * 4;
  z.bytes_lse = (size_t)BH * s->S * 4;
  const size_t sums1 = align_up((size_t)BH * P.sums_rows[0] * d * 4) +
                       align_up((size_t)BH * P.sums_rows[1] * d * 4);
  z.ws_build_pyramid = 3 * sums1;
  z.ws_score = 0;
  z.ws_topk = z.K > 0 ? align_up(lh::topk_ws_bytes(BH, z.C)) : 0;
  z.ws_gather = 0;
  z.ws_attention_backward = 2 * align_up(z.bytes_lse);  // rowsum(dO*O), lse*log2(e)
  z.ws_scatter_backward = sums1;
  // the pooling pass clears the top-K histograms while it writes its float32
  // sums: the two regions must not overlap
  // after the top-K the region is reused by the attention's key-range split
  // (chunk-0 outputs and lambdas; bf16 only)
  const size_t split = s->dtype == LH_BF16 ? align_up(z.bytes_sub_f32) + align_up(z.bytes_lse) : 0;
  z.ws_forward = std::max(align_up(z.ws_build_pyramid) + z.ws_topk, split);
  z.ws_backward = align_up(z.bytes_sub) + 3 * align_up(z.bytes_sub_f32) + z.ws_attention_backward +
                  z.ws_scatter_backward;
  return LH_OK;
}

// f32 sum buffers A and B inside a workspace, for tensor t.
float* sums_ptr(const Plan& P, void* ws, int buf, int t) {
  const size_t d = (size_t)P.g.d;
  const size_t a = align_up((size_t)P.BH * P.sums_rows[0] * d * 4);
  const size_t b = align_up((size_t)P.BH * P.sums_rows[1] * d * 4);
  char* base = static_cast<char*>(ws) + (size_t)t * (a + b);
  return reinterpret_cast<float*>(buf == 0 ? base : base + a);
}

lh_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return LH_OK;
  if (!ws) return fail(LH_EINVAL, "workspace pointer is null");
  if (have < need)
    return fail(LH_EWORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  // its regions start at multiples of 256 bytes from ws and are read and
  // written in 16-byte vectors
  if (reinterpret_cast<uintptr_t>(ws) % 16) return fail(LH_EINVAL, "workspace must be 16-byte aligned");
  return LH_OK;
}

#define LH_NEED(ptr, name) \
  if (!(ptr)) return fail(LH_EINVAL, name " is null")

// Token tensors: non-null and 16-byte aligned (rows are moved in 16-byte
// vectors).
#define LH_TOK(ptr, name)                                                \
  if (!(ptr)) return fail(LH_EINVAL, name " is null");                   \
  if (reinterpret_cast<uintptr_t>(ptr) % 16)                             \
  return fail(LH_EINVAL, name " must be 16-byte aligned")

#define LH_HIP(call, where)                       \
  do {                                            \
    const hipError_t e_ = (call);                 \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

lh_status run_pool(const Plan& P, const void* q, const void* k, const void* v, void* pq, void* pk,
                   void* pv, float* score, void* ws, bool do_pool, bool do_score, hipStream_t st,
                   void* topk_ws = nullptr) {
  const void* lvl0[3] = {q, k, v};
  void* pyr[3] = {pq, pk, pv};
  for (int s = 0; s < P.nstages; ++s) {
    const Stage& t = P.st[s];
    if (t.lam == 0 && !do_score) continue;
    lh::PoolFwdArgs a{};
    for (int i = 0; i < 3; ++i) {
      if (s == 0) a.in[i] = lvl0[i];
      else a.in[i] = do_pool ? sums_ptr(P, ws, P.st[s - 1].out_buf, i) : nullptr;
      a.pyr[i] = do_pool ? pyr[i] : nullptr;
      a.sums_out[i] = (do_pool && t.out_buf >= 0) ? sums_ptr(P, ws, t.out_buf, i) : nullptr;
    }
    a.score = do_score ? score : nullptr;
    a.lin = s == 0 ? P.tin : lh::packed_lay(P.H, t.rows_in, P.g.d);
    a.in_rows = t.rows_in;
    a.out_rows = t.rows_out;
    a.lvl0 = t.lvl0;
    a.lam = t.lam;
    a.chunk = t.chunk;
    a.xl = t.xl;
    if (do_score && topk_ws != nullptr) {  // count the candidates for the top-K
      a.hist = static_cast<uint32_t*>(topk_ws);
      a.hist_stride = lh::topk_hist_stride(P.g.C);
    }
    a.g = P.g;
    LH_HIP(lh::launch_pool_fwd(a, P.dtype, P.BH, s == 0, do_pool, do_score, st), "pyramid");
  }
  return LH_OK;
}

}  // namespace

extern "C" {

const char* lh_last_error(void) { return g_err.c_str(); }

lh_status lh_query_sizes(const lh_shape* shape, lh_sizes* out) {
  Plan P;
  const lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  if (!out) return fail(LH_EINVAL, "sizes output is null");
  *out = P.sz;
  return LH_OK;
}

lh_status lh_build_pyramid(const lh_shape* shape, const void* q, const void* k, const void* v,
                           void* pq, void* pk, void* pv, void* ws, size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_TOK(q, "q");
  LH_TOK(k, "k");
  LH_TOK(v, "v");
  if (P.sz.bytes_pyramid) {
    LH_NEED(pq, "pq");
    LH_NEED(pk, "pk");
    LH_NEED(pv, "pv");
  }
  if ((s = check_ws(ws, ws_bytes, P.sz.ws_build_pyramid)) != LH_OK) return s;
  if (P.g.L == 1) return LH_OK;
  return run_pool(P, q, k, v, pq, pk, pv, nullptr, ws, true, false,
                  static_cast<hipStream_t>(stream));
}

lh_status lh_score(const lh_shape* shape, const void* q, const void* k, float* score, void* ws,
                   size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_TOK(q, "q");
  LH_TOK(k, "k");
  LH_NEED(score, "score");
  (void)ws;
  (void)ws_bytes;
  return run_pool(P, q, k, nullptr, nullptr, nullptr, nullptr, score, nullptr, false, true,
                  static_cast<hipStream_t>(stream));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for later calls.
static lh_status noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LH_EUNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    addr[dev] = p;
  }
  *out = addr[dev];
  return LH_OK;
}

lh_status lh_topk_noalloc(const lh_shape* shape, const float* score, int32_t* sel,
                          void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  if (P.g.K == 0) return LH_OK;
  LH_NEED(score, "score");
  LH_NEED(sel, "sel");
  if (P.sz.ws_topk > kNoAllocScratchBytes)
    return fail(LH_EWORKSPACE, "lh_topk_noalloc: the top-K needs " + std::to_string(P.sz.ws_topk) +
                                   " bytes of scratch, above its static " +
                                   std::to_string(kNoAllocScratchBytes) +
                                   " bytes; use lh_topk with a workspace");
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != LH_OK) return s;
  // the top-K clears its histograms in a kernel of its own, so what an
  // earlier call left in the array does not matter
  LH_HIP(lh::launch_topk(score, sel, ws, P.g, P.BH, false, static_cast<hipStream_t>(stream)), "topk");
  return LH_OK;
}

lh_status lh_topk(const lh_shape* shape, const float* score, int32_t* sel, void* ws,
                  size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  if (P.g.K == 0) return LH_OK;
  LH_NEED(score, "score");
  LH_NEED(sel, "sel");
  if ((s = check_ws(ws, ws_bytes, P.sz.ws_topk)) != LH_OK) return s;
  LH_HIP(lh::launch_topk(score, sel, ws, P.g, P.BH, false, static_cast<hipStream_t>(stream)), "topk");
  return LH_OK;
}

lh_status lh_gather(const lh_shape* shape, const int32_t* sel, const void* q, const void* k,
                    const void* v, const void* pq, const void* pk, const void* pv,
                    int32_t* sub_idx, int32_t* pos, void* qs, void* ks, void* vs, void* ws,
                    size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  (void)ws;
  (void)ws_bytes;
  if (P.g.K > 0) LH_NEED(sel, "sel");
  LH_TOK(q, "q");
  LH_TOK(k, "k");
  LH_TOK(v, "v");
  if (P.sz.bytes_pyramid) {
    LH_NEED(pq, "pq");
    LH_NEED(pk, "pk");
    LH_NEED(pv, "pv");
  }
  LH_NEED(sub_idx, "sub_idx");
  LH_NEED(pos, "pos");
  LH_NEED(qs, "qs");
  LH_NEED(ks, "ks");
  LH_NEED(vs, "vs");
  const void* lv0[3] = {q, k, v};
  const void* pyr[3] = {pq, pk, pv};
  void* sub[3] = {qs, ks, vs};
  LH_HIP(lh::launch_gather(sel, lv0, P.tin, pyr, sub_idx, pos, sub, P.g, P.dtype, P.BH,
                           static_cast<hipStream_t>(stream)),
         "gather");
  return LH_OK;
}

lh_status lh_attention(const lh_shape* shape, const void* qs, const void* ks, const void* vs,
                       float* os, float* lse, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_NEED(qs, "qs");
  LH_NEED(ks, "ks");
  LH_NEED(vs, "vs");
  LH_NEED(os, "os");
  LH_NEED(lse, "lse");
  LH_HIP(lh::launch_attn_fwd(qs, ks, vs, os, lse, P.g.S, P.g.d, P.dtype, P.BH,
                             static_cast<hipStream_t>(stream)),
         "attention");
  return LH_OK;
}

lh_status lh_scatter(const lh_shape* shape, const float* os, const int32_t* pos, void* out,
                     void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_NEED(os, "os");
  LH_NEED(pos, "pos");
  LH_TOK(out, "out");
  lh::BcastArgs a{};
  a.src[0] = os;
  a.out[0] = out;
  a.pos = pos;
  a.mean = 1;
  a.shift = P.sh;
  a.lout = P.tout;
  a.g = P.g;
  LH_HIP(lh::launch_bcast(a, P.dtype, 1, P.BH, static_cast<hipStream_t>(stream)),
         "scatter");
  return LH_OK;
}

static lh_status check_forward_args(const Plan& P, const void* q, const void* k, const void* v,
                                    void* out, const lh_buffers* b) {
  LH_NEED(b, "buffers");
  LH_TOK(q, "q");
  LH_TOK(k, "k");
  LH_TOK(v, "v");
  LH_TOK(out, "out");
  if (P.sz.bytes_pyramid) {
    LH_NEED(b->pq, "buffers.pq");
    LH_NEED(b->pk, "buffers.pk");
    LH_NEED(b->pv, "buffers.pv");
  }
  LH_NEED(b->score, "buffers.score");
  if (P.g.K > 0) LH_NEED(b->sel, "buffers.sel");
  LH_NEED(b->sub_idx, "buffers.sub_idx");
  LH_NEED(b->pos, "buffers.pos");
  LH_NEED(b->qs, "buffers.qs");
  LH_NEED(b->ks, "buffers.ks");
  LH_NEED(b->vs, "buffers.vs");
  LH_NEED(b->os, "buffers.os");
  LH_NEED(b->lse, "buffers.lse");
  return LH_OK;
}

// Forward launch sequence; when `ev` is given, ev[i] is recorded after stage i
// (pyramid+score, top-K, gather, attention, scatter).
static lh_status run_forward(const Plan& P, const void* q, const void* k, const void* v, void* out,
                             const lh_buffers* b, void* ws, hipStream_t st, hipEvent_t* ev) {
  lh_status s;
  // The top-K region follows the pooling sums.  For heads above the
  // small-path size its pass-0 histograms are cleared first and the pooling
  // kernels count the candidate scores into them as they write them.
  const bool counted = P.g.K > 0 && !lh::topk_small_path(P.g.C);
  void* tws = counted ? static_cast<char*>(ws) + align_up(P.sz.ws_build_pyramid) : nullptr;
  if (counted) LH_HIP(lh::launch_topk_zero(tws, P.g.C, P.BH, st), "topk");
  if ((s = run_pool(P, q, k, v, b->pq, b->pk, b->pv, b->score, ws, P.g.L > 1, true, st, tws)) !=
      LH_OK)
    return s;
  if (ev) LH_HIP(hipEventRecord(ev[0], st), "event");
  LH_HIP(lh::launch_topk(b->score, b->sel, tws, P.g, P.BH, counted, st), "topk");
  if (ev) LH_HIP(hipEventRecord(ev[1], st), "event");
  const void* lv0[3] = {q, k, v};
  const void* pyr[3] = {b->pq, b->pk, b->pv};
  void* sub[3] = {b->qs, b->ks, b->vs};
  LH_HIP(lh::launch_gather(b->sel, lv0, P.tin, pyr, b->sub_idx, b->pos, sub, P.g, P.dtype, P.BH, st),
         "gather");
  if (ev) LH_HIP(hipEventRecord(ev[2], st), "event");
  // the attention's split buffers: the start of ws, free once the top-K is done
  lh::FwdSplitBufs sb{static_cast<float*>(ws),
                      reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(P.sz.bytes_sub_f32))};
  LH_HIP(lh::launch_attn_fwd(b->qs, b->ks, b->vs, b->os, b->lse, P.g.S, P.g.d, P.dtype, P.BH, st,
                             P.dtype == LH_BF16 ? &sb : nullptr),
         "attention");
  if (ev) LH_HIP(hipEventRecord(ev[3], st), "event");
  lh::BcastArgs a{};
  a.src[0] = b->os;
  a.out[0] = out;
  a.pos = b->pos;
  a.mean = 1;
  a.shift = P.sh;
  a.lout = P.tout;
  a.g = P.g;
  LH_HIP(lh::launch_bcast(a, P.dtype, 1, P.BH, st), "scatter");
  if (ev) LH_HIP(hipEventRecord(ev[4], st), "event");
  return LH_OK;
}

lh_status lh_forward(const lh_shape* shape, const void* q, const void* k, const void* v,
                     void* out, const lh_buffers* b, void* ws, size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  if ((s = check_forward_args(P, q, k, v, out, b)) != LH_OK) return s;
  if ((s = check_ws(ws, ws_bytes, P.sz.ws_forward)) != LH_OK) return s;
  return run_forward(P, q, k, v, out, b, ws, static_cast<hipStream_t>(stream), nullptr);
}

static lh_status run_scatter_bwd(const Plan& P, const void* dout, const int32_t* pos, void* dos,
                                 void* ws, hipStream_t st) {
  for (int s = 0; s < P.nstages; ++s) {
    const Stage& t = P.st[s];
    lh::PoolBwdArgs a{};
    a.in = s == 0 ? dout : static_cast<const void*>(sums_ptr(P, ws, P.st[s - 1].out_buf, 0));
    a.dos = dos;
    a.sums_out = t.out_buf >= 0 ? sums_ptr(P, ws, t.out_buf, 0) : nullptr;
    a.pos = pos;
    a.lin = s == 0 ? P.tout : lh::packed_lay(P.H, t.brows_in, P.g.d);
    a.in_rows = t.brows_in;
    a.out_rows = t.brows_out;
    a.lvl0 = t.lvl0;
    a.lam = t.lam;
    a.chunk = t.chunk;
    a.xl = t.xl;
    a.shift = P.sh;
    a.g = P.g;
    LH_HIP(lh::launch_pool_bwd(a, P.dtype, P.BH, s == 0, st), "scatter_backward");
  }
  return LH_OK;
}

lh_status lh_scatter_backward(const lh_shape* shape, const void* dout, const int32_t* pos,
                              void* dos, void* ws, size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_TOK(dout, "dout");
  LH_NEED(pos, "pos");
  LH_NEED(dos, "dos");
  if ((s = check_ws(ws, ws_bytes, P.sz.ws_scatter_backward)) != LH_OK) return s;
  return run_scatter_bwd(P, dout, pos, dos, ws, static_cast<hipStream_t>(stream));
}

lh_status lh_attention_backward(const lh_shape* shape, const void* qs, const void* ks,
                                const void* vs, const float* os, const float* lse, const void* dos,
                                float* dqs, float* dks, float* dvs, void* ws, size_t ws_bytes,
                                void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_NEED(qs, "qs");
  LH_NEED(ks, "ks");
  LH_NEED(vs, "vs");
  LH_NEED(os, "os");
  LH_NEED(lse, "lse");
  LH_NEED(dos, "dos");
  LH_NEED(dqs, "dqs");
  LH_NEED(dks, "dks");
  LH_NEED(dvs, "dvs");
  if ((s = check_ws(ws, ws_bytes, P.sz.ws_attention_backward)) != LH_OK) return s;
  float* delta = static_cast<float*>(ws);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(P.sz.bytes_lse));
  LH_HIP(lh::launch_attn_bwd(qs, ks, vs, os, lse, dos, dqs, dks, dvs, delta, lse2, P.g.S, P.g.d,
                             P.dtype, P.BH, static_cast<hipStream_t>(stream), nullptr),
         "attention_backward");
  return LH_OK;
}

lh_status lh_gather_backward(const lh_shape* shape, const float* dqs, const float* dks,
                             const float* dvs, const int32_t* pos, void* dq, void* dk, void* dv,
                             void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_NEED(dqs, "dqs");
  LH_NEED(dks, "dks");
  LH_NEED(dvs, "dvs");
  LH_NEED(pos, "pos");
  LH_TOK(dq, "dq");
  LH_TOK(dk, "dk");
  LH_TOK(dv, "dv");
  lh::BcastArgs a{};
  a.src[0] = dqs;
  a.src[1] = dks;
  a.src[2] = dvs;
  a.out[0] = dq;
  a.out[1] = dk;
  a.out[2] = dv;
  a.pos = pos;
  a.mean = 0;
  a.shift = 0;  // the pooling adjoint: spans, in either scatter reading
  a.lout = P.tin;
  a.g = P.g;
  LH_HIP(lh::launch_bcast(a, P.dtype, 3, P.BH, static_cast<hipStream_t>(stream)),
         "gather_backward");
  return LH_OK;
}

static lh_status check_backward_args(const void* dout, const lh_buffers* b, void* dq, void* dk,
                                     void* dv) {
  LH_NEED(b, "buffers");
  LH_TOK(dout, "dout");
  LH_NEED(b->pos, "buffers.pos");
  LH_NEED(b->qs, "buffers.qs");
  LH_NEED(b->ks, "buffers.ks");
  LH_NEED(b->vs, "buffers.vs");
  LH_NEED(b->os, "buffers.os");
  LH_NEED(b->lse, "buffers.lse");
  LH_TOK(dq, "dq");
  LH_TOK(dk, "dk");
  LH_TOK(dv, "dv");
  return LH_OK;
}

#ifndef LH_BWD_FORK
#define LH_BWD_FORK 1
#endif

// The side stream of lh_backward on one device, with the events of its fork
// and join: one set per host thread and device, made on first use and kept
// until the process ends (so no two threads share one, and a thread's calls
// are ordered on it as on their own streams).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

// The calling thread's side stream for the device of `st`, or null when the
// backward should run on `st` alone: `st` belongs to another device than the
// current one; the side stream does not exist yet and `st` is being captured
// into a graph (it is made only outside captures, where making it cannot
// disturb one: a capture thus forks only after an eager call on the thread);
// the side stream is part of a graph capture that `st` is not (one still
// open from an earlier call); or a HIP call fails (the sequential path then
// reports any real error itself).
static SideStream* side_stream(hipStream_t st) {
  constexpr int kMaxDevices = 64;
  thread_local SideStream side[kMaxDevices];
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (hipStreamGetDevice(st, &sdev) != hipSuccess || sdev != dev) return nullptr;
  hipStreamCaptureStatus cm = hipStreamCaptureStatusNone;
  unsigned long long im = 0;
  if (hipStreamGetCaptureInfo(st, &cm, &im) != hipSuccess) return nullptr;
  SideStream& sd = side[dev];
  if (!sd.s) {
    if (cm != hipStreamCaptureStatusNone) return nullptr;
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (f) (void)hipEventDestroy(f);
      (void)hipStreamDestroy(s);
      return nullptr;
    }
    sd.s = s;
    sd.fork = f;
    sd.join = j;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long is = 0;
  if (hipStreamGetCaptureInfo(sd.s, &cs, &is) != hipSuccess) return nullptr;
  if (cs != hipStreamCaptureStatusNone && (cm != hipStreamCaptureStatusActive || im != is))
    return nullptr;
  if (cm != hipStreamCaptureStatusNone && cm != hipStreamCaptureStatusActive) return nullptr;
  return &sd;
}

// Backward launch sequence; when `ev` is given, ev[i] is recorded after stage
// i (scatter backward, delta, dK/dV pass, dQ pass, gather backward), in the
// order the stages run (bf16: the dQ pass, which forms delta, before dK/dV).
// Without `ev`, with bf16 storage and d = 64, the gather backward of dq runs
// on a side stream beside the dK/dV pass (it needs only the dQ pass, which
// runs first): the broadcast is bound by HBM and the key-block pass by the
// matrix cores, and at d = 64 a compute unit has room for both, so they
// overlap (the 98K step 1% faster); `st` waits for the side stream at the
// end.  At d = 128 the key-block pass fills the compute units' registers,
// the broadcast could only follow it, and the fork measured 0.7% slower.
static lh_status run_backward(const Plan& P, const void* dout, const lh_buffers* b, void* dq,
                              void* dk, void* dv, void* ws, hipStream_t st, hipEvent_t* ev) {
  char* w = static_cast<char*>(ws);
  void* dos = w;
  w += align_up(P.sz.bytes_sub);
  float* dqs = reinterpret_cast<float*>(w);
  w += align_up(P.sz.bytes_sub_f32);
  float* dks = reinterpret_cast<float*>(w);
  w += align_up(P.sz.bytes_sub_f32);
  float* dvs = reinterpret_cast<float*>(w);
  w += align_up(P.sz.bytes_sub_f32);
  float* delta = reinterpret_cast<float*>(w);
  float* lse2 = reinterpret_cast<float*>(w + align_up(P.sz.bytes_lse));
  w += P.sz.ws_attention_backward;
  lh_status s;
  if ((s = run_scatter_bwd(P, dout, b->pos, dos, w, st)) != LH_OK) return s;
  if (ev) LH_HIP(hipEventRecord(ev[0], st), "event");
  SideStream* side =
      LH_BWD_FORK && !ev && P.dtype == 1 && P.g.d == 64 && P.g.S > 0 ? side_stream(st) : nullptr;
  LH_HIP(lh::launch_attn_bwd(b->qs, b->ks, b->vs, b->os, b->lse, dos, dqs, dks, dvs, delta, lse2,
                             P.g.S, P.g.d, P.dtype, P.BH, st, ev ? ev + 1 : nullptr,
                             side ? side->fork : nullptr),
         "attention_backward");
  lh::BcastArgs a{};
  a.src[0] = dqs;
  a.src[1] = dks;
  a.src[2] = dvs;
  a.out[0] = dq;
  a.out[1] = dk;
  a.out[2] = dv;
  a.pos = b->pos;
  a.mean = 0;
  a.shift = 0;  // the pooling adjoint: spans, in either scatter reading
  a.lout = P.tin;
  a.g = P.g;
  if (side) {
    // dq on the side stream once the dQ pass is done; dk, dv here after the
    // key-block pass; then `st` waits for the side stream
    lh::BcastArgs aq = a, akv = a;
    akv.src[0] = dks;
    akv.src[1] = dvs;
    akv.out[0] = dk;
    akv.out[1] = dv;
    LH_HIP(hipStreamWaitEvent(side->s, side->fork, 0), "hipStreamWaitEvent");
    LH_HIP(lh::launch_bcast(aq, P.dtype, 1, P.BH, side->s), "gather_backward");
    LH_HIP(hipEventRecord(side->join, side->s), "hipEventRecord");
    LH_HIP(lh::launch_bcast(akv, P.dtype, 2, P.BH, st), "gather_backward");
    LH_HIP(hipStreamWaitEvent(st, side->join, 0), "hipStreamWaitEvent");
    return LH_OK;
  }
  LH_HIP(lh::launch_bcast(a, P.dtype, 3, P.BH, st), "gather_backward");
  if (ev) LH_HIP(hipEventRecord(ev[4], st), "event");
  return LH_OK;
}

lh_status lh_backward(const lh_shape* shape, const void* dout, const lh_buffers* b, void* dq,
                      void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  if ((s = check_backward_args(dout, b, dq, dk, dv)) != LH_OK) return s;
  if ((s = check_ws(ws, ws_bytes, P.sz.ws_backward)) != LH_OK) return s;
  return run_backward(P, dout, b, dq, dk, dv, ws, static_cast<hipStream_t>(stream), nullptr);
}

lh_status lh_profile_step(const lh_shape* shape, const void* q, const void* k, const void* v,
                          void* out, const lh_buffers* b, const void* dout, void* dq, void* dk,
                          void* dv, void* ws, size_t ws_bytes, float* ms, void* stream) {
  Plan P;
  lh_status s = make_plan(shape, P);
  if (s != LH_OK) return s;
  LH_NEED(ms, "ms");
  if ((s = check_forward_args(P, q, k, v, out, b)) != LH_OK) return s;
  if ((s = check_backward_args(dout, b, dq, dk, dv)) != LH_OK) return s;
  if ((s = check_ws(ws, ws_bytes, std::max(P.sz.ws_forward, P.sz.ws_backward))) != LH_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t ev[LH_PROFILE_STAGES + 1];
  int made = 0;
  for (; made <= LH_PROFILE_STAGES; ++made) {
    const hipError_t e = hipEventCreate(&ev[made]);
    if (e != hipSuccess) {
      for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
      return hip_fail(e, "hipEventCreate");
    }
  }
  hipError_t e = hipEventRecord(ev[0], st);
  if (e == hipSuccess) s = run_forward(P, q, k, v, out, b, ws, st, ev + 1);
  if (e == hipSuccess && s == LH_OK) s = run_backward(P, dout, b, dq, dk, dv, ws, st, ev + 6);
  // ev[i + 1] marks the end of stage i; stages run in index order except
  // that with bf16 storage the dQ pass (8) runs before the dK/dV pass (7)
  int order[LH_PROFILE_STAGES];
  for (int i = 0; i < LH_PROFILE_STAGES; ++i) order[i] = i;
  if (P.dtype == 1) {
    order[7] = 8;
    order[8] = 7;
  }
  if (e == hipSuccess && s == LH_OK) e = hipEventSynchronize(ev[order[LH_PROFILE_STAGES - 1] + 1]);
  for (int i = 0; e == hipSuccess && s == LH_OK && i < LH_PROFILE_STAGES; ++i) {
    const hipEvent_t start = i == 0 ? ev[0] : ev[order[i - 1] + 1];
    e = hipEventElapsedTime(&ms[order[i]], start, ev[order[i] + 1]);
  }
  for (int i = 0; i <= LH_PROFILE_STAGES; ++i) (void)hipEventDestroy(ev[i]);
  if (e != hipSuccess) return hip_fail(e, "profile");
  return s;
}

}  // extern "C"

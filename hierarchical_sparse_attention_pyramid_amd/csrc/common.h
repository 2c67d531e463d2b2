// Shared device-side helpers of the Lighthouse HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

constexpr int kMaxLevels = 16;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// Pyramid geometry of one head, passed by value to kernels.
struct Geo {
  int32_t N, d, p, L;
  int32_t M, S, K, n_coarse, C;
  int32_t log2p;                 // log2(p) when p is a power of two, else -1
  int32_t base[kMaxLevels];      // flat index of the first entry of level l
  int32_t pw[kMaxLevels];        // p^l
  int32_t nlev[kMaxLevels];      // N / p^l
  float inv_pw[kMaxLevels];      // 1 / p^l rounded to float (exact when p is a power of two)
};

// Element strides of a [B, H, rows, d] tensor whose rows are d contiguous
// elements: row r of head bh = b*H + h starts at element b*sb + h*sh + r*sn.
struct Lay {
  int64_t sb, sh, sn;
  int32_t H;
  __host__ __device__ __forceinline__ int64_t head(int64_t bh) const {
    const int64_t b = bh / H;
    return b * sb + (bh - b * H) * sh;
  }
};

// The packed layout [B][H][rows][d].
__host__ __device__ inline Lay packed_lay(int64_t H, int64_t rows, int64_t d) {
  return Lay{H * rows * d, rows * d, d, (int32_t)H};
}

__device__ __forceinline__ int32_t div_pw(int32_t t, const Geo& g, int l) {
  return g.log2p >= 0 ? (t >> (g.log2p * l)) : t / g.pw[l];
}

// Vector loads and stores; the streaming forms (NT = true) mark data that is
// touched once, so that it does not displace reused lines in the caches.
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st(V* p, const V& v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---- 8-element row slices (16 bytes of bf16, 32 bytes of fp32) ----------
template <typename T> struct Row8;

template <> struct Row8<float> {
  template <bool NT = false>
  static __device__ __forceinline__ void load(const float* p, float (&x)[8]) {
    const f32x4 a = ld<NT>(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = ld<NT>(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[e + 4] = b[e]; }
  }
  template <bool NT = false>
  static __device__ __forceinline__ void store(float* p, const float (&x)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[e + 4]; }
    st<NT>(reinterpret_cast<f32x4*>(p), a);
    st<NT>(reinterpret_cast<f32x4*>(p) + 1, b);
  }
};

template <> struct Row8<__bf16> {
  template <bool NT = false>
  static __device__ __forceinline__ void load(const __bf16* p, float (&x)[8]) {
    const bf16x8 v = ld<NT>(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
  }
  // float -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  template <bool NT = false>
  static __device__ __forceinline__ void store(__bf16* p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(x[e]);
    st<NT>(reinterpret_cast<bf16x8*>(p), v);
  }
};

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

}  // namespace lh

// Device-side helpers shared by the FLCE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Element traits: every K step moves 128 bytes of K per operand row, i.e. 8
// chunks of 16 bytes; a chunk holds 8 bf16 or 4 fp32.
template <typename T> struct Elem;
template <> struct Elem<bf16> { static constexpr int size = 2; static constexpr int per_chunk = 8; };
template <> struct Elem<float> { static constexpr int size = 4; static constexpr int per_chunk = 4; };

__device__ __forceinline__ float fast_exp(float x) {
  // e^x = 2^(x log2 e) on the hardware exp2 (v_exp_f32); exp(-inf) = 0.
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

// Logit softcap z = T tanh(m a / T) (Muse Glimmer page, Details > Softcap),
// written from the mathematics on the raw accumulator a:
//  * |m a / T| < 1/4: the odd Maclaurin series of tanh, x - x^3/3 + 2x^5/15
//    - 17x^7/315 + 62x^9/2835 (the first omitted term, 1382x^11/155925, is
//    below 1e-8 relative there), with the powers of s = m / T and the factor
//    T s = m folded into its coefficients:
//      z = a (m + u Q(u)),  u = a^2,  Q(u) = q1 + u (q2 + u (q3 + u q4)),
//      q_j = m c_j s^(2j)  (c_j = -1/3, 2/15, -17/315, 62/2835),
//    seven operations per value;
//  * otherwise tanh|x| = 1 - 2 / (e^{2|x|} + 1) with the sign restored, which
//    saturates to 1 as e^{2|x|} overflows.
// Without a cap, z = m a.  When |s| exceeds 2^12 the folded coefficients
// would overflow (s^8 near |s| = 2^16), so the series is evaluated unfolded on
// x = s a instead, with the same range switch.  tests/test_softcap_host.py checks these functions on
// the host against float64 tanh; the GPU softcap test checks the kernels'
// logits (hardware exp2 and reciprocal) the same way.
__host__ __device__ __forceinline__ float tanh_exp_form(float x) {
  const float ax = __builtin_fabsf(x);
#if defined(__HIP_DEVICE_COMPILE__)
  const float e = __builtin_amdgcn_exp2f(2.0f * kLog2e * ax);
  const float r = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
#else
  const float e = __builtin_exp2f(2.0f * kLog2e * ax);
  const float r = 1.0f - 2.0f / (e + 1.0f);
#endif
  return __builtin_copysignf(r, x);
}
constexpr float kTanhSeriesMax = 0.25f;
constexpr float kSeriesScaleMax = 4096.0f;

// The series on x itself: x + x^3 P(x^2).
__host__ __device__ __forceinline__ float tanh_series(float x) {
  const float x2 = x * x;
  float p = __builtin_fmaf(62.0f / 2835.0f, x2, -17.0f / 315.0f);
  p = __builtin_fmaf(p, x2, 2.0f / 15.0f);
  p = __builtin_fmaf(p, x2, -1.0f / 3.0f);
  return __builtin_fmaf(x, p * x2, x);
}

struct CapSeries {
  float m, s, T, amax, q1, q2, q3, q4;
  bool unfolded;   // |s| > 2^12: the series runs on x = s a (amax = 0 sends every value there)
  __host__ __device__ __forceinline__ CapSeries(float m_, float invT, float T_)
      : m(m_), s(m_ * invT), T(T_), unfolded(false) {
    const float as = __builtin_fabsf(s);
    if (as > kSeriesScaleMax) {
      unfolded = true;
      amax = 0.0f;
      q1 = q2 = q3 = q4 = 0.0f;
      return;
    }
    const float s2 = s * s;
    amax = as > 0.0f ? kTanhSeriesMax / as : __builtin_inff();
    q1 = m * (-1.0f / 3.0f) * s2;
    q2 = m * (2.0f / 15.0f) * (s2 * s2);
    q3 = m * (-17.0f / 315.0f) * (s2 * s2 * s2);
    q4 = m * (62.0f / 2835.0f) * ((s2 * s2) * (s2 * s2));
  }
};

__host__ __device__ __forceinline__ float softcap_series(float a, const CapSeries& c) {
  const float u = a * a;
  float q = __builtin_fmaf(c.q4, u, c.q3);
  q = __builtin_fmaf(q, u, c.q2);
  q = __builtin_fmaf(q, u, c.q1);
  return a * __builtin_fmaf(u, q, c.m);
}

// The capped logit of one raw accumulator value: the rule softcap_cols
// applies to every value, whichever of its branches a wave takes.
__host__ __device__ __forceinline__ float softcap_value(float a, const CapSeries& c) {
  if (c.unfolded) {
    const float x = c.s * a;
    return c.T * (__builtin_fabsf(x) < kTanhSeriesMax ? tanh_series(x) : tanh_exp_form(x));
  }
  return __builtin_fabsf(a) < c.amax ? softcap_series(a, c) : c.T * tanh_exp_form(c.s * a);
}

// Softcap of one token block already copied out of the accumulators
// (x[bm] = acc[bm][bn]), in place.  Waves whose values all lie inside the
// series range skip the range test; every value inside the range takes the
// series in both branches, so a row's logits do not depend on which rows
// share its wave.
template <bool kCap>
__device__ __forceinline__ void softcap_cols(f32x16 (&x)[4], const CapSeries& c) {
  if (!kCap) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[bm][v] *= c.m;
    return;
  }
  float mabs = 0.0f;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int v = 0; v < 16; ++v) mabs = __builtin_fmaxf(mabs, __builtin_fabsf(x[bm][v]));
  if (__builtin_amdgcn_ballot_w64(mabs >= c.amax)) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[bm][v] = softcap_value(x[bm][v], c);
  } else {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[bm][v] = softcap_series(x[bm][v], c);
  }
}

// Online log-sum-exp / argmax state merge (running max m, sum of exp(z - m),
// index of the first maximum).  Equal maxima keep the lower index.  An empty
// state is (-inf, 0, INT_MAX); the merge is branch-free and never forms
// -inf - (-inf).
__device__ __forceinline__ void merge_stats(float& m, float& s, int& a, float m2, float s2, int a2) {
  const float M = __builtin_fmaxf(m, m2);
  const float Mr = M == kNegInf ? 0.0f : M;
  s = __builtin_fmaf(s, fast_exp(m - Mr), s2 * fast_exp(m2 - Mr));
  a = (m > m2) ? a : (m2 > m) ? a2 : (a < a2 ? a : a2);
  m = M;
}

// Store 4 consecutive values as the storage dtype.
__device__ __forceinline__ void store4(bf16* dst, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(dst) = v;
}
__device__ __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

}  // namespace flce

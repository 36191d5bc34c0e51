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

// tanh for the logit softcap, written from the mathematics:
//  * |x| < 0.25: the odd Maclaurin series x - x^3/3 + 2x^5/15 - 17x^7/315
//    + 62x^9/2835 (the first omitted term is below 1e-8 relative there);
//  * otherwise tanh|x| = 1 - 2 / (e^{2|x|} + 1), which saturates to 1 as
//    e^{2|x|} overflows, with the sign restored.
// Relative error is below 1e-6 over the whole range (tested against fp64).
__host__ __device__ __forceinline__ float tanh_series(float x) {
  const float x2 = x * x;
  float p = 62.0f / 2835.0f;
  p = __builtin_fmaf(p, x2, -17.0f / 315.0f);
  p = __builtin_fmaf(p, x2, 2.0f / 15.0f);
  p = __builtin_fmaf(p, x2, -1.0f / 3.0f);
  p = p * x2;
  return __builtin_fmaf(x, p, x);
}
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
__host__ __device__ __forceinline__ float softcap_tanh(float x) {
  return __builtin_fabsf(x) < kTanhSeriesMax ? tanh_series(x) : tanh_exp_form(x);
}

// Logits of one token block bn of a wave's 4 x 4 accumulator blocks:
// z = T tanh(m a / T) (kCap) or m a, in place; `scale` is m / T (kCap) or m.
// The series serves when every lane's |m a / T| < 1/4 (the usual case for
// lm_head logits under a large cap); otherwise the whole wave takes the
// exponential form.
template <bool kCap>
__device__ __forceinline__ void softcap_block(f32x16 (&acc)[4][4], int bn, float scale, float T) {
  bool need = false;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc[bm][bn][v] *= scale;
      if (kCap) need |= __builtin_fabsf(acc[bm][bn][v]) >= kTanhSeriesMax;
    }
  if (kCap) {
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[bm][bn][v] = T * softcap_tanh(acc[bm][bn][v]);
    } else {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[bm][bn][v] = T * tanh_series(acc[bm][bn][v]);
    }
  }
}

// Softcap of one token block already copied out of the accumulators
// (x[bm] = acc[bm][bn]), z = T tanh(s a) with s = m / T, or m a without a cap.
// The series of tanh_series is evaluated on the raw accumulator a with the
// powers of s and the factor T s = m folded into its coefficients:
//   z = a (m + u Q(u)),  u = a^2,  Q(u) = q1 + u (q2 + u (q3 + u q4)),
//   q_j = m c_j s^(2j)  (c_j the series coefficients -1/3, 2/15, -17/315, 62/2835),
// seven operations per value instead of nine (relative error within 1.2e-7 of
// the float64 tanh over |s a| < 1/4, for m in [-1, 1] and T from 1 to 30);
// values outside that range take the exponential form, in waves that hold
// any.
struct CapSeries {
  float m, s, T, amax, q1, q2, q3, q4;
  __device__ __forceinline__ CapSeries(float m_, float invT, float T_) : m(m_), s(m_ * invT), T(T_) {
    const float s2 = s * s;
    const float as = __builtin_fabsf(s);
    amax = as > 0.0f ? kTanhSeriesMax / as : __builtin_inff();
    q1 = m * (-1.0f / 3.0f) * s2;
    q2 = m * (2.0f / 15.0f) * (s2 * s2);
    q3 = m * (-17.0f / 315.0f) * (s2 * s2 * s2);
    q4 = m * (62.0f / 2835.0f) * ((s2 * s2) * (s2 * s2));
  }
};

__device__ __forceinline__ float softcap_series(float a, const CapSeries& c) {
  const float u = a * a;
  float q = __builtin_fmaf(c.q4, u, c.q3);
  q = __builtin_fmaf(q, u, c.q2);
  q = __builtin_fmaf(q, u, c.q1);
  return a * __builtin_fmaf(u, q, c.m);
}

// Every value inside the series range takes the series in both branches, so a
// row's logits do not depend on which rows share its wave.
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
      for (int v = 0; v < 16; ++v) {
        const float a = x[bm][v];
        x[bm][v] = __builtin_fabsf(a) < c.amax ? softcap_series(a, c) : c.T * tanh_exp_form(c.s * a);
      }
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

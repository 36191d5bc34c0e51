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

// The same on one token block already copied out of the accumulators
// (x[bm] = acc[bm][bn]).
template <bool kCap>
__device__ __forceinline__ void softcap_cols(f32x16 (&x)[4], float scale, float T) {
  bool need = false;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[bm][v] *= scale;
      if (kCap) need |= __builtin_fabsf(x[bm][v]) >= kTanhSeriesMax;
    }
  if (kCap) {
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[bm][v] = T * softcap_tanh(x[bm][v]);
    } else {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[bm][v] = T * tanh_series(x[bm][v]);
    }
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

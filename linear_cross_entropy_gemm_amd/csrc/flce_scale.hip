// Upstream-gradient scaling of stored gradients (flce_scale_grads): the
// backward half of an autograd wrapper around the fused call, which has the
// gradients before it knows the upstream gradient of the loss.  The scale
// stays on the device, so nothing waits for the host.
//
//   scale_same_kernel  grad_h_out = grad_h_in * g in the storage dtype (fp32
//                      arithmetic, one rounding; in place with g == 1 every
//                      block returns at once)
//   scale_cast_kernel  grad_W_out = grad_W_in * g, fp32 in, weight dtype out
//
// Both move 16 bytes of the narrower side per thread and step; the tail of
// fewer than one vector is handled element by element by the first threads.
#include <cmath>

#include "device_common.hpp"
#include "flce_internal.hpp"

namespace flce {

namespace {

constexpr int kScaleThreads = 256;

template <typename T>
__global__ __launch_bounds__(kScaleThreads) void scale_same_kernel(const float* g, const T* x, T* y, int64_t n) {
  const float s = *g;
  if (s == 1.0f && x == y) return;
  constexpr int E = 16 / sizeof(T);
  typedef T vec_t __attribute__((ext_vector_type(E)));
  const int64_t nv = n / E;
  const int64_t stride = (int64_t)gridDim.x * kScaleThreads;
  for (int64_t i = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x; i < nv; i += stride) {
    vec_t v = reinterpret_cast<const vec_t*>(x)[i];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = (T)((float)v[e] * s);
    reinterpret_cast<vec_t*>(y)[i] = v;
  }
  const int64_t t = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x;
  if (t < n - nv * E) y[nv * E + t] = (T)((float)x[nv * E + t] * s);
}

template <typename TO>
__global__ __launch_bounds__(kScaleThreads) void scale_cast_kernel(const float* g, const float* in, TO* out,
                                                                   int64_t n) {
  const float s = *g;
  constexpr int E = 16 / sizeof(TO);   // bf16: 8 values (32 bytes in, 16 out); fp32: 4
  typedef TO vec_t __attribute__((ext_vector_type(E)));
  const int64_t nv = n / E;
  const int64_t stride = (int64_t)gridDim.x * kScaleThreads;
  for (int64_t i = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x; i < nv; i += stride) {
    const f32x4* src = reinterpret_cast<const f32x4*>(in) + i * (E / 4);
    vec_t o;
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const f32x4 a = src[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * q + e] = (TO)(a[e] * s);
    }
    reinterpret_cast<vec_t*>(out)[i] = o;
  }
  const int64_t t = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x;
  if (t < n - nv * E) out[nv * E + t] = (TO)(in[nv * E + t] * s);
}

unsigned scale_grid(int64_t vectors) {
  const int64_t b = (vectors + kScaleThreads - 1) / kScaleThreads;
  return (unsigned)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

}  // namespace flce

extern "C" int flce_scale_grads(const float* grad_scale, const void* grad_h_in, void* grad_h_out, int64_t n_h,
                                int h_dtype, const float* grad_W_in, void* grad_W_out, int64_t n_W, int w_dtype,
                                hipStream_t stream) {
  using namespace flce;
  auto dtype_ok = [](int d) { return d == FLCE_DTYPE_BF16 || d == FLCE_DTYPE_F32; };
  if (!grad_scale || (reinterpret_cast<uintptr_t>(grad_scale) & 3) != 0) return FLCE_EINVAL;
  if (n_h < 0 || n_W < 0 || !dtype_ok(h_dtype) || !dtype_ok(w_dtype)) return FLCE_EINVAL;
  const size_t hb = (size_t)n_h * (h_dtype == FLCE_DTYPE_BF16 ? 2 : 4);
  if (n_h > 0) {
    if (!grad_h_in || !grad_h_out || !aligned16(grad_h_in) || !aligned16(grad_h_out)) return FLCE_EINVAL;
    if (grad_h_in != grad_h_out && overlap(grad_h_in, hb, grad_h_out, hb)) return FLCE_EINVAL;
  }
  if (n_W > 0) {
    if (!grad_W_in || !grad_W_out || !aligned16(grad_W_in) || !aligned16(grad_W_out)) return FLCE_EINVAL;
    const size_t wb = (size_t)n_W * (w_dtype == FLCE_DTYPE_BF16 ? 2 : 4);
    const bool same = w_dtype == FLCE_DTYPE_F32 && static_cast<const void*>(grad_W_in) == grad_W_out;
    if (!same && overlap(grad_W_in, (size_t)n_W * 4, grad_W_out, wb)) return FLCE_EINVAL;
  }
  if (n_h > 0) {
    ProfileScope ps(FLCE_KERNEL_SCALE, stream);
    if (h_dtype == FLCE_DTYPE_BF16)
      scale_same_kernel<bf16><<<scale_grid(n_h / 8), kScaleThreads, 0, stream>>>(
          grad_scale, static_cast<const bf16*>(grad_h_in), static_cast<bf16*>(grad_h_out), n_h);
    else
      scale_same_kernel<float><<<scale_grid(n_h / 4), kScaleThreads, 0, stream>>>(
          grad_scale, static_cast<const float*>(grad_h_in), static_cast<float*>(grad_h_out), n_h);
  }
  if (n_W > 0) {
    ProfileScope ps(FLCE_KERNEL_SCALE, stream);
    if (w_dtype == FLCE_DTYPE_BF16)
      scale_cast_kernel<bf16><<<scale_grid(n_W / 8), kScaleThreads, 0, stream>>>(
          grad_scale, grad_W_in, static_cast<bf16*>(grad_W_out), n_W);
    else
      scale_cast_kernel<float><<<scale_grid(n_W / 4), kScaleThreads, 0, stream>>>(
          grad_scale, grad_W_in, static_cast<float*>(grad_W_out), n_W);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_EDEVICE;
}

// Small per-call kernels shared by the fused path (flce_kernels.hip) and the
// materialised-logits path (flce_logits.hip): status header, label scan
// (N_valid and the label range check), and the final reduction of the
// per-row losses with the optional per-row outputs.  Internal linkage: each
// translation unit launches its own copy.
#pragma once

#include "kernel_args.hpp"

namespace flce {

// ---------------------------------------------------------------------------
static __global__ void header_init_kernel(Header* hdr) {
  if (threadIdx.x == 0) {
    hdr->status = FLCE_OK;
    hdr->n_valid = 0ull;
  }
}

static __global__ __launch_bounds__(256) void label_scan_kernel(const int64_t* labels, int64_t N, int64_t V,
                                                         int64_t ignore_index, Header* hdr) {
  __shared__ unsigned long long cnt[256];
  __shared__ int bad[256];
  unsigned long long c = 0;
  int b = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < N; i += (int64_t)gridDim.x * 256) {
    const int64_t l = labels[i];
    if (l != ignore_index) {
      ++c;
      if (l < 0 || l >= V) b = 1;
    }
  }
  cnt[threadIdx.x] = c;
  bad[threadIdx.x] = b;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      cnt[threadIdx.x] += cnt[threadIdx.x + s];
      bad[threadIdx.x] |= bad[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (cnt[0]) atomicAdd(&hdr->n_valid, cnt[0]);
    if (bad[0]) atomicOr(&hdr->status, FLCE_ELABEL);
  }
}

// loss = s * sum of the per-row losses (fp64, fixed order; s = 1 for sum and
// none), n_correct, and the requested per-row outputs.  With valid-row
// packing the sums run over the packed rows and the per-row losses are
// scattered back to the caller's rows (0 on ignored rows).
static __global__ __launch_bounds__(1024) void finalize_kernel(FinalizeArgs p) {
  __shared__ double ls[1024];
  __shared__ long long cs[1024];
  double a = 0.0;
  long long c = 0;
  if (p.ppos) {
    // packed rows: every one is valid; row outputs other than the loss are
    // never requested on this path
    const int64_t nv = (int64_t)p.hdr->n_valid;
    for (int64_t j = threadIdx.x; j < nv; j += 1024) {
      a += (double)p.loss_row[j];
      c += (p.pred[j] == p.plab[j]) ? 1 : 0;
    }
    if (p.loss_rows)
      for (int64_t i = threadIdx.x; i < p.N; i += 1024) {
        const int q = p.ppos[i];
        p.loss_rows[i] = q >= 0 ? p.loss_row[q] : 0.0f;
      }
  } else {
    for (int64_t i = threadIdx.x; i < p.N; i += 1024) {
      const int64_t lab = p.labels[i];
      if (lab != p.ignore_index) {
        a += (double)p.loss_row[i];
        c += (p.pred[i] == lab) ? 1 : 0;
      }
      if (p.loss_rows) p.loss_rows[i] = p.loss_row[i];
      if (p.lse_rows) p.lse_rows[i] = p.lse[i];
      if (p.pred_rows) p.pred_rows[i] = p.pred[i];
    }
  }
  ls[threadIdx.x] = a;
  cs[threadIdx.x] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      ls[threadIdx.x] += ls[threadIdx.x + s];
      cs[threadIdx.x] += cs[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const unsigned long long nv = p.hdr->n_valid;
    const double s = (p.reduction == FLCE_REDUCTION_MEAN) ? (nv ? 1.0 / (double)nv : 0.0) : 1.0;
    *p.loss = (float)(s * ls[0]);
    if (p.n_correct) *p.n_correct = cs[0];
    if (p.status_out) *p.status_out = p.hdr->status;
  }
}

static __global__ __launch_bounds__(256) void zero_f32_kernel(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.0f;
}

}  // namespace flce

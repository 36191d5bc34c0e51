// Materialised-logits path: the non-fused branch that the Liger-Kernel pages
// compare the fused loss against (Muse Glimmer page, Testing Done: the
// non-fused softcap branch, and skip_logits=False in evaluation; DeepSeek-V3
// page, Summary: without labels or outside training the logits are
// materialised and the plain loss function runs on them).
//
//   logits_kernel   z = cap(m * h W^T) written to the caller's [N, ld] buffer
//                   (same MFMA GEMM as the fused forward; columns >= V are not
//                   written)
//   ce_rows_kernel  cross-entropy of given logits, one work-group per row:
//                   online max / sum exp / first argmax and the label's
//                   logit in one pass, then optionally the logit gradient
//                   s * w_i * (softmax - onehot) in a second pass (in place
//                   allowed)
// plus header_init / label_scan / finalize of the fused path.
#include "common_kernels.hpp"

namespace flce {

struct LogitsArgs {
  const void* h;
  const void* W;
  int64_t ldh, ldw;
  int N, H, V;
  float mult, T, invT;
  void* out;
  int64_t ldo;   // bytes
  TileMap map;
};

struct CeArgs {
  const void* z;
  int64_t ldz;          // bytes
  const int64_t* labels;
  int64_t N, ignore_index;
  int V, reduction;
  const Header* hdr;
  float grad_scale;
  const float* grad_rows;
  void* grad;           // may alias z; null: no gradient
  int64_t ldg;          // bytes
  float* lse;
  float* loss_row;
  int* pred;
};

// Store the capped logits of one token block to the caller's row; in the
// last vocabulary tile, vectors that cross V are stored element by element.
// The softcap is the fused forward's (softcap_cols), so both paths produce
// the same logits bit for bit.
template <typename T, bool kCap>
__device__ __forceinline__ void logits_epilogue(f32x16 (&acc)[4][4], const LogitsArgs& p, int tm, int tn) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, lo = lane & 31, hi = lane >> 5;
  const int vbase = tm * kTile + wm * 128 + hi * 4;
  const bool partial = tm * kTile + kTile > p.V;
  const CapSeries cap(p.mult, p.invT, p.T);
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    f32x16 x[4];
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) x[bm] = acc[bm][bn];
    softcap_cols<kCap>(x, cap);
    const int tok = tn * kTile + wn * 128 + bn * 32 + lo;
    if (tok >= p.N) continue;
    T* zr = reinterpret_cast<T*>(static_cast<char*>(p.out) + (int64_t)tok * p.ldo);
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = vbase + bm * 32 + 8 * i;
        const float x0 = x[bm][4 * i], x1 = x[bm][4 * i + 1];
        const float x2 = x[bm][4 * i + 2], x3 = x[bm][4 * i + 3];
        if (!partial || c + 3 < p.V) {
          store4(zr + c, x0, x1, x2, x3);
        } else {
          if (c < p.V) zr[c] = (T)x0;
          if (c + 1 < p.V) zr[c + 1] = (T)x1;
          if (c + 2 < p.V) zr[c + 2] = (T)x2;
        }
      }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads, 1) void logits_kernel(LogitsArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(T) == 2 ? kDLdsBytes : kLdsBytes];
  int tm, tn, sp;
  map_tile(p.map, tm, tn, sp);
  const int64_t kbytes = (int64_t)p.H * Elem<T>::size;
  f32x16 acc[4][4];
  zero_acc(acc);
  if constexpr (sizeof(T) == 2) {
    gemm_kmajor_direct(p.W, p.ldw, tm * kTile, p.V, p.h, p.ldh, tn * kTile, p.N, kbytes, smem, acc);
  } else {
    KMajorLoader la, lb;
    la.init(p.W, p.ldw, tm * kTile, p.V, kbytes, 0);
    lb.init(p.h, p.ldh, tn * kTile, p.N, kbytes, 0);
    gemm_mainloop<T>(la, lb, (int)((kbytes + kKBytes - 1) / kKBytes), smem, acc);
  }
  if (p.T > 0.0f)
    logits_epilogue<T, true>(acc, p, tm, tn);
  else
    logits_epilogue<T, false>(acc, p, tm, tn);
}

// One row of given logits per work-group of 256 threads.  Thread t visits
// 16-byte vectors t, t + 256, ... in increasing column order, so its running
// (max, sum exp, first argmax) keeps the lowest index on ties; the block then
// merges the threads in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void ce_rows_kernel(CeArgs p) {
  constexpr int E = Elem<T>::per_chunk;
  typedef T vec_t __attribute__((ext_vector_type(E)));
  __shared__ float sm[4], ss[4], szl;
  __shared__ int sa[4];
  __shared__ float s_lse;
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t lab = p.labels[row];
  const bool valid = lab != p.ignore_index;
  const int nvec = (p.V + E - 1) / E;
  const char* zr = static_cast<const char*>(p.z) + row * p.ldz;
  float m = kNegInf, s = 0.0f;
  int a = 0x7fffffff;
  if (t == 0) szl = 0.0f;
  __syncthreads();
  for (int j = t; j < nvec; j += 256) {
    const vec_t zv = *reinterpret_cast<const vec_t*>(zr + (int64_t)j * E * sizeof(T));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int v = j * E + e;
      if (v < p.V) {
        const float x = to_f32(zv[e]);
        if (x > m) {
          s = __builtin_fmaf(s, fast_exp(m - x), 1.0f);
          m = x;
          a = v;
        } else {
          s += fast_exp(x - m);
        }
        if ((int64_t)v == lab) szl = x;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    const int a2 = __shfl_xor(a, off);
    merge_stats(m, s, a, m2, s2, a2);
  }
  if (lane == 0) {
    sm[w] = m;
    ss[w] = s;
    sa[w] = a;
  }
  __syncthreads();
  if (t == 0) {
    float M = sm[0], S = ss[0];
    int A = sa[0];
    for (int k = 1; k < 4; ++k) merge_stats(M, S, A, sm[k], ss[k], sa[k]);
    const float l = M + logf(S);
    p.lse[row] = l;
    p.pred[row] = A;
    p.loss_row[row] = valid ? l - szl : 0.0f;
    s_lse = l;
  }
  if (!p.grad) return;
  __syncthreads();
  const float l = s_lse;
  const unsigned long long nv = p.hdr->n_valid;
  const float red = (p.reduction == FLCE_REDUCTION_MEAN) ? (nv ? 1.0f / (float)nv : 0.0f) : 1.0f;
  const float wrow = valid ? red * p.grad_scale * (p.grad_rows ? p.grad_rows[row] : 1.0f) : 0.0f;
  char* gr = static_cast<char*>(p.grad) + row * p.ldg;
  for (int j = t; j < nvec; j += 256) {
    const vec_t zv = *reinterpret_cast<const vec_t*>(zr + (int64_t)j * E * sizeof(T));
    vec_t gv;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int v = j * E + e;
      float g = 0.0f;
      if (v < p.V) g = wrow * (fast_exp(to_f32(zv[e]) - l) - ((int64_t)v == lab ? 1.0f : 0.0f));
      gv[e] = (T)g;
    }
    *reinterpret_cast<vec_t*>(gr + (int64_t)j * E * sizeof(T)) = gv;
  }
}

template <typename T>
static int logits_typed(const LogitsCallArgs& a, hipStream_t st) {
  constexpr int es = Elem<T>::size;
  const int tiles_tok = (int)((a.N + kTile - 1) / kTile);
  const int tiles_voc = (int)((a.V + kTile - 1) / kTile);
  LogitsArgs p;
  p.h = a.h; p.W = a.W; p.ldh = a.H * es; p.ldw = a.H * es;
  p.N = (int)a.N; p.H = (int)a.H; p.V = (int)a.V;
  p.mult = a.multiplier;
  p.T = a.softcap_T > 0.0f ? a.softcap_T : 0.0f;
  p.invT = a.softcap_T > 0.0f ? 1.0f / a.softcap_T : 0.0f;
  p.out = a.out; p.ldo = a.ld_out * es;
  p.map = TileMap{tiles_voc, tiles_tok, 1, 1, 0, 0};
  if (a.N > 0) {
    ProfileScope ps(FLCE_KERNEL_LOGITS, st);
    logits_kernel<T><<<tiles_voc * tiles_tok, kThreads, 0, st>>>(p);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_EDEVICE;
}

int run_logits(const LogitsCallArgs& a, hipStream_t stream) {
  if (a.dtype == FLCE_DTYPE_BF16) return logits_typed<bf16>(a, stream);
  return logits_typed<float>(a, stream);
}

template <typename T>
static int ce_typed(const CeCallArgs& a, hipStream_t st) {
  char* ws = static_cast<char*>(a.workspace);
  Header* hdr = reinterpret_cast<Header*>(ws);
  const size_t rows = (size_t(a.N) * 4 + 255) & ~size_t(255);
  float* lse = reinterpret_cast<float*>(ws + kHeaderBytes);
  float* loss_row = reinterpret_cast<float*>(ws + kHeaderBytes + rows);
  int* pred = reinterpret_cast<int*>(ws + kHeaderBytes + 2 * rows);
  {
    ProfileScope ps(FLCE_KERNEL_LABEL_SCAN, st);
    header_init_kernel<<<1, 64, 0, st>>>(hdr);
    if (a.N > 0) {
      const int64_t g = (a.N + 255) / 256;
      label_scan_kernel<<<(unsigned)(g < 1024 ? g : 1024), 256, 0, st>>>(a.labels, a.N, a.V, a.ignore_index, hdr);
    }
  }
  if (a.N > 0) {
    CeArgs p;
    p.z = a.logits; p.ldz = a.ld_logits * Elem<T>::size;
    p.labels = a.labels; p.N = a.N; p.ignore_index = a.ignore_index;
    p.V = (int)a.V; p.reduction = a.reduction; p.hdr = hdr;
    p.grad_scale = a.grad_scale; p.grad_rows = a.grad_rows;
    p.grad = a.grad; p.ldg = a.ld_grad * Elem<T>::size;
    p.lse = lse; p.loss_row = loss_row; p.pred = pred;
    ProfileScope ps(FLCE_KERNEL_CROSS_ENTROPY, st);
    ce_rows_kernel<T><<<(unsigned)a.N, 256, 0, st>>>(p);
  }
  FinalizeArgs fa;
  fa.labels = a.labels; fa.N = a.N; fa.ignore_index = a.ignore_index;
  fa.loss_row = loss_row; fa.lse = lse; fa.pred = pred; fa.hdr = hdr; fa.reduction = a.reduction;
  fa.loss = a.loss; fa.n_correct = a.n_correct;
  fa.loss_rows = a.loss_rows; fa.lse_rows = a.lse_rows; fa.pred_rows = a.pred_rows;
  {
    ProfileScope ps(FLCE_KERNEL_FINALIZE, st);
    finalize_kernel<<<1, 1024, 0, st>>>(fa);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_EDEVICE;
}

int run_cross_entropy(const CeCallArgs& a, hipStream_t stream) {
  if (a.dtype == FLCE_DTYPE_BF16) return ce_typed<bf16>(a, stream);
  return ce_typed<float>(a, stream);
}

size_t cross_entropy_workspace(int64_t N) {
  const size_t rows = (size_t(N < 0 ? 0 : N) * 4 + 255) & ~size_t(255);
  return kHeaderBytes + 3 * rows;
}

}  // namespace flce

// HIP kernels of the fused linear cross-entropy path for gfx950, and the
// per-call launch sequence.
//
// Per chunk of C tokens (Liger-Kernel DeepSeek-V3 page, Memory: chunked
// transients instead of the [tokens, vocab] logits):
//   fwd_logits     z = cap(m * h_c W^T) on MFMA, epilogue in registers: softcap,
//                  per (token, 256-vocab tile) max / sum exp / first argmax,
//                  the label's logit, z stored as the chunk's transient
//   row_merge      per-token log-sum-exp, loss and argmax from the tile partials
//   grad_logits    z -> G = m s (softmax - onehot) (1 - (z/T)^2), in place
//   grad_h         partial[s] = G W over a slice of the vocabulary (MFMA)
//   grad_h_reduce  grad_h rows = sum of the slices, cast to the storage dtype
//   grad_W         grad_W (+)= G^T h_c (MFMA), fp32, overwrite on the first chunk
//                  unless the caller accumulates
// and once per call: header_init, the label scan with valid-row packing
// (before), finalize (after).  The forward-only entry runs fwd_logits (without
// storing z) and row_merge per chunk, then finalize.
//
// Valid-row packing: ignored rows add nothing to the loss or to either
// gradient, so unless every row's log-sum-exp or argmax is requested the
// valid rows of h are first gathered, in order, into a packed copy, and the
// chunks run over packed rows: the GEMMs skip whole token tiles and K steps
// past N_valid.  N_valid is known only on the device; the host plans for N
// rows and each kernel reads its chunk's row count (chunk_rows), so nothing
// synchronises.
#include "kernel_args.hpp"
#include "gemm_tile.hpp"
#include "common_kernels.hpp"

namespace flce {

// ---------------------------------------------------------------------------
// Forward logit GEMM with the fused epilogue.  A = W rows (vocabulary on the
// M side), B = h rows (tokens on the N side): each lane then owns one token
// per 32 x 32 block and 16 of its vocabulary entries, so the row statistics
// reduce in registers first, then across lanes l and l + 32, then across the
// two waves that share the tokens.
//
// With one wave per SIMD nothing hides the latency of a dependent chain, so
// the running max / first argmax and the exp-sum keep one independent chain
// per 32-column block (bm), merged in column order at the end; the label's
// logit is picked only in waves whose 128 columns hold some lane's label.
constexpr int kZStage = 4096;   // LDS byte offset of the z staging buffers (after the row partials)

template <typename T, bool kCap, bool kStoreZ>
__device__ __forceinline__ void fwd_epilogue(f32x16 (&acc)[4][4], const FwdArgs& p, int tm, int tn, int Ct,
                                             char* smem) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, lo = lane & 31, hi = lane >> 5;
  const int vbase = tm * kTile + wm * 128 + hi * 4;
  const bool partial = tm * kTile + kTile > p.V;   // only the last vocabulary tile
  const CapSeries cap(p.mult, p.invT, p.T);
  float best[4] = {kNegInf, kNegInf, kNegInf, kNegInf}, sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int bidx[4] = {0, 0, 0, 0};
  // One token block (bn) at a time, 64 values per lane, in a loop that is
  // not unrolled: the block's accumulators are copied out first, so the
  // epilogue's code exists once instead of four times (unrolled, it is several
  // times the size of the instruction cache).
#pragma unroll 1
  for (int bn = 0; bn < 4; ++bn) {
    f32x16 x[4];
    if (bn == 0) {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) x[bm] = acc[bm][0];
    } else if (bn == 1) {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) x[bm] = acc[bm][1];
    } else if (bn == 2) {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) x[bm] = acc[bm][2];
    } else {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) x[bm] = acc[bm][3];
    }
    softcap_cols<kCap>(x, cap);
    // padding columns take no part in the statistics (-inf; exp(-inf) = 0)
    if (partial) {
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int col = vbase + bm * 32 + 8 * (v >> 2) + (v & 3);
          x[bm][v] = col < p.V ? x[bm][v] : kNegInf;
        }
    }
    const int tok = tn * kTile + wn * 128 + bn * 32 + lo;
    const bool tok_ok = tok < Ct;
    const int64_t lab64 = tok_ok ? p.labels[tok] : -1;
    // first maximum: one chain per bm, its maximum first, then the lowest
    // column holding it (columns descending, so the lowest is written last)
    float mxb[4];
    int axb[4];
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      mxb[bm] = kNegInf;
      axb[bm] = 0x7fffffff;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v)
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) mxb[bm] = __builtin_fmaxf(mxb[bm], x[bm][v]);
#pragma unroll
    for (int v = 15; v >= 0; --v)
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
        axb[bm] = x[bm][v] == mxb[bm] ? vbase + bm * 32 + 8 * (v >> 2) + (v & 3) : axb[bm];
    float mx = mxb[0];
    int ax = axb[0];
#pragma unroll
    for (int bm = 1; bm < 4; ++bm) {   // later blocks hold higher columns: strict >
      const bool gt = mxb[bm] > mx;
      mx = gt ? mxb[bm] : mx;
      ax = gt ? axb[bm] : ax;
    }
    // the label's logit, in the rare waves whose columns hold a label
    const int64_t d64 = lab64 - (int64_t)(tm * kTile + wm * 128);
    if (__builtin_amdgcn_ballot_w64(d64 >= 0 && d64 < 128)) {
      const int d = (int)d64 - hi * 4;   // offset from this lane's first column
      float zl = 0.0f;
      bool found = false;
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const bool is_lab = d == bm * 32 + 8 * (v >> 2) + (v & 3);
          zl = is_lab ? x[bm][v] : zl;
          found |= is_lab;
        }
      if (found && lab64 < p.V) p.zlab[tok] = zl;
    }
    if constexpr (kStoreZ && sizeof(T) == 2) {
      // Through this wave's LDS so that each store writes whole 256-byte
      // row segments: [32 tokens][16 units of 16 bytes], unit u of row r at
      // u ^ (r & 15).  A lane's 4 values at columns 32 bm + 8 i + 4 hi are
      // the half hi of unit 4 bm + i.  Wave-local: no barrier.
      char* zs = smem + kZStage + wave * 32768 + bn * 8192;
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = (4 * bm + i) ^ (lo & 15);
          store4(reinterpret_cast<bf16*>(zs + lo * 256 + (u << 4) + 8 * hi), x[bm][4 * i],
                 x[bm][4 * i + 1], x[bm][4 * i + 2], x[bm][4 * i + 3]);
        }
      const int u = lane & 15;
      char* zcol = static_cast<char*>(p.z) + (int64_t)(tm * kTile + wm * 128 + 8 * u) * 2;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lane >> 4);
        const u32x4 w = *reinterpret_cast<const u32x4*>(zs + r * 256 + ((u ^ (r & 15)) << 4));
        const int t = tn * kTile + wn * 128 + bn * 32 + r;
        if (t < Ct) *reinterpret_cast<u32x4*>(zcol + (int64_t)t * p.ldz) = w;
      }
    } else if (kStoreZ && tok_ok) {
      T* zr = reinterpret_cast<T*>(static_cast<char*>(p.z) + (int64_t)tok * p.ldz);
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store4(zr + vbase + bm * 32 + 8 * i, x[bm][4 * i], x[bm][4 * i + 1],
                 x[bm][4 * i + 2], x[bm][4 * i + 3]);
    }
    // sum of exp(z - max): one partial sum per bm
    const float mref = mx == kNegInf ? 0.0f : mx;
    const float off = -mref * kLog2e;
    float sb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int v = 0; v < 16; ++v)
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) sb[bm] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[bm][v], kLog2e, off));
    float s = (sb[0] + sb[1]) + (sb[2] + sb[3]);
    const float m2 = __shfl_xor(mx, 32);
    const float s2 = __shfl_xor(s, 32);
    const int a2 = __shfl_xor(ax, 32);
    merge_stats(mx, s, ax, m2, s2, a2);  // lanes 0-31 carry the pair's result onwards
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      best[k] = k == bn ? mx : best[k];
      sum[k] = k == bn ? s : sum[k];
      bidx[k] = k == bn ? ax : bidx[k];
    }
  }
  float* red_m = reinterpret_cast<float*>(smem);
  float* red_s = red_m + 256;
  int* red_a = reinterpret_cast<int*>(red_s + 256);
  if (wm == 1 && hi == 0) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int idx = wn * 128 + bn * 32 + lo;
      red_m[idx] = best[bn];
      red_s[idx] = sum[bn];
      red_a[idx] = bidx[bn];
    }
  }
  // publishes the LDS partials without waiting for this work-group's z stores
  lds_barrier();
  if (wm == 0 && hi == 0) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int idx = wn * 128 + bn * 32 + lo;
      const int tok = tn * kTile + idx;
      if (tok < Ct) {
        merge_stats(best[bn], sum[bn], bidx[bn], red_m[idx], red_s[idx], red_a[idx]);
        const int64_t o = (int64_t)tm * p.ldp + tok;
        p.pmax[o] = best[bn];
        p.psum[o] = sum[bn];
        p.parg[o] = bidx[bn];
      }
    }
  }
}

// kStoreZ: keep the capped logits for the backward (false on the forward-only
// path, which needs only the row statistics).
template <typename T, bool kStoreZ>
__global__ __launch_bounds__(kThreads, 1) void fwd_logits_kernel(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(T) == 2 ? kDLdsBytes : kLdsBytes];
  int tm, tn, sp;
  map_tile(p.map, tm, tn, sp);
  const int Ct = chunk_rows(p.packed, p.c0, p.C_this);
  if (tn * kTile >= Ct) return;   // token tile past the chunk's (packed) rows
  const int64_t kbytes = (int64_t)p.H * Elem<T>::size;
  f32x16 acc[4][4];
  zero_acc(acc);
  if constexpr (sizeof(T) == 2) {
    gemm_kmajor_direct(p.W, p.ldw, tm * kTile, p.V, p.h, p.ldh, tn * kTile, Ct, kbytes, smem, acc);
  } else {
    KMajorLoader la, lb;
    la.init(p.W, p.ldw, tm * kTile, p.V, kbytes, 0);
    lb.init(p.h, p.ldh, tn * kTile, Ct, kbytes, 0);
    gemm_mainloop<T>(la, lb, (int)((kbytes + kKBytes - 1) / kKBytes), smem, acc);
  }
  if (p.T > 0.0f)
    fwd_epilogue<T, true, kStoreZ>(acc, p, tm, tn, Ct, smem);
  else
    fwd_epilogue<T, false, kStoreZ>(acc, p, tm, tn, Ct, smem);
}

// ---------------------------------------------------------------------------
// Per-token merge of the vocabulary-tile partials: 64 tokens per block, 16
// waves each merging every 16th tile, then a fixed-order merge of the waves.
__global__ __launch_bounds__(1024) void row_merge_kernel(MergeArgs p) {
  __shared__ float sm[16][64];
  __shared__ float ss[16][64];
  __shared__ int sa[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tok = blockIdx.x * 64 + lane;
  const int Ct = chunk_rows(p.packed, p.c0, p.C_this);
  float m = kNegInf, s = 0.0f;
  int a = 0x7fffffff;
  if (tok < Ct) {
    for (int vt = w; vt < p.nvt; vt += 16) {
      const int64_t o = (int64_t)vt * p.ldp + tok;
      merge_stats(m, s, a, p.pmax[o], p.psum[o], p.parg[o]);
    }
  }
  sm[w][lane] = m;
  ss[w][lane] = s;
  sa[w][lane] = a;
  __syncthreads();
  if (w == 0 && tok < Ct) {
    for (int k = 1; k < 16; ++k) merge_stats(m, s, a, sm[k][lane], ss[k][lane], sa[k][lane]);
    const float l = m + logf(s);
    const int64_t lab = p.labels[tok];
    p.lse[tok] = l;
    p.pred[tok] = a;
    p.loss_row[tok] = (lab != p.ignore_index) ? l - p.zlab[tok] : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// z -> G in place, 16 bytes per thread.  Padding columns (V <= v < Vp) and
// ignored rows become exact zeros.
template <typename T>
__global__ __launch_bounds__(256) void grad_logits_kernel(GradLogitArgs p) {
  constexpr int E = Elem<T>::per_chunk;
  const int64_t vecs = p.Vp / E;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= vecs * chunk_rows(p.packed, p.c0, p.C_this)) return;
  const int64_t row = idx / vecs;
  const int col0 = (int)(idx - row * vecs) * E;
  T* zr = reinterpret_cast<T*>(static_cast<char*>(p.z) + row * p.ldz) + col0;
  const int64_t lab = p.labels[row];
  const bool valid = lab != p.ignore_index;
  const unsigned long long nv = p.hdr->n_valid;
  const float s = (p.reduction == FLCE_REDUCTION_MEAN) ? (nv ? 1.0f / (float)nv : 0.0f) : 1.0f;
  const float w = p.grad_rows ? p.grad_rows[row] : 1.0f;
  const float scale = s * p.mult * p.grad_scale * w;
  const float l = p.lse[row];
  typedef T vec_t __attribute__((ext_vector_type(E)));
  vec_t zv = *reinterpret_cast<const vec_t*>(zr);
  vec_t gv;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int v = col0 + e;
    const float z = to_f32(zv[e]);
    float g = 0.0f;
    if (valid && v < p.V) {
      float d = fast_exp(z - l) - ((int64_t)v == lab ? 1.0f : 0.0f);
      if (p.T > 0.0f) {
        const float u = z * p.invT;
        d *= __builtin_fmaf(-u, u, 1.0f);
      }
      g = scale * d;
    }
    gv[e] = (T)g;
  }
  *reinterpret_cast<vec_t*>(zr) = gv;
}

// ---------------------------------------------------------------------------
// grad_h partial over one vocabulary slice: rows = tokens (M), cols = hidden
// (N), K = vocabulary.  A = G [C][Vp] (K contiguous), B = W [V][H] (N
// contiguous: bf16 read with transposing LDS reads, fp32 transposed through
// registers).
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void grad_h_kernel(GradHArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(T) == 2 ? kDLdsBytes : kLdsBytes];
  int tm, tn, sp;
  map_tile(p.map, tm, tn, sp);
  const int Ct = chunk_rows(p.packed, p.c0, p.C_this);
  if (tm * kTile >= Ct) return;   // token tile past the chunk's (packed) rows
  const int k0 = sp * p.ksteps_per_split;
  const int rem = p.ksteps_total - k0;
  const int nk = rem < p.ksteps_per_split ? rem : p.ksteps_per_split;
  f32x16 acc[4][4];
  zero_acc(acc);
  if constexpr (sizeof(T) == 2) {
    // the split is planned in 128-byte K steps, the direct pipeline's step
    static_assert(kKBytes == kDKBytes, "one K step per planned step");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    KMajorDirect<false> la;   // rows of Vp elements: whole K steps
    la.init(p.G, p.ldg, tm * kTile, Ct, (int64_t)p.Vp * 2, k0, (wave >> 1) * 128, lane);
    MNMajorDirect lb;
    lb.init(p.W, p.ldw, tn * kTile, p.H, p.V, k0, (wave & 1) * 128, lane);
    gemm_mainloop_direct(la, lb, nk, smem, acc);
  } else {
    KMajorLoader la;
    la.init(p.G, p.ldg, tm * kTile, Ct, (int64_t)p.Vp * Elem<T>::size, k0);
    MNMajorLoader<T> lb;
    lb.init(p.W, p.ldw, tn * kTile, p.H, p.V, k0);
    gemm_mainloop<T>(la, lb, nk, smem, acc);
  }
  // The partial keeps the accumulator order: tile (tm, tn) is 64 K floats,
  // [wave][bm][bn][quad j][lane][4], so every store writes 1 KB contiguous.
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* out = p.part + (int64_t)sp * p.part_stride + ((int64_t)(tm * p.map.tiles_n + tn) << 16) +
               wave * 16384 + lane * 4;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 q = {acc[bm][bn][4 * j], acc[bm][bn][4 * j + 1], acc[bm][bn][4 * j + 2], acc[bm][bn][4 * j + 3]};
        *reinterpret_cast<f32x4*>(out + ((bm * 4 + bn) * 4 + j) * 256) = q;
      }
}

// grad_h rows = sum of the split partials, in split order.  One thread per
// lane group of a tile: its 16 values sit in 4 quads 1 KB apart (the layout
// grad_h_kernel stores) and map to rows 8 (v >> 2) + 4 hi + (v & 3) of a
// 32 x 32 block at column lo.  Packed rows go back to the caller's rows.
template <typename T>
__global__ __launch_bounds__(256) void grad_h_reduce_kernel(GradHReduceArgs p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= p.groups) return;
  const int tile = (int)(g >> 12), r = (int)(g & 4095);
  const int lane = r & 63, blk = r >> 6;           // blk = (wave * 4 + bm) * 4 + bn
  const int wave = blk >> 4, bm = (blk >> 2) & 3, bn = blk & 3;
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
  const int Ct = chunk_rows(p.packed, p.c0, p.C_this);
  if (tm * kTile >= Ct) return;   // no partials were written for this tile
  const int col = tn * kTile + (wave & 1) * 128 + bn * 32 + (lane & 31);
  const int row0 = tm * kTile + (wave >> 1) * 128 + bm * 32 + 4 * (lane >> 5);
  const float* src = p.part + ((int64_t)tile << 16) + blk * 1024 + lane * 4;
  f32x4 a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const f32x4*>(src + j * 256);
  for (int s = 1; s < p.splits; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] += *reinterpret_cast<const f32x4*>(src + s * p.part_stride + j * 256);
  if (col >= p.H) return;
  T* out = static_cast<T*>(p.out);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + 8 * j + e;
      if (row < Ct) {
        const int64_t orow = p.prow ? (int64_t)p.prow[p.c0 + row] : p.c0 + row;
        out[orow * p.H + col] = (T)a[j][e];
      }
    }
}

// ---------------------------------------------------------------------------
// Store one wave's 128 x 128 fp32 accumulator quadrant of grad_W^T (M =
// hidden, N = vocabulary) to the rows of grad_W through LDS, so that every
// store instruction writes whole 256-byte row segments (in the accumulator
// layout a store touches 32 rows, 32 bytes each).  The quadrant goes in two
// halves of 64 hidden values through this wave's own 32 KB of LDS, laid out
// [128 vocabulary rows][16 units of 16 bytes] with unit u of row r at
// u ^ (r & 15), so that both the scattered writes and the row reads hit 16
// distinct 16-byte bank units per 16 lanes.  Wave-local: no barrier.
// kAccumulate adds the stored grad_W: those loads are row segments too, issued
// before the half goes through LDS so that their latency overlaps it.
template <bool kAccumulate>
__device__ __forceinline__ void store_grad_W_rows(const f32x16 (&acc)[4][4], float* gW, int64_t H, int V,
                                                  int n_base, int m_base, char* lds) {
  const int lane = threadIdx.x & 63, lo = lane & 31, hi = lane >> 5;
  // The wave's rows n_base .. n_base + 127 of grad_W as one buffer range
  // (fewer rows at the end of the vocabulary, none past it): loads and stores
  // of rows past V fall outside it (stores are dropped, loads read 0), and
  // columns past H get an offset outside it, so nothing branches and the
  // waits for the stored values can count exactly (with a branch per store,
  // every store waited for all earlier ones).  128 rows of at most 2^21
  // hidden values stay below 2^30 bytes.
  int rows = V - n_base;
  rows = rows < 0 ? 0 : (rows > 128 ? 128 : rows);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc_wave(reinterpret_cast<const char*>(gW + (int64_t)n_base * H), (int64_t)rows * H * 4);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // H is a multiple of 4, so m < H keeps the whole vector inside the row
    const int m = m_base + half * 64 + 4 * (lane & 15);
    const uint32_t col_off = m < H ? (uint32_t)m * 4u : kOOB;
    f32x4 old[32];
    if constexpr (kAccumulate) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const uint32_t off = col_off == kOOB ? kOOB : (uint32_t)(4 * k + (lane >> 4)) * (uint32_t)H * 4u + col_off;
        old[k] = __builtin_bit_cast(f32x4, load16(rs, off));
      }
    }
#pragma unroll
    for (int bml = 0; bml < 2; ++bml)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = bn * 32 + lo;
          const int unit = bml * 8 + 2 * i + hi;
          const f32x16& a = acc[2 * half + bml][bn];
          *reinterpret_cast<f32x4*>(lds + row * 256 + ((unit ^ (row & 15)) << 4)) =
              f32x4{a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
        }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int row = 4 * k + (lane >> 4), u = lane & 15;
      f32x4 v = *reinterpret_cast<const f32x4*>(lds + row * 256 + ((u ^ (row & 15)) << 4));
      if constexpr (kAccumulate) v += old[k];
      const uint32_t off = col_off == kOOB ? kOOB : (uint32_t)row * (uint32_t)H * 4u + col_off;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)off, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// grad_W (+)= G^T h_c, computed as its transpose h_c^T G: rows = hidden (M),
// cols = vocabulary (N), K = tokens.  Both operands are stored with K as the
// slow dimension (bf16: transposing LDS reads; fp32: transposed through
// registers).  With hidden on the M
// side each lane owns 4 consecutive hidden entries of one vocabulary row of
// grad_W per accumulator group, so the fp32 epilogue moves 16 bytes per
// access.  For every chunk after the first (kAccumulate) the epilogue adds
// the stored grad_W (read-modify-write in whole row segments).
template <typename T, bool kAccumulate>
__global__ __launch_bounds__(kThreads, 1) void grad_W_kernel(GradWArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[sizeof(T) == 2 ? kDLdsBytes : kLdsBytes];
  int tm, tn, sp;
  map_tile(p.map, tm, tn, sp);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // K = the chunk's (packed) rows; an empty chunk adds nothing, and the first
  // chunk with no rows still overwrites grad_W with zeros
  const int Ct = chunk_rows(p.packed, p.c0, p.C_this);
  if (kAccumulate && Ct == 0) return;
  f32x16 acc[4][4];
  zero_acc(acc);
  if constexpr (sizeof(T) == 2) {
    MNMajorDirect la, lb;
    la.init(p.h, p.ldh, tm * kTile, p.H, Ct, 0, wm * 128, lane);
    lb.init(p.G, p.ldg, tn * kTile, p.Vp, Ct, 0, wn * 128, lane);
    constexpr int bk = kDKBytes / 2;
    // G (B) streams from memory, the chunk's h rows are mostly cached: G's
    // loads go first in each step, which gives them two steps to land
    gemm_mainloop_direct<true>(la, lb, (Ct + bk - 1) / bk, smem, acc);
  } else {
    MNMajorLoader<T> la, lb;
    la.init(p.h, p.ldh, tm * kTile, p.H, Ct, 0);
    lb.init(p.G, p.ldg, tn * kTile, p.Vp, Ct, 0);
    constexpr int bk = kKBytes / Elem<T>::size;
    gemm_mainloop<T>(la, lb, (Ct + bk - 1) / bk, smem, acc);
  }
  // the K loop ended with a barrier: the LDS is free, 32 KB per wave
  store_grad_W_rows<kAccumulate>(acc, p.gW, p.H, p.V, tn * kTile + wn * 128, tm * kTile + wm * 128,
                                 smem + wave * 32768);
}

// ---------------------------------------------------------------------------
// Valid-row packing (before the first chunk; no host synchronisation).
//   pack_count    per block of kPackRows rows: the valid count, plus N_valid
//                 and the label range check of the label scan
//   pack_offsets  exclusive prefix sum of the block counts (one block)
//   pack_rows     each row's packed position (-1: ignored); for each packed
//                 row its original row, label and upstream row gradient
//   pack_gather   h rows into the packed copy; grad_h rows of ignored rows
//                 are zeroed here (no chunk writes them)
static_assert(kPackRows == 4 * 256, "four rows per thread");

__global__ __launch_bounds__(256) void pack_count_kernel(const int64_t* labels, int64_t N, int64_t V,
                                                         int64_t ignore_index, Header* hdr, int* cnt) {
  __shared__ int sc[256];
  __shared__ int sb[256];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kPackRows + 4 * t;
  int c = 0, b = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (r0 + k < N) {
      const int64_t l = labels[r0 + k];
      if (l != ignore_index) {
        ++c;
        if (l < 0 || l >= V) b = 1;
      }
    }
  }
  sc[t] = c;
  sb[t] = b;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      sc[t] += sc[t + w];
      sb[t] |= sb[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    cnt[blockIdx.x] = sc[0];
    if (sc[0]) atomicAdd(&hdr->n_valid, (unsigned long long)sc[0]);
    if (sb[0]) atomicOr(&hdr->status, FLCE_ELABEL);
  }
}

// In place: cnt[b] becomes the number of valid rows before block b.
__global__ __launch_bounds__(1024) void pack_offsets_kernel(int* cnt, int64_t nb) {
  __shared__ int s[1024];
  const int t = threadIdx.x;
  int carry = 0;
  for (int64_t base = 0; base < nb; base += 1024) {
    const int64_t i = base + t;
    const int v = i < nb ? cnt[i] : 0;
    s[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan
      const int x = t >= off ? s[t - off] : 0;
      __syncthreads();
      s[t] += x;
      __syncthreads();
    }
    if (i < nb) cnt[i] = carry + s[t] - v;
    carry += s[1023];
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void pack_rows_kernel(const int64_t* labels, int64_t N, int64_t ignore_index,
                                                        const int* boff, const float* grad_rows, int* ppos,
                                                        int* prow, int64_t* plab, float* pgrow) {
  __shared__ int s[256];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kPackRows + 4 * t;
  int64_t lab[4];
  bool ok[4];
  int c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    lab[k] = r0 + k < N ? labels[r0 + k] : ignore_index;
    ok[k] = r0 + k < N && lab[k] != ignore_index;
    c += ok[k] ? 1 : 0;
  }
  s[t] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {   // inclusive scan
    const int x = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += x;
    __syncthreads();
  }
  int pos = boff[blockIdx.x] + s[t] - c;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = r0 + k;
    if (i >= N) break;
    if (ok[k]) {
      ppos[i] = pos;
      prow[pos] = (int)i;
      plab[pos] = lab[k];
      if (grad_rows) pgrow[pos] = grad_rows[i];
      ++pos;
    } else {
      ppos[i] = -1;
    }
  }
}

// One row per block pass, 16 bytes per thread; row_bytes is a multiple of 16.
__global__ __launch_bounds__(256) void pack_gather_kernel(const char* h, int64_t N, int64_t row_bytes,
                                                          const int* ppos, char* ph, char* grad_h) {
  const int64_t nvec = row_bytes / 16;
  for (int64_t i = blockIdx.x; i < N; i += gridDim.x) {
    const int q = ppos[i];
    if (q >= 0) {
      const u32x4* src = reinterpret_cast<const u32x4*>(h + i * row_bytes);
      u32x4* dst = reinterpret_cast<u32x4*>(ph + (int64_t)q * row_bytes);
      for (int64_t e = threadIdx.x; e < nvec; e += 256) dst[e] = src[e];
    } else if (grad_h) {
      u32x4* dst = reinterpret_cast<u32x4*>(grad_h + i * row_bytes);
      for (int64_t e = threadIdx.x; e < nvec; e += 256) dst[e] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// ---------------------------------------------------------------------------
// Launch sequence.
static inline unsigned grid_1d(int64_t work, int64_t per_block) {
  return (unsigned)((work + per_block - 1) / per_block);
}

template <typename T>
static int run_typed(const CallArgs& a, const Plan& pl, hipStream_t st) {
  constexpr int es = Elem<T>::size;
  char* ws = static_cast<char*>(a.workspace);
  Header* hdr = reinterpret_cast<Header*>(ws);
  float* lse = reinterpret_cast<float*>(ws + pl.off_lse);
  float* zlab = reinterpret_cast<float*>(ws + pl.off_zlab);
  float* loss_row = reinterpret_cast<float*>(ws + pl.off_loss_row);
  int* pred = reinterpret_cast<int*>(ws + pl.off_pred);
  float* pmax = reinterpret_cast<float*>(ws + pl.off_pmax);
  float* psum = reinterpret_cast<float*>(ws + pl.off_psum);
  int* parg = reinterpret_cast<int*>(ws + pl.off_parg);
  void* zbuf = ws + pl.off_z;
  float* ghpart = reinterpret_cast<float*>(ws + pl.off_ghpart);
  int* pcnt = reinterpret_cast<int*>(ws + pl.off_pcnt);
  int* ppos = reinterpret_cast<int*>(ws + pl.off_ppos);
  int* prow = reinterpret_cast<int*>(ws + pl.off_prow);
  int64_t* plab = reinterpret_cast<int64_t*>(ws + pl.off_plab);
  float* pgrow = reinterpret_cast<float*>(ws + pl.off_pgrow);
  char* ph = ws + pl.off_ph;
  // every row's log-sum-exp and argmax are outputs only without packing
  const bool pack = a.N > 0 && !a.lse_rows && !a.pred_rows;
  const Header* packed = pack ? hdr : nullptr;

  const int H = (int)a.H, V = (int)a.V, Vp = (int)pl.Vp;
  const int C = (int)pl.C;
  const float invT = a.softcap_T > 0.0f ? 1.0f / a.softcap_T : 0.0f;
  const float capT = a.softcap_T > 0.0f ? a.softcap_T : 0.0f;

  {
    ProfileScope ps(a.profile ? FLCE_KERNEL_LABEL_SCAN : -1, st);
    header_init_kernel<<<1, 64, 0, st>>>(hdr);
    if (pack) {
      const int64_t nb = (a.N + kPackRows - 1) / kPackRows;
      pack_count_kernel<<<(unsigned)nb, 256, 0, st>>>(a.labels, a.N, a.V, a.ignore_index, hdr, pcnt);
      pack_offsets_kernel<<<1, 1024, 0, st>>>(pcnt, nb);
      pack_rows_kernel<<<(unsigned)nb, 256, 0, st>>>(a.labels, a.N, a.ignore_index, pcnt, a.grad_rows, ppos,
                                                     prow, plab, pgrow);
      const int64_t g = a.N < 16384 ? a.N : 16384;
      pack_gather_kernel<<<(unsigned)g, 256, 0, st>>>(static_cast<const char*>(a.h), a.N, a.H * es, ppos, ph,
                                                      a.fwd_only ? nullptr : static_cast<char*>(a.grad_h));
    } else if (a.N > 0) {
      const unsigned g = grid_1d(a.N, 256);
      label_scan_kernel<<<g < 1024 ? g : 1024, 256, 0, st>>>(a.labels, a.N, a.V, a.ignore_index, hdr);
    }
  }
  if (pl.n_chunks == 0 && !a.fwd_only && !a.accumulate_grad_W) {
    ProfileScope ps(a.profile ? FLCE_KERNEL_ZERO : -1, st);
    const int64_t n = a.V * a.H;
    const unsigned g = grid_1d(n, 256);
    zero_f32_kernel<<<g < 65536 ? g : 65536, 256, 0, st>>>(a.grad_W, n);
  }
  for (int64_t ck = 0; ck < pl.n_chunks; ++ck) {
    const int64_t c0 = ck * pl.C;
    const int Ct = (int)((a.N - c0) < pl.C ? (a.N - c0) : pl.C);
    // unpacked: the caller's rows c0..; packed: packed rows c0.. (Ct is then
    // an upper bound and the kernels read the chunk's rows on the device)
    const char* hc = (pack ? ph : static_cast<const char*>(a.h)) + c0 * a.H * es;
    const int64_t* lc = (pack ? plab : a.labels) + c0;
    const int tiles_tok = (Ct + kTile - 1) / kTile;
    const int tiles_voc = Vp / kTile;
    const int tiles_hid = (H + kTile - 1) / kTile;

    FwdArgs f;
    f.h = hc; f.W = a.W; f.labels = lc;
    f.ldh = a.H * es; f.ldw = a.H * es;
    f.C_this = Ct; f.H = H; f.V = V; f.Vp = Vp;
    f.mult = a.multiplier; f.T = capT; f.invT = invT;
    f.z = a.fwd_only ? nullptr : zbuf; f.ldz = (int64_t)Vp * es;
    f.pmax = pmax; f.psum = psum; f.parg = parg; f.ldp = C;
    f.zlab = zlab + c0;
    f.map = TileMap{tiles_voc, tiles_tok, 1, 4, 1, 0};
    f.packed = packed; f.c0 = c0;
    {
      ProfileScope ps(a.profile ? FLCE_KERNEL_FWD_LOGITS : -1, st);
      if (a.fwd_only)
        fwd_logits_kernel<T, false><<<tiles_voc * tiles_tok, kThreads, 0, st>>>(f);
      else
        fwd_logits_kernel<T, true><<<tiles_voc * tiles_tok, kThreads, 0, st>>>(f);
    }

    MergeArgs m;
    m.pmax = pmax; m.psum = psum; m.parg = parg; m.ldp = C; m.nvt = tiles_voc;
    m.labels = lc; m.ignore_index = a.ignore_index;
    m.zlab = zlab + c0; m.lse = lse + c0; m.loss_row = loss_row + c0; m.pred = pred + c0;
    m.C_this = Ct;
    m.packed = packed; m.c0 = c0;
    {
      ProfileScope ps(a.profile ? FLCE_KERNEL_ROW_MERGE : -1, st);
      row_merge_kernel<<<grid_1d(Ct, 64), 1024, 0, st>>>(m);
    }
    if (a.fwd_only) continue;

    GradLogitArgs gl;
    gl.z = zbuf; gl.ldz = (int64_t)Vp * es; gl.C_this = Ct; gl.V = V; gl.Vp = Vp;
    gl.labels = lc; gl.ignore_index = a.ignore_index; gl.lse = lse + c0; gl.hdr = hdr;
    gl.reduction = a.reduction; gl.mult = a.multiplier; gl.T = capT; gl.invT = invT;
    gl.grad_scale = a.grad_scale;
    gl.grad_rows = a.grad_rows ? (pack ? pgrow : a.grad_rows) + c0 : nullptr;
    gl.packed = packed; gl.c0 = c0;
    {
      ProfileScope ps(a.profile ? FLCE_KERNEL_GRAD_LOGITS : -1, st);
      grad_logits_kernel<T><<<grid_1d((int64_t)Ct * (Vp / Elem<T>::per_chunk), 256), 256, 0, st>>>(gl);
    }

    GradHArgs gh;
    gh.G = zbuf; gh.ldg = (int64_t)Vp * es; gh.W = a.W; gh.ldw = a.H * es;
    gh.C_this = Ct; gh.H = H; gh.V = V; gh.Vp = Vp;
    gh.ksteps_total = (int)(((int64_t)Vp * es) / kKBytes);
    gh.ksteps_per_split = (gh.ksteps_total + (int)pl.split_k - 1) / (int)pl.split_k;
    const int splits = (gh.ksteps_total + gh.ksteps_per_split - 1) / gh.ksteps_per_split;
    const int64_t part_stride = ((int64_t)((C + kTile - 1) / kTile) * tiles_hid) << 16;
    gh.part = ghpart; gh.part_stride = part_stride;
    gh.map = TileMap{tiles_tok, tiles_hid, splits, tiles_tok, 0, 0};
    gh.packed = packed; gh.c0 = c0;
    {
      ProfileScope ps(a.profile ? FLCE_KERNEL_GRAD_H : -1, st);
      grad_h_kernel<T><<<tiles_tok * tiles_hid * splits, kThreads, 0, st>>>(gh);
    }

    GradHReduceArgs gr;
    gr.part = ghpart; gr.part_stride = part_stride; gr.splits = splits;
    gr.C_this = Ct; gr.H = H; gr.tiles_n = tiles_hid;
    gr.groups = (int64_t)tiles_tok * tiles_hid * 4096;
    gr.out = a.grad_h;
    gr.packed = packed; gr.c0 = c0; gr.prow = pack ? prow : nullptr;
    {
      ProfileScope ps(a.profile ? FLCE_KERNEL_GRAD_H_REDUCE : -1, st);
      grad_h_reduce_kernel<T><<<grid_1d(gr.groups, 256), 256, 0, st>>>(gr);
    }

    GradWArgs gw;
    gw.G = zbuf; gw.ldg = (int64_t)Vp * es; gw.h = hc; gw.ldh = a.H * es;
    gw.C_this = Ct; gw.H = H; gw.V = V; gw.Vp = Vp;
    gw.gW = a.grad_W; gw.accumulate = (ck > 0 || a.accumulate_grad_W) ? 1 : 0;
    gw.map = TileMap{tiles_hid, tiles_voc, 1, 4, 1, 1};
    gw.packed = packed; gw.c0 = c0;
    {
      ProfileScope ps(a.profile ? FLCE_KERNEL_GRAD_W : -1, st);
      if (gw.accumulate)
        grad_W_kernel<T, true><<<tiles_hid * tiles_voc, kThreads, 0, st>>>(gw);
      else
        grad_W_kernel<T, false><<<tiles_hid * tiles_voc, kThreads, 0, st>>>(gw);
    }
  }
  FinalizeArgs fa;
  fa.labels = a.labels; fa.N = a.N; fa.ignore_index = a.ignore_index;
  fa.loss_row = loss_row; fa.lse = lse; fa.pred = pred; fa.hdr = hdr; fa.reduction = a.reduction;
  fa.loss = a.loss; fa.n_correct = a.n_correct;
  fa.loss_rows = a.loss_rows; fa.lse_rows = a.lse_rows; fa.pred_rows = a.pred_rows;
  fa.status_out = a.status_out;
  if (pack) {
    fa.ppos = ppos;
    fa.plab = plab;
  }
  {
    ProfileScope ps(a.profile ? FLCE_KERNEL_FINALIZE : -1, st);
    finalize_kernel<<<1, 1024, 0, st>>>(fa);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_EDEVICE;
}

int run_call(const CallArgs& a, const Plan& pl, hipStream_t stream) {
  if (a.dtype == FLCE_DTYPE_BF16) return run_typed<bf16>(a, pl, stream);
  return run_typed<float>(a, pl, stream);
}

}  // namespace flce

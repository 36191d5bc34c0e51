// Tiled MFMA GEMM core for gfx950, shared by the forward logit GEMM, the
// grad_h GEMM and the grad_W GEMM.
//
// A work-group of 256 threads (4 waves of 64) owns a 256 x 256 output tile;
// each wave owns a 128 x 128 quadrant computed as 4 x 4 blocks of the
// 32 x 32 MFMA (bf16: v_mfma_f32_32x32x16_bf16, fp32: v_mfma_f32_32x32x2_f32).
// Operand tiles are staged in LDS, double buffered (2 stages x (A + B) x
// 32 KiB = 128 KiB of the 160 KiB per CU), always with K contiguous per row:
// one K step is 128 bytes of K per row (64 bf16 or 32 fp32), i.e. 8 chunks of
// 16 bytes.  Chunk c of row r sits at chunk slot c ^ ((r ^ (r >> 3)) & 7), so
// that both the fragment reads (8 consecutive rows, same chunk) and the
// transposing stores (rows 8 apart, same chunk) hit 8 distinct 16-byte bank
// groups.
//
// MFMA operand layout: for the 32x32 shapes each lane l supplies, for row
// (l & 31) of its operand, one 16-byte chunk of K: chunk 2ks + (l >> 5) of the
// current K step.  A and B use the same lane -> K mapping, so the contraction
// is exact whatever order the instruction sums its K slots in.  The fp32
// variant consumes the chunk's 4 elements with 4 MFMAs of K = 2 (lanes 0-31 and
// 32-63 supply the two K slots).
//
// Result layout (32x32 MFMA): lane l holds column (l & 31) and rows
// 8 * (v >> 2) + 4 * (l >> 5) + (v & 3) for accumulator element v = 0..15.
#pragma once

#include "device_common.hpp"

namespace flce {

constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kKBytes = 128;
constexpr int kOperandStage = kTile * kKBytes;   // 32 KiB
constexpr int kStageBytes = 2 * kOperandStage;   // A + B
constexpr int kLdsBytes = 2 * kStageBytes;       // double buffered: 128 KiB

__device__ __forceinline__ int lds_swizzle(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_offset(int row, int chunk) {
  return row * kKBytes + ((chunk ^ lds_swizzle(row)) << 4);
}

// ---------------------------------------------------------------------------
// Tile scheduling: maps blockIdx.x to (tile_m, tile_n, split).
//   xcd_contiguous: blocks are dispatched round-robin over the 8 XCDs; remap
//     so that each XCD walks a contiguous range of logical tiles (its own L2
//     then sees neighbouring tiles).
//   group_m: within a split, tiles are walked in groups of group_m M-tiles
//     by all N-tiles, M fastest inside a group (group_m = 1: N fastest;
//     group_m >= tiles_m: M fastest over the whole column).
struct TileMap {
  int tiles_m, tiles_n, splits, group_m, xcd_contiguous;
};

__device__ __forceinline__ void map_tile(const TileMap& t, int& tm, int& tn, int& split) {
  const int total = t.tiles_m * t.tiles_n * t.splits;
  int L = blockIdx.x;
  if (t.xcd_contiguous) {
    const int per = total / 8, rem = total % 8;
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    L = x * per + (x < rem ? x : rem) + i;
  }
  const int per_split = t.tiles_m * t.tiles_n;
  split = L / per_split;
  L -= split * per_split;
  const int gsz = t.group_m * t.tiles_n;
  const int g = L / gsz;
  const int r = L - g * gsz;
  const int rows_left = t.tiles_m - g * t.group_m;
  const int gm = rows_left < t.group_m ? rows_left : t.group_m;
  tm = g * t.group_m + r % gm;
  tn = r / gm;
}

// ---------------------------------------------------------------------------
// Loader for an operand stored [mn][k] with k contiguous (row stride `ld`
// bytes).  Thread t moves chunk (t & 7) of rows (t >> 3) + 32 i, i = 0..7.
// Rows >= mn_valid and K bytes >= k_bytes read as zero.
struct KMajorLoader {
  const char* p;
  int64_t rstride;
  int64_t kbyte;
  int64_t k_bytes;
  uint32_t row_mask;
  u32x4 buf[8];

  __device__ __forceinline__ void init(const void* base, int64_t ld, int mn0, int mn_valid,
                                       int64_t k_bytes_, int kstep0) {
    const int t = threadIdx.x;
    const int r = t >> 3, kc = t & 7;
    kbyte = (int64_t)kstep0 * kKBytes + kc * 16;
    p = static_cast<const char*>(base) + (int64_t)(mn0 + r) * ld + kbyte;
    rstride = 32 * ld;
    k_bytes = k_bytes_;
    row_mask = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) row_mask |= (mn0 + r + 32 * i < mn_valid) ? (1u << i) : 0u;
  }
  __device__ __forceinline__ void fetch() {
    const bool kok = kbyte < k_bytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kok && ((row_mask >> i) & 1u)) v = *reinterpret_cast<const u32x4*>(p + i * rstride);
      buf[i] = v;
    }
    p += kKBytes;
    kbyte += kKBytes;
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int t = threadIdx.x;
    const int r = t >> 3, kc = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(lds + lds_offset(r + 32 * i, kc)) = buf[i];
  }
};

// Loader for an operand stored [k][mn] with mn contiguous: the tile is read
// in 16-byte row pieces and transposed in registers so that LDS again holds K
// contiguous per mn row.  mn_valid must be a multiple of the chunk width.
template <typename T> struct MNMajorLoader;

// bf16: thread t moves the 8 x 8 block k = 8 (t >> 5) + 0..7, mn = 8 (t & 31) + 0..7.
template <> struct MNMajorLoader<bf16> {
  const char* p;
  int64_t ld;
  int krow, k_valid;
  bool mn_ok;
  u32x4 buf[8];

  __device__ __forceinline__ void init(const void* base, int64_t ld_, int mn0, int mn_valid,
                                       int k_valid_, int kstep0) {
    const int t = threadIdx.x;
    const int kb = t >> 5, mb = t & 31;
    ld = ld_;
    krow = kstep0 * 64 + kb * 8;
    k_valid = k_valid_;
    mn_ok = mn0 + mb * 8 < mn_valid;
    p = static_cast<const char*>(base) + (int64_t)krow * ld + (int64_t)(mn0 + mb * 8) * 2;
  }
  __device__ __forceinline__ void fetch() {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (mn_ok && krow + j < k_valid) v = *reinterpret_cast<const u32x4*>(p + j * ld);
      buf[j] = v;
    }
    p += 64 * ld;
    krow += 64;
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int t = threadIdx.x;
    const int kb = t >> 5, mb = t & 31;
    // buf[j] holds mn = 0..7 of k row j (dword d: mn 2d low half, 2d+1 high half).
    // Output chunk c holds k = 0..7 of mn column c (dword e: k 2e low, 2e+1 high).
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = buf[2 * e][c >> 1], y = buf[2 * e + 1][c >> 1];
        o[e] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
      }
      *reinterpret_cast<u32x4*>(lds + lds_offset(mb * 8 + c, kb)) = o;
    }
  }
};

// fp32: thread t moves two 4 x 4 blocks b = t + 256 u: k = 4 (b >> 6) + 0..3,
// mn = 4 (b & 63) + 0..3.
template <> struct MNMajorLoader<float> {
  const char* p[2];
  int64_t ld;
  int krow[2], k_valid;
  bool mn_ok;
  u32x4 buf[8];

  __device__ __forceinline__ void init(const void* base, int64_t ld_, int mn0, int mn_valid,
                                       int k_valid_, int kstep0) {
    const int t = threadIdx.x;
    const int mb = t & 63;
    ld = ld_;
    k_valid = k_valid_;
    mn_ok = mn0 + mb * 4 < mn_valid;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb = (t >> 6) + 4 * u;
      krow[u] = kstep0 * 32 + kb * 4;
      p[u] = static_cast<const char*>(base) + (int64_t)krow[u] * ld + (int64_t)(mn0 + mb * 4) * 4;
    }
  }
  __device__ __forceinline__ void fetch() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (mn_ok && krow[u] + j < k_valid) v = *reinterpret_cast<const u32x4*>(p[u] + j * ld);
        buf[4 * u + j] = v;
      }
      p[u] += 32 * ld;
      krow[u] += 32;
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int t = threadIdx.x;
    const int mb = t & 63;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb = (t >> 6) + 4 * u;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 o = {buf[4 * u + 0][c], buf[4 * u + 1][c], buf[4 * u + 2][c], buf[4 * u + 3][c]};
        *reinterpret_cast<u32x4*>(lds + lds_offset(mb * 4 + c, kb)) = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// One chunk of K for every block of the wave's quadrant.  Operands are
// reinterpreted as whole vectors (a bit cast of a single vector element is not
// used: it does not select the element).  The fp32 form issues the chunk's 4
// K slots outermost so that consecutive MFMAs write different accumulators.
__device__ __forceinline__ void mma_quadrant(f32x16 (&acc)[4][4], const u32x4 (&a)[4],
                                             const u32x4 (&b)[4], bf16) {
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
      acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[bm]),
                                                            __builtin_bit_cast(bf16x8, b[bn]),
                                                            acc[bm][bn], 0, 0, 0);
}
__device__ __forceinline__ void mma_quadrant(f32x16 (&acc)[4][4], const u32x4 (&a)[4],
                                             const u32x4 (&b)[4], float) {
  f32x4 af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    af[i] = __builtin_bit_cast(f32x4, a[i]);
    bf[i] = __builtin_bit_cast(f32x4, b[i]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn)
        acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[bm][e], bf[bn][e], acc[bm][bn], 0, 0, 0);
}

// One K step (four sub-steps of two chunks) of the wave's 128 x 128 quadrant.
template <typename T>
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[4][4], const char* As, const char* Bs,
                                          int wm, int wn, int lane) {
  const int lo = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
      a[bm] = *reinterpret_cast<const u32x4*>(As + lds_offset(wm * 128 + bm * 32 + lo, 2 * ks + hi));
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
      b[bn] = *reinterpret_cast<const u32x4*>(Bs + lds_offset(wn * 128 + bn * 32 + lo, 2 * ks + hi));
    mma_quadrant(acc, a, b, T{});
  }
}

// Full K loop: acc = sum over nk K steps of A_tile * B_tile^T.  Ends with a
// barrier, after which the LDS may be reused by the epilogue.
template <typename T, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, f32x16 (&acc)[4][4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bm][bn][v] = 0.0f;
  if (nk <= 0) return;
  la.fetch();
  lb.fetch();
  la.store(smem);
  lb.store(smem + kOperandStage);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    char* cur = smem + (it & 1) * kStageBytes;
    char* nxt = smem + ((it & 1) ^ 1) * kStageBytes;
    const bool more = it + 1 < nk;
    if (more) {
      la.fetch();
      lb.fetch();
    }
    mma_stage<T>(acc, cur, cur + kOperandStage, wm, wn, lane);
    if (more) {
      la.store(nxt);
      lb.store(nxt + kOperandStage);
    }
    __syncthreads();
  }
}

}  // namespace flce

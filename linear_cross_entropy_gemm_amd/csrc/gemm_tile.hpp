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
//   swap_walk: walk as if M and N were exchanged (groups of N-tiles by all
//     M-tiles), for kernels whose reused operand sits on the N side.
struct TileMap {
  int tiles_m, tiles_n, splits, group_m, xcd_contiguous, swap_walk;
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
  const int wm = t.swap_walk ? t.tiles_n : t.tiles_m;
  const int wn = t.swap_walk ? t.tiles_m : t.tiles_n;
  const int gsz = t.group_m * wn;
  const int g = L / gsz;
  const int r = L - g * gsz;
  const int rows_left = wm - g * t.group_m;
  const int gm = rows_left < t.group_m ? rows_left : t.group_m;
  const int a = g * t.group_m + r % gm;
  const int b = r / gm;
  tm = t.swap_walk ? b : a;
  tn = t.swap_walk ? a : b;
}

// ---------------------------------------------------------------------------
// Global loads are raw buffer loads: a descriptor (base, byte range) lives in
// scalar registers and each lane supplies a byte offset.  Offsets at or past
// the range read as zero, so tails and padding need no branches; an offset of
// kOOB is always past the range.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int64_t kMaxRange = 0x7FFFFFFF;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRange ? kMaxRange : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Loader for an operand stored [mn][k] with k contiguous (row stride `ld`
// bytes).  Thread t moves chunk (t & 7) of rows (t >> 3) + 32 i, i = 0..7.
// Rows >= mn_valid and K bytes >= k_bytes read as zero.  The descriptor base
// advances by one K step per fetch, so the per-lane offsets never change.
struct KMajorLoader {
  const char* base;
  int64_t range0;    // valid bytes from the tile base (all valid rows)
  int64_t kpos;      // byte offset of the current K step
  int64_t k_bytes;
  int kc16;
  uint32_t voff[8];
  u32x4 buf[8];

  __device__ __forceinline__ void init(const void* base_, int64_t ld, int mn0, int mn_valid,
                                       int64_t k_bytes_, int kstep0) {
    const int t = threadIdx.x;
    const int r = t >> 3;
    kc16 = (t & 7) * 16;
    int rows = mn_valid - mn0;
    rows = rows < 0 ? 0 : (rows > kTile ? kTile : rows);
    base = static_cast<const char*>(base_) + (int64_t)mn0 * ld;
    range0 = (int64_t)rows * ld;
    kpos = (int64_t)kstep0 * kKBytes;
    k_bytes = k_bytes_;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      voff[i] = (r + 32 * i < rows) ? (uint32_t)((r + 32 * i) * ld + kc16) : kOOB;
  }
  __amdgpu_buffer_rsrc_t rs;
  bool kok;
  // fetch = begin_fetch + fetch_part(0..7) + end_fetch; store = store_part(0..7)
  __device__ __forceinline__ void begin_fetch() {
    rs = make_rsrc(base + kpos, range0 - kpos);
    kok = kpos + kc16 < k_bytes;
  }
  __device__ __forceinline__ void fetch_part(int i) { buf[i] = load16(rs, kok ? voff[i] : kOOB); }
  __device__ __forceinline__ void end_fetch() { kpos += kKBytes; }
  __device__ __forceinline__ void fetch() {
    begin_fetch();
#pragma unroll
    for (int i = 0; i < 8; ++i) fetch_part(i);
    end_fetch();
  }
  __device__ __forceinline__ void store_part(char* lds, int i) const {
    const int t = threadIdx.x;
    *reinterpret_cast<u32x4*>(lds + lds_offset((t >> 3) + 32 * i, t & 7)) = buf[i];
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) store_part(lds, i);
  }
};

// Loader for an operand stored [k][mn] with mn contiguous: the tile is read
// in 16-byte row pieces and transposed in registers so that LDS again holds K
// contiguous per mn row.  mn_valid must be a multiple of the chunk width.
// The descriptor is rebased at the first K row of each step; rows past
// k_valid fall outside its range.
template <typename T> struct MNMajorLoader;

// bf16: thread t moves the 8 x 8 block k = 8 (t >> 5) + 0..7, mn = 8 (t & 31) + 0..7.
template <> struct MNMajorLoader<bf16> {
  const char* base;
  int64_t ld;
  int krow0, k_valid;
  uint32_t voff[8];
  u32x4 buf[8];

  __device__ __forceinline__ void init(const void* base_, int64_t ld_, int mn0, int mn_valid,
                                       int k_valid_, int kstep0) {
    const int t = threadIdx.x;
    const int kb = t >> 5, mb = t & 31;
    ld = ld_;
    base = static_cast<const char*>(base_);
    krow0 = kstep0 * 64;
    k_valid = k_valid_;
    const bool mn_ok = mn0 + mb * 8 < mn_valid;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      voff[j] = mn_ok ? (uint32_t)((kb * 8 + j) * ld + (int64_t)(mn0 + mb * 8) * 2) : kOOB;
  }
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ void begin_fetch() {
    rs = make_rsrc(base + (int64_t)krow0 * ld, (int64_t)(k_valid - krow0) * ld);
  }
  __device__ __forceinline__ void fetch_part(int j) { buf[j] = load16(rs, voff[j]); }
  __device__ __forceinline__ void end_fetch() { krow0 += 64; }
  __device__ __forceinline__ void fetch() {
    begin_fetch();
#pragma unroll
    for (int j = 0; j < 8; ++j) fetch_part(j);
    end_fetch();
  }
  // buf[j] holds mn = 0..7 of k row j (dword d: mn 2d low half, 2d+1 high half).
  // Output chunk c holds k = 0..7 of mn column c (dword e: k 2e low, 2e+1 high).
  __device__ __forceinline__ void store_part(char* lds, int c) const {
    const int t = threadIdx.x;
    const int kb = t >> 5, mb = t & 31;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = buf[2 * e][c >> 1], y = buf[2 * e + 1][c >> 1];
      o[e] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
    }
    *reinterpret_cast<u32x4*>(lds + lds_offset(mb * 8 + c, kb)) = o;
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int c = 0; c < 8; ++c) store_part(lds, c);
  }
};

// fp32: thread t moves two 4 x 4 blocks b = t + 256 u: k = 4 (b >> 6) + 0..3,
// mn = 4 (b & 63) + 0..3.
template <> struct MNMajorLoader<float> {
  const char* base;
  int64_t ld;
  int krow0, k_valid;
  uint32_t voff[8];
  u32x4 buf[8];

  __device__ __forceinline__ void init(const void* base_, int64_t ld_, int mn0, int mn_valid,
                                       int k_valid_, int kstep0) {
    const int t = threadIdx.x;
    const int mb = t & 63;
    ld = ld_;
    base = static_cast<const char*>(base_);
    krow0 = kstep0 * 32;
    k_valid = k_valid_;
    const bool mn_ok = mn0 + mb * 4 < mn_valid;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kr = ((t >> 6) + 4 * u) * 4 + j;
        voff[4 * u + j] = mn_ok ? (uint32_t)(kr * ld + (int64_t)(mn0 + mb * 4) * 4) : kOOB;
      }
  }
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ void begin_fetch() {
    rs = make_rsrc(base + (int64_t)krow0 * ld, (int64_t)(k_valid - krow0) * ld);
  }
  __device__ __forceinline__ void fetch_part(int j) { buf[j] = load16(rs, voff[j]); }
  __device__ __forceinline__ void end_fetch() { krow0 += 32; }
  __device__ __forceinline__ void fetch() {
    begin_fetch();
#pragma unroll
    for (int j = 0; j < 8; ++j) fetch_part(j);
    end_fetch();
  }
  // part p: block u = p >> 2, column c = p & 3
  __device__ __forceinline__ void store_part(char* lds, int p) const {
    const int t = threadIdx.x;
    const int u = p >> 2, c = p & 3;
    const int kb = (t >> 6) + 4 * u;
    u32x4 o = {buf[4 * u + 0][c], buf[4 * u + 1][c], buf[4 * u + 2][c], buf[4 * u + 3][c]};
    *reinterpret_cast<u32x4*>(lds + lds_offset((t & 63) * 4 + c, kb)) = o;
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int p = 0; p < 8; ++p) store_part(lds, p);
  }
};

// ---------------------------------------------------------------------------
// MFMAs of one block row (bm) of the wave's quadrant for one chunk of K.
// Operands are reinterpreted as whole vectors (a bit cast of a single vector
// element is not used: it does not select the element).
__device__ __forceinline__ void mma_row(f32x16 (&acc)[4][4], const u32x4& a, const u32x4 (&b)[4], int bm,
                                        bf16) {
#pragma unroll
  for (int bn = 0; bn < 4; ++bn)
    acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b[bn]),
                                                          acc[bm][bn], 0, 0, 0);
}
// fp32: the chunk's 4 K values feed 4 MFMAs of K = 2, issued slot-outermost so
// that consecutive MFMAs write different accumulators.
__device__ __forceinline__ void mma_row(f32x16 (&acc)[4][4], const u32x4& a, const u32x4 (&b)[4], int bm,
                                        float) {
  const f32x4 af = __builtin_bit_cast(f32x4, a);
  f32x4 bf[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) bf[bn] = __builtin_bit_cast(f32x4, b[bn]);
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
      acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[bn][e], acc[bm][bn], 0, 0, 0);
}

// Per-lane LDS byte offsets of the wave's fragments: A rows wm*128 + bm*32 +
// (l & 31), B rows wn*128 + bn*32 + (l & 31), chunk 2 ks + (l >> 5).
struct FragAddr {
  int a[4][4];   // [bm][ks]
  int b[4][4];   // [bn][ks]
  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    const int lo = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        a[i][ks] = lds_offset(wm * 128 + i * 32 + lo, 2 * ks + hi);
        b[i][ks] = kOperandStage + lds_offset(wn * 128 + i * 32 + lo, 2 * ks + hi);
      }
  }
};

__device__ __forceinline__ u32x4 lds_read16(const char* stage, int off) {
  return *reinterpret_cast<const u32x4*>(stage + off);
}

#define FLCE_FENCE() __builtin_amdgcn_sched_barrier(0)

// Full K loop: acc = sum over nk K steps of A_tile * B_tile^T.
//
// A K step is four sub-steps of 16 MFMAs (4 block rows x 4 block columns),
// each split into four groups of one block row; fences keep the program
// order.  Alongside the MFMAs of sub-step s, the fragments of sub-step s + 1
// are read (B fragments first, so that every MFMA's operands were requested
// at least 8 MFMAs earlier):
//   sub-step 0: -
//   sub-step 1: write the registers fetched one step earlier to the other
//               LDS stage (4 chunks per group)
//   sub-step 2: issue the loads for two steps ahead (4 per group)
//   barrier: everyone is done reading this stage and writing the other
//   sub-step 3: its fragments come from registers; read sub-step 0 of the
//               next stage.
// Fetches and stores run every step (past the last K step the loads are out
// of range and read zeros).  Ends with a barrier, after which the LDS may be
// reused by the epilogue.
template <typename T, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, f32x16 (&acc)[4][4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  FragAddr fa;
  fa.init(wave >> 1, wave & 1, lane);
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
  la.fetch();
  lb.fetch();
  __syncthreads();
  u32x4 a[2][4], b[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[0][i] = lds_read16(smem, fa.b[i][0]);
    a[0][i] = lds_read16(smem, fa.a[i][0]);
  }
  for (int it = 0; it < nk; ++it) {
    const char* cur = smem + (it & 1) * kStageBytes;
    char* nxt = smem + ((it & 1) ^ 1) * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int p = ks & 1, q = p ^ 1;
      if (ks == 2) {
        la.begin_fetch();
        lb.begin_fetch();
      }
      if (ks == 3) {
        FLCE_FENCE();
        __syncthreads();
        FLCE_FENCE();
      }
      const char* src = ks == 3 ? nxt : cur;
      const int nks = (ks + 1) & 3;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        FLCE_FENCE();
        mma_row(acc, a[p][g], b[p], g, T{});
        // fragments of the next sub-step: B first (groups 0-1), then A (2-3)
        if (g < 2) {
          b[q][2 * g] = lds_read16(src, fa.b[2 * g][nks]);
          b[q][2 * g + 1] = lds_read16(src, fa.b[2 * g + 1][nks]);
        } else {
          a[q][2 * g - 4] = lds_read16(src, fa.a[2 * g - 4][nks]);
          a[q][2 * g - 3] = lds_read16(src, fa.a[2 * g - 3][nks]);
        }
        if (ks == 1) {
          la.store_part(nxt, 2 * g);
          la.store_part(nxt, 2 * g + 1);
          lb.store_part(nxt + kOperandStage, 2 * g);
          lb.store_part(nxt + kOperandStage, 2 * g + 1);
        }
        if (ks == 2) {
          la.fetch_part(2 * g);
          la.fetch_part(2 * g + 1);
          lb.fetch_part(2 * g);
          lb.fetch_part(2 * g + 1);
        }
      }
      if (ks == 2) {
        la.end_fetch();
        lb.end_fetch();
      }
    }
  }
  FLCE_FENCE();
  __syncthreads();
}

}  // namespace flce

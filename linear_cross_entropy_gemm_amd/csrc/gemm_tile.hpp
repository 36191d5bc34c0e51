// Tiled MFMA GEMM core for gfx950, shared by the forward logit GEMM, the
// grad_h GEMM and the grad_W GEMM.
//
// A work-group of 256 threads (4 waves of 64) owns a 256 x 256 output tile;
// each wave owns a 128 x 128 quadrant computed as 4 x 4 blocks of the
// 32 x 32 MFMA (bf16: v_mfma_f32_32x32x16_bf16, fp32: v_mfma_f32_32x32x2_f32).
// One K step is 128 bytes of K per operand row (64 bf16 or 32 fp32).
//
// bf16 (every lm_head shape): the direct-to-LDS pipeline further below, a
// ring of five 32 KB operand slots (160 KB) filled by buffer loads that write
// LDS directly; MN-major operands are read back with transposing LDS reads.
//
// fp32 (the small parity workload): the register-staged pipeline that comes
// first, double buffered (2 stages x (A + B) x 32 KiB = 128 KiB), always with
// K contiguous per row in LDS: 8 chunks of 16 bytes per row, chunk c of row r
// at chunk slot c ^ ((r ^ (r >> 3)) & 7), so that both the fragment reads (8
// consecutive rows, same chunk) and the transposing stores (rows 8 apart,
// same chunk) hit 8 distinct 16-byte bank groups.
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

#include <type_traits>

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

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bm][bn][v] = 0.0f;
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
// The same for a base and size that are the same in every lane of the wave
// but which the compiler cannot prove uniform (derived from the wave index):
// taken from the first lane, so the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_wave(const char* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRange ? kMaxRange : bytes);
  const int nu = __builtin_amdgcn_readfirstlane((int)n);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(((uint64_t)hi << 32) | lo), (short)0, nu,
                                           0x00020000);
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
// of range and read zeros).  The products are added to the values `acc`
// holds on entry.  Ends with a barrier, after which the LDS may be reused by
// the epilogue.
template <typename T, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, f32x16 (&acc)[4][4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  FragAddr fa;
  fa.init(wave >> 1, wave & 1, lane);
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

// ===========================================================================
// bf16 pipeline with direct-to-LDS loads.
//
// Global tiles go straight into LDS with buffer_load_dwordx4 ... lds (lane l
// of an instruction fills the 16 bytes at M0 + 16 l; out-of-range offsets
// fill zeros), so no registers stage the operands and no LDS store
// instructions are issued.  A K step moves 128 bytes of K per operand row, so
// every request of a K-major operand is a whole 128-byte line; the load path
// sustains far more bandwidth with whole-line requests than with half lines.
//
// The LDS holds a ring of five operand slots of 32 KB (one operand's 256 rows
// for one K step; 160 KB in all).  Step t computes from A_t and B_t; A_{t+1},
// B_{t+1} and A_{t+2} are in flight or landed, and the slots of A_t and B_t
// are refilled once the step's barrier has released them.  With A_t in slot
// 2t mod 5 and B_t in slot 2t + 1 mod 5, B_{t+2} goes to A_t's slot and A_{t+3}
// to B_t's.
//
// The LDS serves 256 bytes (64 banks of 4 bytes) per cycle: a 16-byte read
// instruction is serviced 16 lanes at a time and an 8-byte one 32 lanes at a
// time, so the layouts below spread those lane groups over 16 distinct
// 16-byte bank units.
//
// K-major operand slot (rows = M or N index, kDCpr chunks of 16 bytes of K
// per row): the kDRpb rows r of one 256-byte bank row B = r / kDRpb hold
// chunk c at unit ((r % kDRpb) * kDCpr + c) ^ (B % kDCpr), so 16 consecutive
// rows reading the same chunk hit 16 different units.
//
// MN-major operand slot (rows = K index, 256 MN values = 512 bytes per row):
// 16-byte unit u of row k sits at unit u ^ (4 (k & 3)).  A fragment is read
// with two ds_read_b64_tr_b16: in each 16-lane group, lane p fetches 4
// consecutive MN values of K row k0 + (p >> 2); the hardware hands lane p the
// 4 K values of MN column (p) -- the same lane -> (row, K) assignment as a
// K-major 16-byte fragment read.
constexpr int kDKBytes = 128;                   // K bytes per row per step (64 bf16)
constexpr int kDSlots = 5;
constexpr int kDSub = kDKBytes / 32;            // 16-wide MFMA sub-steps per K step
constexpr int kDCpr = kDKBytes / 16;            // chunks per K-major row
constexpr int kDRpb = 256 / kDKBytes;           // K-major rows per 256-byte bank row
constexpr int kDLoads = kDKBytes / 16;          // load instructions per wave per operand per step
constexpr int kDOperand = kTile * kDKBytes;     // one slot
constexpr int kDLdsBytes = kDSlots * kDOperand;
static_assert(kDLdsBytes <= 160 * 1024, "LDS capacity");
static_assert(kDSub == 4 && kDLoads == 8, "the K loop issues one or two loads per MFMA group");

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define FLCE_AS3 __attribute__((address_space(3)))

// Buffer descriptor as four scalar dwords (base, stride 0, byte range, raw
// dword format) for the direct-to-LDS load below.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4s make_rsrc_words(const char* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > kMaxRange ? kMaxRange : bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)n, 0x00020000u};
}

// One direct-to-LDS load: lane l's 16 bytes at byte offset soff + voff of the
// buffer land at LDS byte address lds + 16 l (zeros when the offset is out of
// range).  `lds` is wave-uniform and goes to M0 through the register
// constraint, so the compiler forms it there with one scalar add.  Written as
// inline assembly so that the compiler does not treat it as an LDS write that
// every later LDS read must wait for: the K loop orders these loads itself with
// explicit vmcnt waits and barriers, and waits for all of them (vmcnt(0))
// before the LDS is reused.
__device__ __forceinline__ void lds_dma16(const u32x4s& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma16(const u32x4s& r, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(lds) : "memory");
}

// LDS byte address of a __shared__ buffer, and this wave's scalar offset of
// its first 1 KB load destination inside a slot.
__device__ __forceinline__ uint32_t lds_address(const char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const FLCE_AS3 char*)p);
}
__device__ __forceinline__ uint32_t wave_lds_offset() {
  return __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) * kDLoads * 1024);
}

__device__ __forceinline__ int kd_offset(int r, int c) {
  const int B = r / kDRpb;
  return B * 256 + ((((r % kDRpb) * kDCpr + c) ^ (B % kDCpr)) << 4);
}

// K-major operand [mn][k] (k contiguous, row stride `ld` bytes).
// kTail: the K extent may end inside a 128-byte step (rows of H elements
// with H not a multiple of 64), so each chunk is checked against it.
template <bool kTail>
struct KMajorDirect {
  u32x4s rs;           // the tile's rows; the K position goes in the scalar offset
  uint32_t range0;     // bytes of the tile's rows
  int kpos, k_bytes;   // K bytes per row stay below 2^31 (planner limits)
  uint32_t lds_wave;
  uint32_t voff[kDLoads];
  int c16[kDLoads];
  int frag[kDSub];   // per-lane fragment offsets of block 0 per sub-step

  __device__ __forceinline__ void init(const void* base_, int64_t ld, int mn0, int mn_valid, int64_t k_bytes_,
                                       int kstep0, int row0, int lane) {
    const int t = threadIdx.x, w = t >> 6, lam = t & 63;
    int rows = mn_valid - mn0;
    rows = rows < 0 ? 0 : (rows > kTile ? kTile : rows);
    // Lanes of rows in range read kpos + voff < rows * ld, inside the tile's
    // rows, whether or not the range check counts the scalar offset; steps
    // past the K extent (the pipeline runs two ahead) get no records at all.
    rs = make_rsrc_words(static_cast<const char*>(base_) + (int64_t)mn0 * ld, (int64_t)rows * ld);
    range0 = rs[2];
    kpos = kstep0 * kDKBytes;
    // kept in a scalar register: the offset field takes no literal constants
    asm volatile("" : "+s"(kpos));
    k_bytes = (int)k_bytes_;
    set_records();
    lds_wave = wave_lds_offset();
#pragma unroll
    for (int j = 0; j < kDLoads; ++j) {
      const int B = (w * kDLoads + j) * 4 + (lam >> 4);
      const int x = (lam & 15) ^ (B % kDCpr);
      const int r = B * kDRpb + x / kDCpr, c = x % kDCpr;
      voff[j] = r < rows ? (uint32_t)(r * ld + c * 16) : kOOB;
      c16[j] = c * 16;
    }
    const int lo = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kDSub; ++ks) frag[ks] = kd_offset(row0 + lo, 2 * ks + hi);
  }
  // Issue this wave's load j of the current K step into the slot at LDS
  // byte address `slot`; with kTail, chunks past the row's K extent read as
  // zeros.
  __device__ __forceinline__ void issue_part(uint32_t slot, int j) {
    uint32_t off = voff[j];
    if constexpr (kTail) off = c16[j] < k_bytes - kpos ? off : kOOB;
    lds_dma16(rs, slot + lds_wave + j * 1024, off, (uint32_t)kpos);
  }
  __device__ __forceinline__ void set_records() {
    rs[2] = __builtin_amdgcn_readfirstlane(kpos < k_bytes ? range0 : 0u);
  }
  __device__ __forceinline__ void advance() {
    kpos += kDKBytes;
    set_records();
  }
  // Fragment of block b (rows row0 + 32 b + (l & 31)) for sub-step ks.
  __device__ __forceinline__ u32x4 read(const char* stage, int b, int ks) const {
    return *reinterpret_cast<const u32x4*>(stage + frag[ks] + b * 32 * kDKBytes);
  }
};

// MN-major operand [k][mn] (mn contiguous, row stride `ld` bytes).
struct MNMajorDirect {
  const char* kbase;   // K row krow0 of the operand
  int ldb;             // row pitch in bytes; 64 rows of it stay below 2^31
  int krem;            // K rows left from krow0
  u32x4s rs;           // this step's rows (none past the K extent)
  uint32_t lds_wave;
  uint32_t voff[kDLoads];
  int frag[4];   // per-lane offsets of blocks 0..3 (sub-step 0, first half)

  __device__ __forceinline__ void init(const void* base_, int64_t ld_, int mn0, int mn_valid, int k_valid_,
                                       int kstep0, int row0, int lane) {
    const int t = threadIdx.x, w = t >> 6, lam = t & 63;
    const int krow0 = kstep0 * (kDKBytes / 2);
    ldb = (int)ld_;
    kbase = static_cast<const char*>(base_) + (int64_t)krow0 * ld_;
    krem = k_valid_ - krow0;
    set_rsrc();
    lds_wave = wave_lds_offset();
#pragma unroll
    for (int j = 0; j < kDLoads; ++j) {
      const int kr = (w * kDLoads + j) * 2 + (lam >> 5);
      const int u = (lam & 31) ^ ((kr & 3) << 2);
      voff[j] = mn0 + 8 * u < mn_valid ? (uint32_t)(kr * ld_ + (int64_t)(mn0 + 8 * u) * 2) : kOOB;
    }
    // lane (g, p): K row 8 (g >> 1) + (p >> 2) (+ 16 ks + 4 half), MN unit
    // row0/8 + 4 b + 2 (g & 1) + ((p & 3) >> 1), byte (p & 1) * 8 of the unit
    const int g = lane >> 4, p = lane & 15;
    const int q = p >> 2;
    const int x = 2 * (g & 1) + ((p & 3) >> 1);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      frag[b] = (8 * (g >> 1) + q) * 512 + (((4 * b + x) ^ (4 * q)) << 4) + (p & 1) * 8 + row0 * 2;
  }
  // The step's 64 K rows, or the rows left before the K extent (zeros past it).
  __device__ __forceinline__ void set_rsrc() {
    const int rows = krem < kDKBytes / 2 ? (krem < 0 ? 0 : krem) : kDKBytes / 2;
    const uint64_t a = reinterpret_cast<uint64_t>(kbase);
    rs = u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu,
                (uint32_t)__builtin_amdgcn_readfirstlane(rows * ldb), 0x00020000u};
  }
  __device__ __forceinline__ void issue_part(uint32_t slot, int j) {
    lds_dma16(rs, slot + lds_wave + j * 1024, voff[j]);
  }
  __device__ __forceinline__ void advance() {
    kbase += (int64_t)ldb * (kDKBytes / 2);
    krem -= kDKBytes / 2;
    set_rsrc();
  }
  __device__ __forceinline__ u32x4 read(const char* stage, int b, int ks) const {
    const char* q = stage + frag[b] + ks * 8192;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FLCE_AS3 i16x4*)(q));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FLCE_AS3 i16x4*)(q + 4 * 512));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
};

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
#define FLCE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))
// ... and also every LDS access of this wave (lgkmcnt = 0): before a barrier
// after which other waves refill the stage this wave has just read.
#define FLCE_WAIT_VMCNT_LDS(n) __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))

// Workgroup barrier that publishes this wave's LDS writes but, unlike
// __syncthreads, does not wait for its outstanding global stores.  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// K loop of the direct-to-LDS pipeline.  Per K step, four sub-steps of 16
// MFMAs per wave, each split into 4 block-row groups fenced in program order;
// a group issues its global loads first, then its MFMAs and reads of the
// next sub-step's fragments (B first).
// Sub-steps 0 and 1 issue A_{t+2} (one load per group).  Before the last sub-step
// the wave waits for A_{t+1} and B_{t+1} and for its own LDS reads, and the
// barrier both publishes them and frees the slots of A_t and B_t; the last
// sub-step then runs from registers while reading sub-step 0 of step t + 1
// and issuing B_{t+2}.  So A's loads have about 1.5 steps to land and B's
// one; the stream is latency-bound, so the operand that comes from farther
// away (more misses in L2) should go first: kBFirst swaps the roles (B_{t+2}
// during sub-steps 0 and 1, A_{t+2} after the barrier).  The last two steps issue no
// loads (nothing past the K extent is fetched) and wait for everything
// before their barriers.  The products are added to the values `acc` holds
// on entry.  Ends with every load landed and a barrier, after which the LDS
// may be reused by the epilogue.
template <bool kBFirst = false, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop_direct(LA& la, LB& lb, int nk, char* smem, f32x16 (&acc)[4][4]) {
  if (nk <= 0) return;
  auto slot = [&](int q) -> char* { return smem + q * kDOperand; };
  const uint32_t smem_lds = lds_address(smem);
  auto slot_lds = [&](int q) -> uint32_t { return smem_lds + q * kDOperand; };
  auto issue_all = [&](auto& ld, int q) {
#pragma unroll
    for (int j = 0; j < kDLoads; ++j) ld.issue_part(slot_lds(q), j);
    ld.advance();
  };
  constexpr int kA0 = kBFirst ? 1 : 0, kB0 = kBFirst ? 0 : 1;
  if constexpr (kBFirst) {
    issue_all(lb, 0);
    issue_all(la, 1);
    issue_all(lb, 2);
    issue_all(la, 3);
  } else {
    issue_all(la, 0);
    issue_all(lb, 1);
    issue_all(la, 2);
    issue_all(lb, 3);
  }
  FLCE_WAIT_VMCNT(2 * kDLoads);
  __syncthreads();
  u32x4 a[2][4], b[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[0][i] = lb.read(slot(kB0), i, 0);
    a[0][i] = la.read(slot(kA0), i, 0);
  }
  int sa = kA0, sb = kB0, sfree = 4;   // slots of A_t, B_t and the free one
  // One K step.  kAhead: step t + 2 exists and is loaded.  The last two steps
  // run without loads (nothing past the K extent is fetched), so there nothing
  // newer than step t + 1 is in flight when the step waits for it.
  auto step = [&](auto ahead_tag) {
    constexpr bool kAhead = decltype(ahead_tag)::value;
    const int na = sa + 2 >= kDSlots ? sa + 2 - kDSlots : sa + 2;
    const int nb = sb + 2 >= kDSlots ? sb + 2 - kDSlots : sb + 2;
#pragma unroll
    for (int ks = 0; ks < kDSub; ++ks) {
      const int p = ks & 1, q = p ^ 1;
      const bool last = ks == kDSub - 1;
      if (last) {
        FLCE_FENCE();
        if constexpr (kAhead)
          FLCE_WAIT_VMCNT_LDS(kDLoads);
        else
          FLCE_WAIT_VMCNT_LDS(0);
        __syncthreads();
        FLCE_FENCE();
      }
      const char* srca = slot(last ? na : sa);
      const char* srcb = slot(last ? nb : sb);
      const int nks = last ? 0 : ks + 1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        FLCE_FENCE();
        if constexpr (kAhead) {
          // first operand: one load per group over sub-steps 0 and 1;
          // second: two per group once the barrier has freed its slot
          if constexpr (kBFirst) {
            if (ks < 2) {
              lb.issue_part(slot_lds(sfree), 4 * ks + g);
            } else if (last) {
              la.issue_part(slot_lds(sb), 2 * g);
              la.issue_part(slot_lds(sb), 2 * g + 1);
            }
          } else {
            if (ks < 2) {
              la.issue_part(slot_lds(sfree), 4 * ks + g);
            } else if (last) {
              lb.issue_part(slot_lds(sa), 2 * g);
              lb.issue_part(slot_lds(sa), 2 * g + 1);
            }
          }
        }
        mma_row(acc, a[p][g], b[p], g, bf16{});
        if (g < 2) {
          b[q][2 * g] = lb.read(srcb, 2 * g, nks);
          b[q][2 * g + 1] = lb.read(srcb, 2 * g + 1, nks);
        } else {
          a[q][2 * g - 4] = la.read(srca, 2 * g - 4, nks);
          a[q][2 * g - 3] = la.read(srca, 2 * g - 3, nks);
        }
      }
      if (kAhead && ks == 1) {
        if constexpr (kBFirst)
          lb.advance();
        else
          la.advance();
      }
    }
    if (kAhead) {
      if constexpr (kBFirst)
        la.advance();
      else
        lb.advance();
    }
    sfree = kBFirst ? sa : sb;
    sa = na;
    sb = nb;
  };
  int it = 0;
  for (; it < nk - 2; ++it) step(std::true_type{});
  for (; it < nk; ++it) step(std::false_type{});
  FLCE_FENCE();
  FLCE_WAIT_VMCNT(0);
  __syncthreads();
}

// Both operands K-major (rows of kbytes bytes): A rows a0.. (of a_valid) on
// the M side, B rows b0.. (of b_valid) on the N side.  The K tail check is
// compiled in only when the rows end inside a 128-byte step.
__device__ __forceinline__ void gemm_kmajor_direct(const void* A, int64_t lda, int a0, int a_valid, const void* B,
                                                   int64_t ldb, int b0, int b_valid, int64_t kbytes, char* smem,
                                                   f32x16 (&acc)[4][4]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nk = (int)((kbytes + kDKBytes - 1) / kDKBytes);
  if (kbytes % kDKBytes == 0) {
    KMajorDirect<false> la, lb;
    la.init(A, lda, a0, a_valid, kbytes, 0, (wave >> 1) * 128, lane);
    lb.init(B, ldb, b0, b_valid, kbytes, 0, (wave & 1) * 128, lane);
    gemm_mainloop_direct(la, lb, nk, smem, acc);
  } else {
    KMajorDirect<true> la, lb;
    la.init(A, lda, a0, a_valid, kbytes, 0, (wave >> 1) * 128, lane);
    lb.init(B, ldb, b0, b_valid, kbytes, 0, (wave & 1) * 128, lane);
    gemm_mainloop_direct(la, lb, nk, smem, acc);
  }
}

}  // namespace flce

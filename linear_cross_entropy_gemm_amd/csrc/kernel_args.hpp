// Argument blocks of the FLCE kernels (passed by value at launch).
#pragma once

#include "flce_internal.hpp"

#include "gemm_tile.hpp"

namespace flce {

// Rows of the current chunk.  `rows` is the host's count; with valid-row
// packing (`packed` = the header) the chunk starts at packed row c0 and holds
// the valid rows left from there, at most `rows`: N_valid is known only on
// the device, so every kernel of the chunk reads it there.
__device__ __forceinline__ int chunk_rows(const Header* packed, int64_t c0, int rows) {
  if (!packed) return rows;
  const int64_t left = (int64_t)packed->n_valid - c0;
  return left <= 0 ? 0 : (left < rows ? (int)left : rows);
}

struct FwdArgs {
  const void* h;
  const void* W;
  const int64_t* labels;
  int64_t ldh, ldw;
  int C_this, H, V, Vp;
  float mult, T, invT;
  void* z;
  int64_t ldz;
  float* pmax;
  float* psum;
  int* parg;
  int ldp;
  float* zlab;
  TileMap map;
  const Header* packed = nullptr;   // valid-row packing: chunk rows from N_valid (null: C_this)
  int64_t c0 = 0;                   // first (packed) row of the chunk
};

struct MergeArgs {
  const float* pmax;
  const float* psum;
  const int* parg;
  int ldp, nvt;
  const int64_t* labels;
  int64_t ignore_index;
  const float* zlab;
  float* lse;
  float* loss_row;
  int* pred;
  int C_this;
  const Header* packed = nullptr;   // valid-row packing: chunk rows from N_valid (null: C_this)
  int64_t c0 = 0;                   // first (packed) row of the chunk
};

struct GradLogitArgs {
  void* z;
  int64_t ldz;
  int C_this, V, Vp;
  const int64_t* labels;
  int64_t ignore_index;
  const float* lse;
  const Header* hdr;
  int reduction;
  float mult, T, invT;
  float grad_scale;         // upstream gradient of the scalar loss
  const float* grad_rows;   // per-row upstream gradients (reduction none) or null
  const Header* packed = nullptr;   // valid-row packing: chunk rows from N_valid (null: C_this)
  int64_t c0 = 0;                   // first (packed) row of the chunk
};

struct GradHArgs {
  const void* G;
  int64_t ldg;
  const void* W;
  int64_t ldw;
  int C_this, H, V, Vp;
  int ksteps_per_split, ksteps_total;
  float* part;
  int64_t part_stride;
  TileMap map;
  const Header* packed = nullptr;   // valid-row packing: chunk rows from N_valid (null: C_this)
  int64_t c0 = 0;                   // first (packed) row of the chunk
};

struct GradHReduceArgs {
  const float* part;
  int64_t part_stride;
  int splits;
  int C_this, H, tiles_n;
  int64_t groups;   // 16-value lane groups: 4096 per 256 x 256 tile
  void* out;
  const Header* packed = nullptr;
  int64_t c0 = 0;
  const int* prow = nullptr;   // packed: original row of each packed row (null: rows c0 + r of out)
};

struct GradWArgs {
  const void* G;
  int64_t ldg;
  const void* h;
  int64_t ldh;
  int C_this, H, V, Vp;
  float* gW;
  int accumulate;
  TileMap map;
  const Header* packed = nullptr;   // valid-row packing: chunk rows from N_valid (null: C_this)
  int64_t c0 = 0;                   // first (packed) row of the chunk
};

struct FinalizeArgs {
  const int64_t* labels;
  int64_t N, ignore_index;
  const float* loss_row;
  const float* lse;
  const int* pred;
  const Header* hdr;
  int reduction;
  float* loss;
  int64_t* n_correct;
  float* loss_rows;     // optional per-row outputs (null: skipped)
  float* lse_rows;
  int64_t* pred_rows;
  // valid-row packing (null: unpacked): loss_row / pred hold the N_valid
  // packed rows, ppos maps each row to its packed row (-1: ignored), plab
  // holds the packed labels
  const int* ppos = nullptr;
  const int64_t* plab = nullptr;
  int* status_out = nullptr;   // receives the header's final status word (null: none)
};

}  // namespace flce

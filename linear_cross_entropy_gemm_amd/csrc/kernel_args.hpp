// Argument blocks of the FLCE kernels (passed by value at launch).
#pragma once

#include "flce_internal.hpp"

#include "gemm_tile.hpp"

namespace flce {

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
};

struct GradHReduceArgs {
  const float* part;
  int64_t part_stride;
  int splits;
  int C_this, H, tiles_n;
  int64_t groups;   // 16-value lane groups: 4096 per 256 x 256 tile
  void* out;
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
};

}  // namespace flce

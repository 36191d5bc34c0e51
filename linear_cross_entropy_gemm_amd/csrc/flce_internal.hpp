// Internal interfaces between the C ABI (flce_api.cpp), the chunk planner
// (flce_plan.cpp) and the kernels (flce_kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "flce.h"

namespace flce {

// First 256 bytes of the workspace.
struct Header {
  int status;                  // FLCE_OK or FLCE_ELABEL, set on the device
  int pad0;
  unsigned long long n_valid;  // non-ignored rows of the call
};

constexpr size_t kHeaderBytes = 256;
constexpr int64_t kVocabTile = 256;
constexpr int64_t kRowTile = 256;

// Chunk plan and workspace layout (byte offsets from the workspace base).
// A forward-only plan has no logits transient and no grad_h partials.
struct Plan {
  int64_t N, H, V, es;
  int64_t C, n_chunks, Vp, nvt, split_k;
  bool fwd_only;
  size_t off_lse, off_zlab, off_loss_row, off_pred;
  size_t off_pmax, off_psum, off_parg;
  size_t off_z, off_ghpart;
  // valid-row packing: per 1024-row block counts / offsets, packed position
  // of each row (-1: ignored), original row of each packed row, packed
  // labels, packed upstream row gradients, packed h rows [N, H]
  size_t off_pcnt, off_ppos, off_prow, off_plab, off_pgrow, off_ph;
  size_t total;
};

// Rows per block of the valid-row packing scan.
constexpr int64_t kPackRows = 1024;

// Returns FLCE_OK and fills `out`, or an error code (no plan fits the budget).
int make_plan(int64_t N, int64_t H, int64_t V, int dtype, size_t budget, bool fwd_only, Plan* out);

struct CallArgs {
  const void* h;
  const void* W;
  const int64_t* labels;
  int64_t N, H, V, ignore_index;
  float softcap_T, multiplier;
  int reduction, dtype;
  float* loss;
  void* grad_h;       // unused when forward only
  float* grad_W;      // unused when forward only
  int64_t* n_correct;
  void* workspace;
  // options (flce_options_t); defaults: no row outputs, scale 1, overwrite
  float* loss_rows = nullptr;
  float* lse_rows = nullptr;
  int64_t* pred_rows = nullptr;
  const float* grad_rows = nullptr;
  float grad_scale = 1.0f;
  bool accumulate_grad_W = false;
  bool fwd_only = false;
  int* status_out = nullptr;   // device copy of the final status word (null: none)
  bool profile = true;         // false: no timing events even when profiling is on
};

// Enqueue the whole call on `stream`.  Returns FLCE_OK or FLCE_EDEVICE.
int run_call(const CallArgs& a, const Plan& pl, hipStream_t stream);

// Host-side argument checks of the fused entry points (grad_h / grad_W only
// when `with_grads`) and the call description they hand to run_call.
int validate_call(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H, int64_t V,
                  float softcap_T, float multiplier, int reduction, const float* loss, const void* grad_h,
                  const float* grad_W, const int64_t* n_correct, int dtype, const void* workspace,
                  const flce_options_t* o, bool with_grads);
CallArgs make_call_args(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H, int64_t V,
                        int64_t ignore_index, float softcap_T, float multiplier, int reduction, float* loss,
                        void* grad_h, float* grad_W, int64_t* n_correct, int dtype, void* workspace,
                        const flce_options_t* o, bool fwd_only);

// Materialised-logits path (flce_logits / flce_cross_entropy).
struct LogitsCallArgs {
  const void* h;
  const void* W;
  int64_t N, H, V;
  float softcap_T, multiplier;
  void* out;
  int64_t ld_out;   // elements
  int dtype;
};
int run_logits(const LogitsCallArgs& a, hipStream_t stream);

struct CeCallArgs {
  const void* logits;
  int64_t ld_logits;   // elements
  const int64_t* labels;
  int64_t N, V, ignore_index;
  int reduction, dtype;
  float* loss;
  int64_t* n_correct;
  void* grad;          // may alias logits; null: no gradient
  int64_t ld_grad;     // elements
  void* workspace;
  float* loss_rows = nullptr;
  float* lse_rows = nullptr;
  int64_t* pred_rows = nullptr;
  const float* grad_rows = nullptr;
  float grad_scale = 1.0f;
};
int run_cross_entropy(const CeCallArgs& a, hipStream_t stream);
size_t cross_entropy_workspace(int64_t N);

// Brackets one kernel launch with timing events when profiling is enabled
// (kind < 0: never).
class ProfileScope {
 public:
  ProfileScope(int kind, hipStream_t st);
  ~ProfileScope();
  ProfileScope(const ProfileScope&) = delete;
  ProfileScope& operator=(const ProfileScope&) = delete;

 private:
  int kind_;
  hipStream_t st_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

}  // namespace flce

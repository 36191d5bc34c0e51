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

// Split of grad_h = G W over the vocabulary (K = V: long K, narrow output),
// so that the split tiles fill whole waves of the 256 CUs.  Among the splits
// s <= s_max that leave >= 64 K steps per split (or s = 1), the best wave
// efficiency (tiles * splits / (waves * 256), compared exactly); among
// equally efficient ones, the smallest that gives at least 12 waves of tiles
// still >= 256 K steps long, else the smallest.  (The last chunk of a call
// holds only the valid rows left, often fewer token tiles: with few, long
// waves its tiles fill the last wave poorly, with 12 or more the loss stays
// small.)  `splits` counts the nonempty splits of `per` K steps each.
struct SplitChoice {
  int splits, per;
};
inline SplitChoice grad_h_split(int64_t tiles, int64_t ksteps, int64_t s_max) {
  constexpr int64_t kCUs = 256, kMinSplitSteps = 64;
  if (s_max > 16) s_max = 16;
  if (s_max < 1) s_max = 1;
  if (ksteps < 1) return SplitChoice{1, 1};
  // the splits considered: s = 1, and s > 1 while >= 64 K steps per split
  int64_t last = 1;
  while (last < s_max && ksteps / (last + 1) >= kMinSplitSteps) ++last;
  // best efficiency work / (waves * 256), kept as the pair (work, waves) and
  // compared exactly by cross-multiplying
  int64_t best_work = 0, best_waves = 1;
  for (int64_t s = 1; s <= last; ++s) {
    const int64_t per = (ksteps + s - 1) / s, work = tiles * ((ksteps + per - 1) / per);
    const int64_t waves = (work + kCUs - 1) / kCUs;
    if (s == 1 || work * best_waves > best_work * waves) {
      best_work = work;
      best_waves = waves;
    }
  }
  int64_t pick = 0, pick_any = 0;
  for (int64_t s = 1; s <= last && !pick; ++s) {
    const int64_t per = (ksteps + s - 1) / s, real = (ksteps + per - 1) / per, work = tiles * real;
    const int64_t waves = (work + kCUs - 1) / kCUs;
    if (work * best_waves != best_work * waves) continue;
    if (!pick_any) pick_any = s;
    if (waves >= 12 && ksteps / real >= 256) pick = s;
  }
  if (!pick) pick = pick_any ? pick_any : 1;
  const int64_t per = (ksteps + pick - 1) / pick;
  return SplitChoice{(int)((ksteps + per - 1) / per), (int)per};
}

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

// C ABI of the FLCE library: argument validation, planning, dispatch.
#include <cmath>
#include <cstdint>

#include "flce_internal.hpp"

using flce::Plan;

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

extern "C" int flce_plan(int64_t N, int64_t H, int64_t V, int dtype, size_t budget_bytes,
                         flce_plan_t* out) {
  if (!out) return FLCE_EINVAL;
  Plan p;
  const int rc = flce::make_plan(N, H, V, dtype, budget_bytes, false, &p);
  if (rc != FLCE_OK) return rc;
  out->chunk_rows = p.C;
  out->n_chunks = p.n_chunks;
  out->vocab_padded = p.Vp;
  out->split_k = p.split_k;
  out->logits_chunk_bytes = size_t(p.C) * size_t(p.Vp) * size_t(p.es);
  out->workspace_bytes = p.total;
  out->grad_W_bytes = size_t(4) * size_t(V) * size_t(H);
  return FLCE_OK;
}

extern "C" size_t flce_workspace_size(int64_t N, int64_t H, int64_t V, int dtype, size_t budget_bytes) {
  Plan p;
  if (flce::make_plan(N, H, V, dtype, budget_bytes, false, &p) != FLCE_OK) return 0;
  return p.total;
}

extern "C" size_t flce_fwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype, size_t budget_bytes) {
  Plan p;
  if (flce::make_plan(N, H, V, dtype, budget_bytes, true, &p) != FLCE_OK) return 0;
  return p.total;
}

namespace {

// T and m finite, and with a cap 1 / T and m / T finite too (the kernels
// scale by both).
bool scalars_ok(float softcap_T, float multiplier) {
  if (!std::isfinite(softcap_T) || !std::isfinite(multiplier)) return false;
  if (softcap_T > 0.0f && (!std::isfinite(1.0f / softcap_T) || !std::isfinite(multiplier / softcap_T)))
    return false;
  return true;
}

}  // namespace

namespace flce {

// Host-side checks shared by the entry points; nothing is enqueued before
// they pass.  grad_h / grad_W are checked only when `with_grads`.
int validate_call(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H, int64_t V,
                  float softcap_T, float multiplier, int reduction, const float* loss, const void* grad_h,
                  const float* grad_W, const int64_t* n_correct, int dtype, const void* workspace,
                  const flce_options_t* o, bool with_grads) {
  if (dtype != FLCE_DTYPE_BF16 && dtype != FLCE_DTYPE_F32) return FLCE_EINVAL;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM && reduction != FLCE_REDUCTION_NONE)
    return FLCE_EINVAL;
  if (N < 0 || H < 1 || V < 1) return FLCE_EINVAL;
  if (!W || !loss || !workspace) return FLCE_EINVAL;
  if (N > 0 && (!h || !labels)) return FLCE_EINVAL;
  if (!scalars_ok(softcap_T, multiplier)) return FLCE_EINVAL;
  if (!aligned(W, 16) || !aligned(loss, 4) || !aligned(workspace, 256)) return FLCE_EINVAL;
  if (N > 0 && (!aligned(h, 16) || !aligned(labels, 8))) return FLCE_EINVAL;
  if (n_correct && !aligned(n_correct, 8)) return FLCE_EINVAL;
  if (with_grads) {
    if (!grad_W || !aligned(grad_W, 16)) return FLCE_EINVAL;
    if (N > 0 && (!grad_h || !aligned(grad_h, 16))) return FLCE_EINVAL;
  }
  if (reduction == FLCE_REDUCTION_NONE && (!o || !o->loss_rows)) return FLCE_EINVAL;
  if (o) {
    if (o->loss_rows && !aligned(o->loss_rows, 4)) return FLCE_EINVAL;
    if (o->lse_rows && !aligned(o->lse_rows, 4)) return FLCE_EINVAL;
    if (o->pred_rows && !aligned(o->pred_rows, 8)) return FLCE_EINVAL;
    if (with_grads) {
      if (o->grad_rows && (reduction != FLCE_REDUCTION_NONE || !aligned(o->grad_rows, 4))) return FLCE_EINVAL;
      if (o->use_grad_scale != 0 && o->use_grad_scale != 1) return FLCE_EINVAL;
      if (o->use_grad_scale && !std::isfinite(o->grad_scale)) return FLCE_EINVAL;
      if (o->accumulate_grad_W != 0 && o->accumulate_grad_W != 1) return FLCE_EINVAL;
    }
  }
  return FLCE_OK;
}

CallArgs make_call_args(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H, int64_t V,
                        int64_t ignore_index, float softcap_T, float multiplier, int reduction, float* loss,
                        void* grad_h, float* grad_W, int64_t* n_correct, int dtype, void* workspace,
                        const flce_options_t* o, bool fwd_only) {
  CallArgs a;
  a.h = h;
  a.W = W;
  a.labels = labels;
  a.N = N;
  a.H = H;
  a.V = V;
  a.ignore_index = ignore_index;
  a.softcap_T = softcap_T;
  a.multiplier = multiplier;
  a.reduction = reduction;
  a.dtype = dtype;
  a.loss = loss;
  a.grad_h = grad_h;
  a.grad_W = grad_W;
  a.n_correct = n_correct;
  a.workspace = workspace;
  a.fwd_only = fwd_only;
  if (o) {
    a.loss_rows = o->loss_rows;
    a.lse_rows = o->lse_rows;
    a.pred_rows = o->pred_rows;
    if (!fwd_only) {
      a.grad_rows = o->grad_rows;
      a.grad_scale = o->use_grad_scale ? o->grad_scale : 1.0f;
      a.accumulate_grad_W = o->accumulate_grad_W != 0;
    }
  }
  return a;
}

}  // namespace flce

extern "C" int flce_fwd_bwd_ex(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                               int64_t V, int64_t ignore_index, float softcap_T, float multiplier,
                               int reduction, float* loss, void* grad_h, float* grad_W, int64_t* n_correct,
                               hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes,
                               const flce_options_t* options) {
  int rc = flce::validate_call(h, W, labels, N, H, V, softcap_T, multiplier, reduction, loss, grad_h, grad_W,
                    n_correct, dtype, workspace, options, true);
  if (rc != FLCE_OK) return rc;
  Plan p;
  rc = flce::make_plan(N, H, V, dtype, workspace_bytes, false, &p);
  if (rc != FLCE_OK) return rc;
  if (p.total > workspace_bytes) return FLCE_EWORKSPACE;
  const flce::CallArgs a = flce::make_call_args(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier, reduction,
                                     loss, grad_h, grad_W, n_correct, dtype, workspace, options, false);
  return flce::run_call(a, p, stream);
}

extern "C" int flce_fwd_bwd(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                            int64_t V, int64_t ignore_index, float softcap_T, float multiplier,
                            int reduction, float* loss, void* grad_h, float* grad_W, int64_t* n_correct,
                            hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes) {
  if (reduction == FLCE_REDUCTION_NONE) return FLCE_EINVAL;   // needs options.loss_rows
  return flce_fwd_bwd_ex(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier, reduction, loss,
                         grad_h, grad_W, n_correct, stream, dtype, workspace, workspace_bytes, nullptr);
}

extern "C" int flce_fwd(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                        int64_t V, int64_t ignore_index, float softcap_T, float multiplier, int reduction,
                        float* loss, int64_t* n_correct, hipStream_t stream, int dtype, void* workspace,
                        size_t workspace_bytes, const flce_options_t* options) {
  int rc = flce::validate_call(h, W, labels, N, H, V, softcap_T, multiplier, reduction, loss, nullptr, nullptr,
                    n_correct, dtype, workspace, options, false);
  if (rc != FLCE_OK) return rc;
  Plan p;
  rc = flce::make_plan(N, H, V, dtype, workspace_bytes, true, &p);
  if (rc != FLCE_OK) return rc;
  if (p.total > workspace_bytes) return FLCE_EWORKSPACE;
  const flce::CallArgs a = flce::make_call_args(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier, reduction,
                                     loss, nullptr, nullptr, n_correct, dtype, workspace, options, true);
  return flce::run_call(a, p, stream);
}

namespace {

// Row stride rules of the materialised path: ld >= V and 16-byte rows.
bool rows_ok(const void* p, int64_t ld, int64_t V, int64_t es) {
  return p && aligned(p, 16) && ld >= V && (ld * es) % 16 == 0;
}

int check_shape(int64_t N, int64_t H, int64_t V, int dtype) {
  // the planner's shape limits (32-bit tile offsets, H alignment)
  flce::Plan p;
  const int rc = flce::make_plan(N, H, V, dtype, size_t(1) << 62, true, &p);
  return rc == FLCE_EWORKSPACE ? FLCE_OK : rc;
}

}  // namespace

extern "C" int flce_logits(const void* h, const void* W, int64_t N, int64_t H, int64_t V, float softcap_T,
                           float multiplier, void* logits, int64_t ld_logits, hipStream_t stream, int dtype) {
  if (dtype != FLCE_DTYPE_BF16 && dtype != FLCE_DTYPE_F32) return FLCE_EINVAL;
  if (N < 0 || H < 1 || V < 1) return FLCE_EINVAL;
  if (!W || !aligned(W, 16)) return FLCE_EINVAL;
  if (!scalars_ok(softcap_T, multiplier)) return FLCE_EINVAL;
  const int64_t es = dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  if (N > 0 && (!h || !aligned(h, 16) || !rows_ok(logits, ld_logits, V, es))) return FLCE_EINVAL;
  int rc = check_shape(N, H, V, dtype);
  if (rc != FLCE_OK) return rc;
  if ((int64_t(1) << 31) / 256 <= ld_logits * es) return FLCE_EUNSUPPORTED;
  flce::LogitsCallArgs a;
  a.h = h;
  a.W = W;
  a.N = N;
  a.H = H;
  a.V = V;
  a.softcap_T = softcap_T;
  a.multiplier = multiplier;
  a.out = logits;
  a.ld_out = ld_logits;
  a.dtype = dtype;
  return flce::run_logits(a, stream);
}

extern "C" size_t flce_cross_entropy_workspace_size(int64_t N) {
  return N < 0 ? 0 : flce::cross_entropy_workspace(N);
}

extern "C" int flce_cross_entropy(const void* logits, int64_t ld_logits, const int64_t* labels, int64_t N,
                                  int64_t V, int64_t ignore_index, int reduction, float* loss,
                                  int64_t* n_correct, void* grad_logits, int64_t ld_grad, hipStream_t stream,
                                  int dtype, void* workspace, size_t workspace_bytes,
                                  const flce_options_t* o) {
  if (dtype != FLCE_DTYPE_BF16 && dtype != FLCE_DTYPE_F32) return FLCE_EINVAL;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM && reduction != FLCE_REDUCTION_NONE)
    return FLCE_EINVAL;
  if (N < 0 || V < 1 || V > (int64_t(1) << 30)) return FLCE_EINVAL;
  if (N > (int64_t(1) << 31) - 1) return FLCE_EUNSUPPORTED;
  if (!loss || !aligned(loss, 4) || !workspace || !aligned(workspace, 256)) return FLCE_EINVAL;
  if (n_correct && !aligned(n_correct, 8)) return FLCE_EINVAL;
  const int64_t es = dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  if (N > 0) {
    if (!labels || !aligned(labels, 8) || !rows_ok(logits, ld_logits, V, es)) return FLCE_EINVAL;
    if (grad_logits && !rows_ok(grad_logits, ld_grad, V, es)) return FLCE_EINVAL;
    if (grad_logits == logits && ld_grad != ld_logits) return FLCE_EINVAL;
  }
  if (reduction == FLCE_REDUCTION_NONE && (!o || !o->loss_rows)) return FLCE_EINVAL;
  if (o) {
    if (o->loss_rows && !aligned(o->loss_rows, 4)) return FLCE_EINVAL;
    if (o->lse_rows && !aligned(o->lse_rows, 4)) return FLCE_EINVAL;
    if (o->pred_rows && !aligned(o->pred_rows, 8)) return FLCE_EINVAL;
    if (o->grad_rows && (reduction != FLCE_REDUCTION_NONE || !aligned(o->grad_rows, 4))) return FLCE_EINVAL;
    if (o->use_grad_scale != 0 && o->use_grad_scale != 1) return FLCE_EINVAL;
    if (o->use_grad_scale && !std::isfinite(o->grad_scale)) return FLCE_EINVAL;
  }
  if (workspace_bytes < flce::cross_entropy_workspace(N)) return FLCE_EWORKSPACE;
  flce::CeCallArgs a;
  a.logits = logits;
  a.ld_logits = ld_logits;
  a.labels = labels;
  a.N = N;
  a.V = V;
  a.ignore_index = ignore_index;
  a.reduction = reduction;
  a.dtype = dtype;
  a.loss = loss;
  a.n_correct = n_correct;
  a.grad = grad_logits;
  a.ld_grad = ld_grad;
  a.workspace = workspace;
  if (o) {
    a.loss_rows = o->loss_rows;
    a.lse_rows = o->lse_rows;
    a.pred_rows = o->pred_rows;
    a.grad_rows = o->grad_rows;
    a.grad_scale = o->use_grad_scale ? o->grad_scale : 1.0f;
  }
  return flce::run_cross_entropy(a, stream);
}

// The workspace header's fields sit where flce.h documents them.
static_assert(offsetof(flce::Header, status) == 0, "status word at byte 0");
static_assert(offsetof(flce::Header, n_valid) == FLCE_WS_N_VALID_OFFSET, "N_valid at FLCE_WS_N_VALID_OFFSET");

extern "C" int flce_read_status(const void* workspace, hipStream_t stream) {
  if (!workspace) return FLCE_EINVAL;
  flce::Header hdr;
  if (hipMemcpyAsync(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return FLCE_EDEVICE;
  if (hipStreamSynchronize(stream) != hipSuccess) return FLCE_EDEVICE;
  return hdr.status;
}

extern "C" const char* flce_strerror(int code) {
  switch (code) {
    case FLCE_OK: return "success";
    case FLCE_EINVAL: return "invalid argument (null pointer, size, enum, alignment or non-finite scalar)";
    case FLCE_EWORKSPACE: return "workspace too small for any chunk plan";
    case FLCE_EDEVICE: return "HIP launch or runtime call failed";
    case FLCE_ELABEL: return "a label outside [0, V) that is not ignore_index";
    case FLCE_EUNSUPPORTED: return "unsupported shape (H must be a multiple of 8 for bf16, 4 for fp32; H <= 2^21; V <= 2^22 - 256 for bf16, 2^21 - 256 for fp32)";
    case FLCE_ESCRATCH: return "no chunk plan fits the 256 MiB static scratch of flce_fwd_bwd_noalloc (use flce_fwd_bwd_ex with a workspace)";
    default: return "unknown error code";
  }
}

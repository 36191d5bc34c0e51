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
  const int rc = flce::make_plan(N, H, V, dtype, budget_bytes, &p);
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
  if (flce::make_plan(N, H, V, dtype, budget_bytes, &p) != FLCE_OK) return 0;
  return p.total;
}

extern "C" int flce_fwd_bwd(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                            int64_t V, int64_t ignore_index, float softcap_T, float multiplier,
                            int reduction, float* loss, void* grad_h, float* grad_W, int64_t* n_correct,
                            hipStream_t stream, int dtype, void* workspace, size_t workspace_bytes) {
  if (dtype != FLCE_DTYPE_BF16 && dtype != FLCE_DTYPE_F32) return FLCE_EINVAL;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM) return FLCE_EINVAL;
  if (N < 0 || H < 1 || V < 1) return FLCE_EINVAL;
  if (!W || !grad_W || !loss || !workspace) return FLCE_EINVAL;
  if (N > 0 && (!h || !labels || !grad_h)) return FLCE_EINVAL;
  if (std::isnan(softcap_T) || std::isinf(softcap_T) || !std::isfinite(multiplier)) return FLCE_EINVAL;
  if (!aligned(W, 16) || !aligned(grad_W, 16) || !aligned(loss, 4) || !aligned(workspace, 256))
    return FLCE_EINVAL;
  if (N > 0 && (!aligned(h, 16) || !aligned(grad_h, 16) || !aligned(labels, 8))) return FLCE_EINVAL;
  if (n_correct && !aligned(n_correct, 8)) return FLCE_EINVAL;
  Plan p;
  const int rc = flce::make_plan(N, H, V, dtype, workspace_bytes, &p);
  if (rc != FLCE_OK) return rc;
  if (p.total > workspace_bytes) return FLCE_EWORKSPACE;

  flce::CallArgs a;
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
  return flce::run_call(a, p, stream);
}

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
    default: return "unknown error code";
  }
}

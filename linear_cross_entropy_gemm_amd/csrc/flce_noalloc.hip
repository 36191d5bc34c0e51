// flce_fwd_bwd_noalloc: flce_fwd_bwd_ex without a workspace argument, for
// callers that cannot allocate device memory (code under stream capture,
// tight training loops, harnesses that forbid allocation).  Its scratch is a
// file-scope device array of kScratchBytes that every GPU running the library
// holds until the process ends; calls plan their chunks to fit it and are
// rejected (FLCE_ESCRATCH) when no plan does.  The device-side status word
// (out-of-range labels) is copied to the caller's `status` at the end of the
// call, since the caller holds no workspace to read it from.
//
// Host code never passes the array's name to a kernel or a copy: in host code
// the name stands for a host-side shadow, not for device memory.  The array's
// device address is looked up once per device, with that device current, by
// hipGetSymbolAddress, and that address is what the kernels receive.  Every
// call on one GPU shares the array, so calls that overlap in time on one GPU
// race; the call clears what must start at zero (the status word and the
// valid-row count) in its first kernel and writes everything else before
// reading it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "flce_internal.hpp"

namespace {

constexpr size_t kScratchBytes = FLCE_NOALLOC_SCRATCH_BYTES;   // 256 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there), or an error code.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLCE_EDEVICE;
  if (dev >= kMaxDevices) return FLCE_EUNSUPPORTED;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FLCE_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace

extern "C" int flce_fwd_bwd_noalloc(const void* h, const void* W, const int64_t* labels, int64_t N, int64_t H,
                                    int64_t V, int64_t ignore_index, float softcap_T, float multiplier,
                                    int reduction, float* loss, void* grad_h, float* grad_W, int64_t* n_correct,
                                    int* status, hipStream_t stream, int dtype, const flce_options_t* options) {
  // the workspace check of validate_call is met by any aligned non-null
  // stand-in: the scratch address is looked up only once the arguments pass
  alignas(256) static const char kStandIn = 0;
  int rc = flce::validate_call(h, W, labels, N, H, V, softcap_T, multiplier, reduction, loss, grad_h, grad_W,
                               n_correct, dtype, &kStandIn, options, true);
  if (rc != FLCE_OK) return rc;
  if (status && (reinterpret_cast<uintptr_t>(status) & 3) != 0) return FLCE_EINVAL;
  flce::Plan p;
  rc = flce::make_plan(N, H, V, dtype, kScratchBytes, false, &p);
  if (rc == FLCE_EWORKSPACE || (rc == FLCE_OK && p.total > kScratchBytes)) return FLCE_ESCRATCH;
  if (rc != FLCE_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FLCE_OK) return rc;
  flce::CallArgs a = flce::make_call_args(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier, reduction,
                                          loss, grad_h, grad_W, n_correct, dtype, ws, options, false);
  a.status_out = status;
  a.profile = false;   // the timing facility creates events: not here
  return flce::run_call(a, p, stream);
}

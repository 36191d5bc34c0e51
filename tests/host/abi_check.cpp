// Host-only build of the C ABI's argument checks and chunk planner
// (flce_api.cpp, flce_plan.cpp) for tests/test_abi_sanitized.py, which
// compiles it with g++ -fsanitize=address,undefined.  The kernels are
// replaced by stubs that count launches and check the plan they receive, and
// the two HIP runtime calls of flce_read_status by stubs, so nothing touches
// a GPU.  Every case checks a return code and that rejected calls launch
// nothing; the planner is swept over seeded random shapes and budgets.
// Prints one line per failed check and exits non-zero if any failed.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>

#include "flce.h"
#include "flce_internal.hpp"

namespace {
int g_launches = 0;
int g_failed = 0;
size_t g_last_ws = 0;   // workspace bytes of the call being checked

void expect(bool ok, const char* what, long long a = 0, long long b = 0) {
  if (!ok) {
    ++g_failed;
    std::printf("FAIL %s (%lld, %lld)\n", what, a, b);
  }
}
}  // namespace

namespace flce {
int run_call(const CallArgs& a, const Plan& pl, hipStream_t) {
  ++g_launches;
  expect(pl.total <= g_last_ws, "plan larger than the workspace", (long long)pl.total, (long long)g_last_ws);
  expect(a.N == pl.N && a.H == pl.H && a.V == pl.V, "plan of another shape");
  expect(pl.N == 0 || (pl.C >= 1 && pl.n_chunks == (pl.N + pl.C - 1) / pl.C), "chunk count");
  return FLCE_OK;
}
int run_logits(const LogitsCallArgs&, hipStream_t) { ++g_launches; return FLCE_OK; }
int run_cross_entropy(const CeCallArgs&, hipStream_t) { ++g_launches; return FLCE_OK; }
size_t cross_entropy_workspace(int64_t N) {
  const size_t rows = (size_t(N < 0 ? 0 : N) * 4 + 255) & ~size_t(255);
  return kHeaderBytes + 3 * rows;
}
ProfileScope::ProfileScope(int kind, hipStream_t st) : kind_(kind), st_(st) {}
ProfileScope::~ProfileScope() {}
}  // namespace flce

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);   // the "device" workspace is host memory here
  return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

namespace {

// Fake, aligned device addresses: the stubs never dereference them.
void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

struct Call {
  uintptr_t h = 16, W = 16, labels = 8, loss = 4, grad_h = 16, grad_W = 16, n_correct = 0, ws = 256;
  int64_t N = 4, H = 8, V = 8, ignore = -100;
  float T = 0.0f, m = 1.0f;
  int reduction = 0, dtype = 0;
  size_t ws_bytes = 64;
  int fwd_bwd() const {
    g_last_ws = ws_bytes;
    return flce_fwd_bwd(P(h), P(W), (const int64_t*)P(labels), N, H, V, ignore, T, m, reduction, (float*)P(loss),
                        P(grad_h), (float*)P(grad_W), (int64_t*)P(n_correct), nullptr, dtype, P(ws), ws_bytes);
  }
  int ex(const flce_options_t* o) const {
    g_last_ws = ws_bytes;
    return flce_fwd_bwd_ex(P(h), P(W), (const int64_t*)P(labels), N, H, V, ignore, T, m, reduction,
                           (float*)P(loss), P(grad_h), (float*)P(grad_W), (int64_t*)P(n_correct), nullptr, dtype,
                           P(ws), ws_bytes, o);
  }
  int fwd(const flce_options_t* o) const {
    g_last_ws = ws_bytes;
    return flce_fwd(P(h), P(W), (const int64_t*)P(labels), N, H, V, ignore, T, m, reduction, (float*)P(loss),
                    (int64_t*)P(n_correct), nullptr, dtype, P(ws), ws_bytes, o);
  }
};

void check_rejects(const char* what, int got, int want) {
  const int before = g_launches;
  expect(got == want, what, got, want);
  expect(g_launches == before, "a rejected call launched");
}

void validation_cases() {
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
  struct Case {
    const char* name;
    void (*edit)(Call&);
    int want;
  };
  const Case cases[] = {
      {"dtype", [](Call& c) { c.dtype = 3; }, FLCE_EINVAL},
      {"reduction none without options", [](Call& c) { c.reduction = 2; }, FLCE_EINVAL},
      {"reduction", [](Call& c) { c.reduction = 3; }, FLCE_EINVAL},
      {"N", [](Call& c) { c.N = -1; }, FLCE_EINVAL},
      {"H", [](Call& c) { c.H = 0; }, FLCE_EINVAL},
      {"V", [](Call& c) { c.V = 0; }, FLCE_EINVAL},
      {"W null", [](Call& c) { c.W = 0; }, FLCE_EINVAL},
      {"grad_W null", [](Call& c) { c.grad_W = 0; }, FLCE_EINVAL},
      {"loss null", [](Call& c) { c.loss = 0; }, FLCE_EINVAL},
      {"workspace null", [](Call& c) { c.ws = 0; }, FLCE_EINVAL},
      {"h null", [](Call& c) { c.h = 0; }, FLCE_EINVAL},
      {"labels null", [](Call& c) { c.labels = 0; }, FLCE_EINVAL},
      {"grad_h null", [](Call& c) { c.grad_h = 0; }, FLCE_EINVAL},
      {"h misaligned", [](Call& c) { c.h = 24; }, FLCE_EINVAL},
      {"W misaligned", [](Call& c) { c.W = 8; }, FLCE_EINVAL},
      {"workspace misaligned", [](Call& c) { c.ws = 512 + 16; }, FLCE_EINVAL},
      {"labels misaligned", [](Call& c) { c.labels = 12; }, FLCE_EINVAL},
      {"T nan", [](Call& c) { c.T = std::numeric_limits<float>::quiet_NaN(); }, FLCE_EINVAL},
      {"T inf", [](Call& c) { c.T = std::numeric_limits<float>::infinity(); }, FLCE_EINVAL},
      {"m inf", [](Call& c) { c.m = std::numeric_limits<float>::infinity(); }, FLCE_EINVAL},
      {"1/T overflows", [](Call& c) { c.T = 1e-39f; }, FLCE_EINVAL},
      {"m/T overflows", [](Call& c) { c.T = 1e-30f; c.m = 1e10f; }, FLCE_EINVAL},
      {"H not a multiple of 8", [](Call& c) { c.H = 12; }, FLCE_EUNSUPPORTED},
      {"H too large", [](Call& c) { c.H = (int64_t(1) << 21) + 8; }, FLCE_EUNSUPPORTED},
      {"V too large", [](Call& c) { c.V = (int64_t(1) << 22) - 255; }, FLCE_EUNSUPPORTED},
      {"N too large", [](Call& c) { c.N = int64_t(1) << 31; }, FLCE_EUNSUPPORTED},
      {"workspace too small", [](Call&) {}, FLCE_EWORKSPACE},
  };
  for (const Case& k : cases) {
    Call c;
    k.edit(c);
    check_rejects(k.name, c.fwd_bwd(), k.want);
  }
  // options of flce_fwd_bwd_ex
  auto opts = [] {
    flce_options_t o;
    std::memset(&o, 0, sizeof(o));
    return o;
  };
  {
    Call c;
    c.reduction = 2;
    flce_options_t o = opts();
    o.lse_rows = (float*)P(64);
    check_rejects("none without loss_rows", c.ex(&o), FLCE_EINVAL);
    o.loss_rows = (float*)P(66);
    check_rejects("loss_rows misaligned", c.ex(&o), FLCE_EINVAL);
    o.loss_rows = (float*)P(64);
    o.grad_rows = (const float*)P(66);
    check_rejects("grad_rows misaligned", c.ex(&o), FLCE_EINVAL);
  }
  {
    Call c;
    flce_options_t o = opts();
    o.loss_rows = (float*)P(64);
    o.grad_rows = (const float*)P(64);
    check_rejects("grad_rows without none", c.ex(&o), FLCE_EINVAL);
    o = opts();
    o.pred_rows = (int64_t*)P(68);
    check_rejects("pred_rows misaligned", c.ex(&o), FLCE_EINVAL);
    o = opts();
    o.grad_scale = nan;
    o.use_grad_scale = 1;
    check_rejects("grad_scale nan", c.ex(&o), FLCE_EINVAL);
    o.grad_scale = inf;
    check_rejects("grad_scale inf", c.ex(&o), FLCE_EINVAL);
    o.grad_scale = nan;
    o.use_grad_scale = 0;
    check_rejects("unused grad_scale", c.ex(&o), FLCE_EWORKSPACE);
    o = opts();
    o.use_grad_scale = 2;
    check_rejects("use_grad_scale", c.ex(&o), FLCE_EINVAL);
    o = opts();
    o.accumulate_grad_W = 2;
    check_rejects("accumulate_grad_W", c.ex(&o), FLCE_EINVAL);
    check_rejects("ex without options", c.ex(nullptr), FLCE_EWORKSPACE);
  }
  // forward only
  {
    Call c;
    c.reduction = 2;
    check_rejects("fwd none without loss_rows", c.fwd(nullptr), FLCE_EINVAL);
    c.reduction = 0;
    c.h = 24;
    check_rejects("fwd h misaligned", c.fwd(nullptr), FLCE_EINVAL);
    c.h = 16;
    c.H = 12;
    check_rejects("fwd H", c.fwd(nullptr), FLCE_EUNSUPPORTED);
    c.H = 8;
    check_rejects("fwd workspace", c.fwd(nullptr), FLCE_EWORKSPACE);
  }
  // materialised path
  {
    const int before = g_launches;
    expect(flce_logits(P(16), P(16), 4, 8, 8, 0.0f, 1.0f, P(16), 4, nullptr, 0) == FLCE_EINVAL, "logits ld");
    expect(flce_logits(P(16), P(8), 4, 8, 8, 0.0f, 1.0f, P(16), 8, nullptr, 0) == FLCE_EINVAL, "logits W");
    expect(flce_logits(P(16), P(16), 4, 8, 8, nan, 1.0f, P(16), 8, nullptr, 0) == FLCE_EINVAL, "logits T");
    expect(flce_logits(P(16), P(16), 4, 12, 8, 0.0f, 1.0f, P(16), 8, nullptr, 0) == FLCE_EUNSUPPORTED,
           "logits H");
    expect(flce_cross_entropy(P(16), 8, (const int64_t*)P(8), 4, 8, -100, 3, (float*)P(4), nullptr, nullptr, 0,
                              nullptr, 0, P(256), 1 << 20, nullptr) == FLCE_EINVAL,
           "ce reduction");
    expect(flce_cross_entropy(P(16), 8, (const int64_t*)P(8), 4, 8, -100, 0, (float*)P(4), nullptr, nullptr, 0,
                              nullptr, 0, P(256), 64, nullptr) == FLCE_EWORKSPACE,
           "ce workspace");
    expect(g_launches == before, "a rejected materialised call launched");
  }
}

// Valid calls reach the (stubbed) launch with a plan that fits the workspace.
void valid_calls() {
  for (int64_t N : {int64_t(0), int64_t(1), int64_t(255), int64_t(257), int64_t(8192)}) {
    Call c;
    c.N = N;
    c.H = 6656;
    c.V = 202048;
    c.ws_bytes = flce_workspace_size(N, c.H, c.V, 0, 0);
    expect(c.ws_bytes > 0, "workspace size", N);
    const int before = g_launches;
    expect(c.fwd_bwd() == FLCE_OK, "valid call", N);
    expect(g_launches == before + 1, "valid call launched once", N);
    c.ws_bytes = flce_fwd_workspace_size(N, c.H, c.V, 0, 0);
    expect(c.fwd(nullptr) == FLCE_OK, "valid forward-only call", N);
  }
  flce::Header hdr{};
  hdr.status = FLCE_ELABEL;
  expect(flce_read_status(&hdr, nullptr) == FLCE_ELABEL, "read_status");
  expect(flce_read_status(nullptr, nullptr) == FLCE_EINVAL, "read_status null");
  for (int code = -2; code < 12; ++code) expect(flce_strerror(code) != nullptr, "strerror", code);
}

// Seeded sweep of the planner: shapes from tiny to past the limits, budgets
// from tiny to huge.  Every accepted plan must hold its invariants.
void planner_sweep() {
  std::mt19937_64 rng(20241203);
  int ok = 0, small = 0, rejected = 0;
  auto pick = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
  for (int it = 0; it < 20000; ++it) {
    const int dtype = int(pick(0, 1));
    const int64_t N = pick(0, 3) == 0 ? pick(0, 3) : pick(1, int64_t(1) << pick(1, 24)) + (pick(0, 20) == 0 ? (int64_t(1) << 31) : 0);
    const int64_t H = (pick(0, 4) == 0 ? pick(1, 64) : pick(1, 1 << 11)) * (dtype == 0 ? 8 : 4);
    const int64_t V = pick(0, 3) == 0 ? pick(1, 300) : pick(1, int64_t(1) << pick(9, 22));
    const size_t budget = pick(0, 4) == 0 ? 0 : size_t(1) << pick(8, 44);
    flce_plan_t p;
    const int rc = flce_plan(N, H, V, dtype, budget, &p);
    expect(rc == FLCE_OK || rc == FLCE_EWORKSPACE || rc == FLCE_EUNSUPPORTED, "plan code", rc);
    if (rc != FLCE_OK) {
      expect(flce_workspace_size(N, H, V, dtype, budget) == 0, "size of a rejected plan");
      rejected += rc == FLCE_EWORKSPACE;
      continue;
    }
    ++ok;
    small += budget != 0 && p.chunk_rows < (N + 1) / 2 / 256 * 256;
    const int64_t es = dtype == 0 ? 2 : 4;
    expect(budget == 0 || p.workspace_bytes <= budget, "plan over budget", (long long)p.workspace_bytes);
    expect(p.vocab_padded % 256 == 0 && p.vocab_padded >= V && p.vocab_padded - 256 < V, "padded vocabulary");
    expect(p.split_k >= 1 && p.split_k <= 16, "split", p.split_k);
    if (N == 0) {
      expect(p.n_chunks == 0, "empty plan");
      continue;
    }
    expect(p.chunk_rows >= 1 && p.chunk_rows <= (N + 1) / 2 + (N == 1 ? 1 : 0), "chunk rows", p.chunk_rows, N);
    expect(p.n_chunks == (N + p.chunk_rows - 1) / p.chunk_rows, "chunk count", p.n_chunks);
    expect(p.logits_chunk_bytes == size_t(p.chunk_rows) * size_t(p.vocab_padded) * size_t(es), "logits bytes");
    expect(p.grad_W_bytes == size_t(4) * size_t(V) * size_t(H), "grad_W bytes");
    expect(flce_workspace_size(N, H, V, dtype, budget) == p.workspace_bytes, "workspace size agrees");
  }
  std::printf("planner sweep: %d plans (%d shrunk by the budget), %d rejected for the budget\n", ok, small,
              rejected);
  expect(ok > 5000 && small > 300 && rejected > 1000, "sweep coverage", ok, small);
}

}  // namespace

int main() {
  validation_cases();
  valid_calls();
  planner_sweep();
  std::printf("%d launches, %d failed checks\n", g_launches, g_failed);
  return g_failed == 0 ? 0 : 1;
}

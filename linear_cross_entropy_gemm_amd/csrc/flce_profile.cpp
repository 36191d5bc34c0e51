// Per-kernel timing with HIP events on the caller's stream (measurement only).
//
// When enabled, run_call brackets every kernel launch with a pair of events
// recorded on the launch stream.  flce_profile_read synchronises the stream,
// folds the elapsed times into per-kind totals and recycles the events.
#include <mutex>
#include <vector>

#include "flce_internal.hpp"

namespace flce {

namespace {

struct Pending {
  int kind;
  hipEvent_t a, b;
};

struct State {
  std::mutex mu;
  bool on = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[FLCE_KERNEL_KINDS] = {};
  int64_t launches[FLCE_KERNEL_KINDS] = {};
};

State& state() {
  static State s;
  return s;
}

hipEvent_t take_event(State& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool profile_on() { return state().on; }

ProfileScope::ProfileScope(int kind, hipStream_t st) : kind_(kind), st_(st) {
  State& s = state();
  if (!s.on || kind < 0) return;
  std::lock_guard<std::mutex> g(s.mu);
  a_ = take_event(s);
  b_ = take_event(s);
  // a pair that cannot be recorded is not timed: its events go back to the pool
  if (!a_ || !b_ || hipEventRecord(a_, st_) != hipSuccess) {
    if (a_) s.pool.push_back(a_);
    if (b_) s.pool.push_back(b_);
    a_ = b_ = nullptr;
  }
}

ProfileScope::~ProfileScope() {
  if (!a_ || !b_) return;
  State& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (hipEventRecord(b_, st_) != hipSuccess) {
    s.pool.push_back(a_);
    s.pool.push_back(b_);
    return;
  }
  s.pending.push_back({kind_, a_, b_});
}

}  // namespace flce

extern "C" int flce_profile_enable(int on) {
  flce::State& s = flce::state();
  std::lock_guard<std::mutex> g(s.mu);
  s.on = on != 0;
  return FLCE_OK;
}

extern "C" int flce_profile_read(hipStream_t stream, double* total_ms, int64_t* launches, int reset) {
  if (!total_ms || !launches) return FLCE_EINVAL;
  flce::State& s = flce::state();
  if (hipStreamSynchronize(stream) != hipSuccess) return FLCE_EDEVICE;
  std::lock_guard<std::mutex> g(s.mu);
  int rc = FLCE_OK;
  for (auto& p : s.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
      rc = FLCE_EDEVICE;
    } else {
      s.total_ms[p.kind] += ms;
      s.launches[p.kind] += 1;
    }
    s.pool.push_back(p.a);
    s.pool.push_back(p.b);
  }
  s.pending.clear();
  for (int k = 0; k < FLCE_KERNEL_KINDS; ++k) {
    total_ms[k] = s.total_ms[k];
    launches[k] = s.launches[k];
    if (reset) {
      s.total_ms[k] = 0.0;
      s.launches[k] = 0;
    }
  }
  return rc;
}

// Opt-in kernel timing: timing events recorded on the launch stream around each library kernel.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

namespace fsm {

namespace {
using Rec = ProfRec;
std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
// a stack call that fills moe_stack_stats_t collects its own launches here (this thread only)
thread_local std::vector<Rec>* t_sink = nullptr;
}  // namespace

bool prof_on() { return g_on.load(std::memory_order_relaxed); }

ProfScope::ProfScope(int kind, hipStream_t s) : kind_(kind), s_(s), a_(nullptr), b_(nullptr) {
  if (!prof_on() && !t_sink) return;
  if (hipEventCreate(&a_) != hipSuccess) { a_ = nullptr; return; }
  if (hipEventCreate(&b_) != hipSuccess) { (void)hipEventDestroy(a_); a_ = nullptr; b_ = nullptr; return; }
  if (hipEventRecord(a_, s_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    (void)hipEventDestroy(b_);
    a_ = b_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!a_) return;
  if (hipEventRecord(b_, s_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    (void)hipEventDestroy(b_);
    return;
  }
  if (t_sink) {
    t_sink->push_back({kind_, s_, a_, b_});
    return;
  }
  std::lock_guard<std::mutex> g(g_mu);
  g_recs.push_back({kind_, s_, a_, b_});
}

namespace {
// total length of the union of intervals (sorted by start)
double union_len(std::vector<std::pair<double, double>> v) {
  std::sort(v.begin(), v.end());
  double total = 0.0, a = 0.0, b = 0.0;
  bool open = false;
  for (const auto& iv : v) {
    if (!open || iv.first > b) {
      if (open) total += b - a;
      a = iv.first;
      b = iv.second;
      open = true;
    } else if (iv.second > b) {
      b = iv.second;
    }
  }
  return open ? total + (b - a) : 0.0;
}
}  // namespace

StatsScope::StatsScope(moe_stack_stats_t* out, hipStream_t main) : out_(out), main_(main) {
  if (out_) t_sink = &recs_;
}

StatsScope::~StatsScope() {
  if (out_) t_sink = nullptr;
  for (const Rec& r : recs_) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
}

int StatsScope::finish() {
  if (!out_) return MOE_OK;
  t_sink = nullptr;
  *out_ = moe_stack_stats_t{};
  for (const Rec& r : recs_) {
    const hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "stack stats: %s", hipGetErrorString(e));
  }
  std::vector<std::pair<double, double>> m, s, all;
  double lo = 0.0, hi = 0.0;
  for (size_t i = 0; i < recs_.size(); ++i) {
    const Rec& r = recs_[i];
    float t0 = 0.f, t1 = 0.f;
    hipError_t e = hipEventElapsedTime(&t0, recs_[0].a, r.a);
    if (e == hipSuccess) e = hipEventElapsedTime(&t1, recs_[0].a, r.b);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "stack stats: %s", hipGetErrorString(e));
    (r.s == main_ ? m : s).push_back({double(t0), double(t1)});
    all.push_back({double(t0), double(t1)});
    lo = i == 0 ? t0 : std::min(lo, double(t0));
    hi = i == 0 ? t1 : std::max(hi, double(t1));
  }
  const double um = union_len(m), us = union_len(s), ua = union_len(all);
  out_->wall_ms = hi - lo;
  out_->main_busy_ms = um;
  out_->side_busy_ms = us;
  out_->overlap_ms = std::max(0.0, um + us - ua);   // |M n S| = |M| + |S| - |M u S|
  out_->overlap_of_side = us > 0.0 ? out_->overlap_ms / us : 0.0;
  out_->overlap_of_main = um > 0.0 ? out_->overlap_ms / um : 0.0;
  out_->launches_main = int32_t(m.size());
  out_->launches_side = int32_t(s.size());
  return MOE_OK;
}

}  // namespace fsm

extern "C" {

int moe_profile_enable(int on) {
  fsm::g_on.store(on != 0);
  return MOE_OK;
}

int moe_profile_collect_intervals(moe_kernel_time_t* out, moe_kernel_interval_t* iv, int32_t cap, int32_t* n) {
  if (!out || !n || (cap > 0 && !iv))
    return fsm::fail(MOE_ERR_INVALID_ARG, "moe_profile_collect_intervals: out, n (and iv with cap > 0) are required");
  for (int i = 0; i < MOE_KERNEL_KINDS; ++i) out[i] = moe_kernel_time_t{0, 0.0};
  std::vector<fsm::Rec> recs;
  {
    std::lock_guard<std::mutex> g(fsm::g_mu);
    recs.swap(fsm::g_recs);
  }
  *n = int32_t(recs.size());
  int rc = MOE_OK;
  // every end event has completed once the last one of each stream has; wait for all of them
  for (const fsm::Rec& r : recs) {
    if (rc != MOE_OK) break;
    const hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) rc = fsm::fail(MOE_ERR_HIP, "moe_profile_collect: %s", hipGetErrorString(e));
  }
  for (size_t i = 0; i < recs.size() && rc == MOE_OK; ++i) {
    const fsm::Rec& r = recs[i];
    float ms = 0.f, t0 = 0.f, t1 = 0.f;
    hipError_t e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e == hipSuccess && int64_t(i) < cap) {
      e = hipEventElapsedTime(&t0, recs[0].a, r.a);
      if (e == hipSuccess) e = hipEventElapsedTime(&t1, recs[0].a, r.b);
    }
    if (e != hipSuccess) {
      rc = fsm::fail(MOE_ERR_HIP, "moe_profile_collect: %s", hipGetErrorString(e));
      break;
    }
    if (r.kind >= 0 && r.kind < MOE_KERNEL_KINDS) {
      out[r.kind].count += 1;
      out[r.kind].total_ms += ms;
    }
    if (int64_t(i) < cap)
      iv[i] = moe_kernel_interval_t{r.kind, 0, uint64_t(reinterpret_cast<uintptr_t>(r.s)), double(t0), double(t1)};
  }
  for (const fsm::Rec& r : recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  return rc;
}

int moe_profile_collect(moe_kernel_time_t* out) {
  if (!out) return fsm::fail(MOE_ERR_INVALID_ARG, "moe_profile_collect: out is required");
  int32_t n = 0;
  return moe_profile_collect_intervals(out, nullptr, 0, &n);
}

}  // extern "C"

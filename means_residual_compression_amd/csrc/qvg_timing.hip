// Opt-in per-kernel launch timing: when enabled, every kernel launch of the
// library is bracketed by two HIP events recorded on the launch stream, and
// qvg_timing_read() sums the elapsed times per kernel name.  Disabled (the
// default) it costs one relaxed atomic load per launch.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "qvg.h"
#include "qvg_internal.h"

namespace qvg {
namespace {
std::atomic<bool> g_on{false};
std::mutex g_mu;
struct Entry {
  const char *name;
  hipEvent_t a, b;
};
std::vector<Entry> g_entries;
std::vector<hipEvent_t> g_pool;
size_t g_used = 0;

hipEvent_t take_event() {
  if (g_used == g_pool.size()) {
    hipEvent_t e = nullptr;
    // timing-only events: no system-scope fence (cache write-back and
    // invalidate) when they are recorded, so they barely perturb the work
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_used++];
}
}  // namespace

TimerScope::TimerScope(const char *name, hipStream_t s) : name_(name), s_(s), a_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = take_event();
  if (a_) (void)hipEventRecord(a_, s_);
}

TimerScope::~TimerScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (!b) return;
  (void)hipEventRecord(b, s_);
  g_entries.push_back({name_, a_, b});
}

}  // namespace qvg

extern "C" {

void qvg_timing_enable(int on) { qvg::g_on.store(on != 0); }

void qvg_timing_reset(void) {
  std::lock_guard<std::mutex> lk(qvg::g_mu);
  for (auto &e : qvg::g_entries) (void)hipEventSynchronize(e.b);
  qvg::g_entries.clear();
  qvg::g_used = 0;
}

int64_t qvg_timing_read(const char *kernel, double *total_ms) {
  std::lock_guard<std::mutex> lk(qvg::g_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (auto &e : qvg::g_entries) {
    if (std::string(e.name) != kernel) continue;
    if (hipEventSynchronize(e.b) != hipSuccess) return -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) return -1;
    sum += ms;
    ++n;
  }
  if (total_ms) *total_ms = sum;
  return n;
}

}  // extern "C"

// Per-kernel event timing (see timing.h) and its C entry points.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "mla.h"
#include "timing.h"

namespace mla {
namespace {

struct Pending {
  std::string name;
  hipEvent_t start, stop;
};
struct Total {
  std::string name;
  double ms;
  long launches;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<Total> g_totals;

void drain_locked() {
  for (auto& p : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      bool found = false;
      for (auto& t : g_totals)
        if (t.name == p.name) {
          t.ms += ms;
          t.launches += 1;
          found = true;
        }
      if (!found) g_totals.push_back({p.name, static_cast<double>(ms), 1});
    }
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
}

}  // namespace

bool timing_enabled() { return g_on.load(std::memory_order_relaxed); }

hipEvent_t timing_begin(const char* kernel, hipStream_t st) {
  if (!timing_enabled()) return nullptr;
  Pending p{kernel, nullptr, nullptr};
  if (hipEventCreate(&p.start) != hipSuccess) return nullptr;
  if (hipEventCreate(&p.stop) != hipSuccess) {
    (void)hipEventDestroy(p.start);
    return nullptr;
  }
  (void)hipEventRecord(p.start, st);
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back(p);
  return p.stop;
}

}  // namespace mla

extern "C" {

void mla_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(mla::g_mu);
  mla::drain_locked();
  mla::g_totals.clear();
  mla::g_on.store(on != 0, std::memory_order_relaxed);
}

int32_t mla_timing_read(const char* kernel, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(mla::g_mu);
  mla::drain_locked();
  for (auto& t : mla::g_totals)
    if (t.name == kernel) {
      if (total_ms) *total_ms = t.ms;
      if (launches) *launches = t.launches;
      return 1;
    }
  if (total_ms) *total_ms = 0.0;
  if (launches) *launches = 0;
  return 0;
}

}  // extern "C"

// msa_timing.hip -- optional per-kernel timing: while a measurement harness
// has it switched on, every launch of a timed kernel kind is bracketed by two
// HIP events recorded on the stream the kernel is launched on, and the
// elapsed times are summed per kind when the harness reads them.  Off (the
// default), a launch pays one relaxed atomic load.
#include "msa_internal.h"

#include <atomic>
#include <mutex>
#include <vector>

namespace msa {
namespace {

struct Rec {
  int kind;
  size_t ev;  // index of the start event; the stop event follows it
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<hipEvent_t> g_ev;
std::vector<Rec> g_recs;
int64_t g_dropped = 0;

}  // namespace

bool timing_enabled() { return g_on.load(std::memory_order_relaxed); }

int timing_open(int kind, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load(std::memory_order_relaxed)) return -1;
  const size_t i = 2 * g_recs.size();
  if (i + 2 > g_ev.size()) {
    ++g_dropped;
    return -1;
  }
  if (hipEventRecord(g_ev[i], st) != hipSuccess) {
    ++g_dropped;
    return -1;
  }
  g_recs.push_back(Rec{kind, i});
  return static_cast<int>(i);
}

void timing_close(int slot, hipStream_t st) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (static_cast<size_t>(slot) + 1 < g_ev.size()) (void)hipEventRecord(g_ev[slot + 1], st);
}

hipError_t timing_start(int64_t max_launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_on.load()) return hipErrorInvalidValue;
  g_ev.assign(static_cast<size_t>(2 * max_launches), nullptr);
  for (size_t i = 0; i < g_ev.size(); ++i) {
    const hipError_t e = hipEventCreate(&g_ev[i]);
    if (e != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(g_ev[j]);
      g_ev.clear();
      return e;
    }
  }
  g_recs.clear();
  g_dropped = 0;
  g_on.store(true);
  return hipSuccess;
}

hipError_t timing_stop(double* ms, int64_t* launches, int nkinds, int64_t* dropped) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on.load()) return hipErrorInvalidValue;
  g_on.store(false);
  for (int k = 0; k < nkinds; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  hipError_t err = hipSuccess;
  for (const Rec& r : g_recs) {
    hipError_t e = hipEventSynchronize(g_ev[r.ev + 1]);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, g_ev[r.ev], g_ev[r.ev + 1]);
    if (e != hipSuccess) {
      if (err == hipSuccess) err = e;
      continue;
    }
    if (r.kind >= 0 && r.kind < nkinds) {
      ms[r.kind] += t;
      ++launches[r.kind];
    }
  }
  for (hipEvent_t e : g_ev) (void)hipEventDestroy(e);
  g_ev.clear();
  g_recs.clear();
  *dropped = g_dropped;
  return err;
}

}  // namespace msa

// Status strings, last HIP error, device properties.
#include <cstring>
#include <mutex>
#include <vector>

#include "lrc_internal.h"

namespace lrc {

static thread_local int g_last_hip_error = 0;

void set_last_hip_error(hipError_t e) { g_last_hip_error = int(e); }

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = v;
  return v;
}

// ---- measurement support
namespace {
struct ProfEvent {
  const char* name;
  hipEvent_t e0, e1;
};
struct ProfTotal {
  const char* name;
  int64_t launches = 0;
  double ms = 0.0, flops = 0.0, bytes = 0.0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfEvent> g_prof_events;
std::vector<ProfTotal> g_prof_totals;
std::vector<hipEvent_t> g_prof_pool;  // recorded events are recycled after lrc_profile_stop

hipEvent_t acquire_event() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

ProfTotal& total_for(const char* name) {
  for (auto& t : g_prof_totals)
    if (std::strcmp(t.name, name) == 0) return t;
  g_prof_totals.push_back(ProfTotal{name});
  return g_prof_totals.back();
}
}  // namespace

bool prof_enabled() { return g_prof_on; }

void prof_add_work(const char* name, double flops, double bytes) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  ProfTotal& t = total_for(name);
  t.flops += flops;
  t.bytes += bytes;
}

ProfScope::ProfScope(const char* n, hipStream_t s, double f, double b) : name(n), st(s), flops(f), bytes(b) {
  if (!g_prof_on) return;
  e0 = acquire_event();
  if (e0) (void)hipEventRecord(e0, st);
}

ProfScope::~ProfScope() {
  if (!e0) return;
  hipEvent_t e1 = acquire_event();
  if (!e1) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pool.push_back(e0);
    return;
  }
  (void)hipEventRecord(e1, st);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_events.push_back(ProfEvent{name, e0, e1});
  ProfTotal& t = total_for(name);
  t.launches += 1;
  t.flops += flops;
  t.bytes += bytes;
}

ProfKernel::ProfKernel(const char* n, double f, double b) : name(n), flops(f), bytes(b) {
  if (!g_prof_on) return;
  start = acquire_event();
  stop = acquire_event();
  if (!start || !stop) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (start) g_prof_pool.push_back(start);
    if (stop) g_prof_pool.push_back(stop);
    start = stop = nullptr;
  }
}

ProfKernel::~ProfKernel() {
  if (!start) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_events.push_back(ProfEvent{name, start, stop});
  ProfTotal& t = total_for(name);
  t.launches += 1;
  t.flops += flops;
  t.bytes += bytes;
}

}  // namespace lrc

extern "C" lrc_status lrc_profile_start(void) {
  std::lock_guard<std::mutex> lk(lrc::g_prof_mu);
  for (auto& e : lrc::g_prof_events) {
    lrc::g_prof_pool.push_back(e.e0);
    lrc::g_prof_pool.push_back(e.e1);
  }
  lrc::g_prof_events.clear();
  lrc::g_prof_totals.clear();
  lrc::g_prof_on = true;
  return LRC_OK;
}

extern "C" lrc_status lrc_profile_stop(void) {
  std::lock_guard<std::mutex> lk(lrc::g_prof_mu);
  lrc::g_prof_on = false;
  // every recorded pair goes back to the pool exactly once and the list is cleared, also
  // when an event reports an error (the first error is returned; later pairs still count)
  hipError_t first = hipSuccess;
  for (auto& e : lrc::g_prof_events) {
    hipError_t r = hipEventSynchronize(e.e1);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, e.e0, e.e1);
    if (r == hipSuccess)
      lrc::total_for(e.name).ms += ms;
    else if (first == hipSuccess)
      first = r;
    lrc::g_prof_pool.push_back(e.e0);
    lrc::g_prof_pool.push_back(e.e1);
  }
  lrc::g_prof_events.clear();
  if (first != hipSuccess) {
    lrc::set_last_hip_error(first);
    return LRC_EHIP;
  }
  return LRC_OK;
}

extern "C" int lrc_profile_kernels(void) { return int(lrc::g_prof_totals.size()); }

extern "C" lrc_status lrc_profile_kernel(int index, const char** name, int64_t* launches, double* total_ms,
                                         double* flops, double* bytes) {
  if (index < 0 || index >= int(lrc::g_prof_totals.size())) return LRC_EINVAL;
  const auto& t = lrc::g_prof_totals[size_t(index)];
  if (name) *name = t.name;
  if (launches) *launches = t.launches;
  if (total_ms) *total_ms = t.ms;
  if (flops) *flops = t.flops;
  if (bytes) *bytes = t.bytes;
  return LRC_OK;
}

extern "C" const char* lrc_status_string(lrc_status s) {
  switch (s) {
    case LRC_OK: return "LRC_OK";
    case LRC_EINVAL: return "LRC_EINVAL: invalid argument";
    case LRC_EDTYPE: return "LRC_EDTYPE: unsupported dtype or flags";
    case LRC_EWORKSPACE: return "LRC_EWORKSPACE: workspace missing or too small";
    case LRC_EHIP: return "LRC_EHIP: HIP runtime error";
    case LRC_ENOTPD: return "LRC_ENOTPD: covariance not positive definite";
    case LRC_ENOCONV: return "LRC_ENOCONV: eigensolver did not converge";
    case LRC_ENONFINITE: return "LRC_ENONFINITE: non-finite value";
  }
  return "unknown lrc_status";
}

extern "C" int lrc_last_hip_error(void) { return lrc::g_last_hip_error; }

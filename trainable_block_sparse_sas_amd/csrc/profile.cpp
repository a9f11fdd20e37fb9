// Kernel timing for diagnostics.  While enabled, ProfScope records a HIP event
// on the launch stream before and after each kernel; sas_profile_read waits
// for the recorded events, sums the durations per kernel name and clears the
// record.  Disabled (the default), a launch costs one relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/sas.h"
#include "internal.h"

namespace sas {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;

hipEvent_t new_event() {
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  a_ = new_event();
  if (a_ && hipEventRecord(a_, s_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    a_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!a_) return;
  hipEvent_t b = new_event();
  if (!b || hipEventRecord(b, s_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    if (b) (void)hipEventDestroy(b);
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back({name_, a_, b});
}

}  // namespace sas

extern "C" {

int sas_profile_enable(int on) {
  sas::g_on.store(on != 0);
  return SAS_OK;
}

int sas_profile_read(int max_entries, char* names, int name_bytes, double* ms, int* counts) {
  if (max_entries < 0 || name_bytes < 1 || (max_entries > 0 && (!names || !ms || !counts)))
    return SAS_EINVAL;
  std::vector<sas::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(sas::g_mu);
    recs.swap(sas::g_recs);
  }
  std::vector<const char*> keys;
  std::vector<double> tot;
  std::vector<int> cnt;
  int status = SAS_OK;
  for (const auto& r : recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      status = SAS_EHIP;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    size_t i = 0;
    while (i < keys.size() && std::strcmp(keys[i], r.name) != 0) ++i;
    if (i == keys.size()) {
      keys.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += t;
    cnt[i] += 1;
  }
  if (status != SAS_OK) return status;
  const int n = int(keys.size());
  for (int i = 0; i < n && i < max_entries; ++i) {
    std::strncpy(names + size_t(i) * name_bytes, keys[i], name_bytes - 1);
    names[size_t(i) * name_bytes + name_bytes - 1] = '\0';
    ms[i] = tot[i];
    counts[i] = cnt[i];
  }
  return n;
}

}  // extern "C"

// Opt-in per-launch timing: when enabled, every kernel launch of the library is bracketed by a
// pair of hipEvents recorded on the launch stream, and csa_profile_stop() returns the summed
// event time per kernel name.  Off by default; when off a ProfScope does nothing.
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kernels.h"

namespace csa {

namespace {
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), stream_(s), a_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  a_ = take_event();
  if (a_) hipEventRecord(static_cast<hipEvent_t>(a_), s);
}

ProfScope::~ProfScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (!b) return;
  hipEventRecord(b, stream_);
  g_recs.push_back(Rec{name_, static_cast<hipEvent_t>(a_), b});
}

int profile_start() {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    g_free.push_back(r.a);
    g_free.push_back(r.b);
  }
  g_recs.clear();
  g_on = true;
  return 0;
}

int profile_stop(ProfTotal* out, int max, int* n) {
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = false;
    recs.swap(g_recs);
  }
  std::vector<ProfTotal> tot;
  hipError_t err = hipSuccess;
  for (auto& r : recs) {
    if (err == hipSuccess) err = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.a, r.b);
    size_t i = 0;
    for (; i < tot.size(); ++i)
      if (std::strcmp(tot[i].name, r.name) == 0) break;
    if (i == tot.size()) {
      ProfTotal t{};
      std::strncpy(t.name, r.name, sizeof(t.name) - 1);
      tot.push_back(t);
    }
    tot[i].launches += 1;
    tot[i].total_ms += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& r : recs) {
      g_free.push_back(r.a);
      g_free.push_back(r.b);
    }
  }
  const int cnt = static_cast<int>(tot.size()) < max ? static_cast<int>(tot.size()) : max;
  for (int i = 0; i < cnt; ++i) out[i] = tot[i];
  *n = cnt;
  return err == hipSuccess ? 0 : -1;
}

hipError_t ensure_max_lds(const void* fn, size_t bytes) {
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> set;
  std::lock_guard<std::mutex> lk(mu);
  auto it = set.find(fn);
  if (it != set.end() && it->second >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(bytes));
  if (e == hipSuccess) set[fn] = bytes;
  return e;
}

}  // namespace csa

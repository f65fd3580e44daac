// Opt-in per-kernel timing: hipEvent pairs around every library launch, reduced to
// per-kernel-name totals on demand.
#include "profile.h"

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dflash.h"

namespace dflash {
namespace {

struct Pending {
  const char *name;
  hipEvent_t start, end;
};
struct Total {
  const char *name;
  int64_t launches;
  double ms;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<Total> g_totals;
std::vector<hipEvent_t> g_free;
std::vector<std::string> g_filter;  // empty: every launch

bool selected(const char *name) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_filter.empty()) return true;
  for (const std::string &f : g_filter)
    if (f == name) return true;
  return false;
}

hipEvent_t take_event() {
  std::lock_guard<std::mutex> lk(g_mu);
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

bool profile_enabled() { return g_enabled.load(std::memory_order_relaxed); }

ProfScope::ProfScope(const char *name, hipStream_t stream) : name_(name), stream_(stream) {
  if (!profile_enabled() || !selected(name)) return;
  start_ = take_event();
  if (start_ && hipEventRecord(start_, stream_) != hipSuccess) start_ = nullptr;
}

ProfScope::~ProfScope() {
  if (!start_) return;
  hipEvent_t end = take_event();
  if (!end || hipEventRecord(end, stream_) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({name_, start_, end});
}

}  // namespace dflash

using namespace dflash;

extern "C" {

dflash_status dflash_profile_enable(int32_t on) {
  g_enabled.store(on != 0);
  return DFLASH_OK;
}

dflash_status dflash_profile_filter(const char *names) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_filter.clear();
  if (!names) return DFLASH_OK;
  std::string cur;
  for (const char *c = names;; ++c) {
    if (*c == ',' || *c == '\0') {
      if (!cur.empty()) g_filter.push_back(cur);
      cur.clear();
      if (*c == '\0') break;
    } else {
      cur += *c;
    }
  }
  return DFLASH_OK;
}

dflash_status dflash_profile_collect(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  dflash_status st = DFLASH_OK;
  for (const Pending &p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.end) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.end) != hipSuccess) {
      st = DFLASH_ERR_HIP;
    } else {
      bool found = false;
      for (Total &t : g_totals)
        if (strcmp(t.name, p.name) == 0) {
          t.launches += 1;
          t.ms += ms;
          found = true;
          break;
        }
      if (!found) g_totals.push_back({p.name, 1, ms});
    }
    g_free.push_back(p.start);
    g_free.push_back(p.end);
  }
  g_pending.clear();
  return st;
}

void dflash_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_totals.clear();
}

int32_t dflash_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int32_t)g_totals.size();
}

dflash_status dflash_profile_entry(int32_t i, const char **name, int64_t *launches, double *total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int32_t)g_totals.size() || !name || !launches || !total_ms) return DFLASH_ERR_INVALID_ARGUMENT;
  *name = g_totals[i].name;
  *launches = g_totals[i].launches;
  *total_ms = g_totals[i].ms;
  return DFLASH_OK;
}

}  // extern "C"

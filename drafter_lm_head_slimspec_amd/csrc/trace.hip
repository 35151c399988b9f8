// Opt-in per-kernel timing: when enabled, every launch made by the library is bracketed by
// two events recorded on the launch stream; sh_trace_read() waits for them and reports the
// per-kernel-name count and total / min / max durations.  Disabled by default (no events).
#include <algorithm>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spechead.h"
#include "trace.h"

namespace sh {
namespace {

struct Rec {
  const char* name;
  int a, b;  // indices into the event pool
};

std::mutex g_mu;
std::vector<hipEvent_t> g_pool;
std::vector<Rec> g_recs;
size_t g_next = 0;
bool g_on = false;

}  // namespace

TraceScope::TraceScope(const char* name, hipStream_t st, bool by_launch)
    : name_(name), st_(st), idx_(-1), by_launch_(by_launch) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_next + 2 > g_pool.size()) return;
  idx_ = static_cast<int>(g_next);
  g_next += 2;
  if (!by_launch_) (void)hipEventRecord(g_pool[idx_], st_);
}

TraceScope::~TraceScope() {
  if (idx_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!by_launch_) (void)hipEventRecord(g_pool[idx_ + 1], st_);
  g_recs.push_back(Rec{name_, idx_, idx_ + 1});
}

hipEvent_t TraceScope::start() const { return idx_ < 0 ? nullptr : g_pool[idx_]; }
hipEvent_t TraceScope::stop() const { return idx_ < 0 ? nullptr : g_pool[idx_ + 1]; }

}  // namespace sh

extern "C" {

int sh_trace_enable(int64_t max_records) {
  std::lock_guard<std::mutex> lk(sh::g_mu);
  for (hipEvent_t e : sh::g_pool) (void)hipEventDestroy(e);
  sh::g_pool.clear();
  sh::g_recs.clear();
  sh::g_next = 0;
  sh::g_on = false;
  if (max_records <= 0) return SH_OK;
  if (max_records > (int64_t{1} << 20)) return SH_ERR_PARAM;
  sh::g_pool.resize(static_cast<size_t>(2 * max_records));
  for (auto& e : sh::g_pool) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      return SH_ERR_HIP;
    }
  }
  sh::g_on = true;
  return SH_OK;
}

int sh_trace_read(char* buf, size_t bytes) {
  std::lock_guard<std::mutex> lk(sh::g_mu);
  struct Agg {
    long n = 0;
    double tot = 0, mn = 1e300, mx = 0;
  };
  std::map<std::string, Agg> agg;
  for (const auto& r : sh::g_recs) {
    if (hipEventSynchronize(sh::g_pool[r.b]) != hipSuccess) return SH_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, sh::g_pool[r.a], sh::g_pool[r.b]) != hipSuccess) return SH_ERR_HIP;
    Agg& a = agg[r.name];
    const double us = 1000.0 * ms;
    a.n += 1;
    a.tot += us;
    a.mn = std::min(a.mn, us);
    a.mx = std::max(a.mx, us);
  }
  sh::g_recs.clear();
  sh::g_next = 0;
  std::string out = "{";
  bool first = true;
  for (const auto& kv : agg) {
    char line[256];
    snprintf(line, sizeof(line), "%s\"%s\": {\"count\": %ld, \"total_us\": %.3f, \"min_us\": %.3f, \"max_us\": %.3f}",
             first ? "" : ", ", kv.first.c_str(), kv.second.n, kv.second.tot, kv.second.mn, kv.second.mx);
    out += line;
    first = false;
  }
  out += "}";
  if (buf == nullptr || bytes < out.size() + 1) return SH_ERR_PARAM;
  std::copy(out.begin(), out.end(), buf);
  buf[out.size()] = '\0';
  return SH_OK;
}

}  // extern "C"

// Internal: RAII bracket of one kernel launch for the opt-in timing facility.
#pragma once

#include <hip/hip_runtime.h>

namespace sh {

// by_launch: the launch itself stamps the two events (hipExtLaunchKernelGGL with start() and
// stop()), so the interval is the kernel's own execution; otherwise the scope records them on
// the stream before and after the launch (which adds the dispatch gap).
class TraceScope {
 public:
  TraceScope(const char* name, hipStream_t st, bool by_launch = false);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;
  hipEvent_t start() const;   // nullptr when tracing is off
  hipEvent_t stop() const;

 private:
  const char* name_;
  hipStream_t st_;
  int idx_;
  bool by_launch_;
};

}  // namespace sh

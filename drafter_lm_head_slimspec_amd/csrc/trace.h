// Internal: RAII bracket of one kernel launch for the opt-in timing facility.
#pragma once

#include <hip/hip_runtime.h>

namespace sh {

class TraceScope {
 public:
  TraceScope(const char* name, hipStream_t st);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  int idx_;
};

}  // namespace sh

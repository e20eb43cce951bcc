// Optional per-kernel timing: when enabled on the calling thread, every
// kernel launch of the library is bracketed by a pair of hipEvents recorded
// on the launch stream.  Aggregation happens on request (msa_profile_collect).
#pragma once
#include <hip/hip_runtime.h>

namespace msa {

bool prof_enabled();
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

struct ProfScope {
  hipStream_t s;
  bool on;
  ProfScope(const char* name, hipStream_t st) : s(st), on(prof_enabled()) {
    if (on) prof_begin(name, s);
  }
  ~ProfScope() {
    if (on) prof_end(s);
  }
};

}  // namespace msa

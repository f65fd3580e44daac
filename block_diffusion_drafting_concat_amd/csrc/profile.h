// Opt-in per-kernel timing with hipEvents (see dflash_profile_* in include/dflash.h).
#pragma once

#include <hip/hip_runtime.h>

namespace dflash {

bool profile_enabled();

// Brackets one kernel launch: records a start event on construction and an end event on
// destruction, both on `stream`, when profiling is enabled; does nothing otherwise.
class ProfScope {
 public:
  ProfScope(const char *name, hipStream_t stream);
  ~ProfScope();
  ProfScope(const ProfScope &) = delete;
  ProfScope &operator=(const ProfScope &) = delete;

 private:
  const char *name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

}  // namespace dflash

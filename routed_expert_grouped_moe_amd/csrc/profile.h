// RAII bracket of one launch for the opt-in per-stage timing (moe_profile_enable).
#pragma once

#include "moe_internal.h"

namespace moe {

class MOE_HIDDEN ProfScope {
 public:
  ProfScope(int stage, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  int stage_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};

}  // namespace moe

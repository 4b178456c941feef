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

// Device counters of the stage's sampled clocks while profiling is on (else NULL): [0] sums
// core-clock ticks (s_memtime) and [1] real-time ticks (s_memrealtime, 100 MHz) that thread 0
// of each workgroup of the stage's GEMM kernels spent between its start and its last store.
MOE_HIDDEN unsigned long long* prof_clock(int stage);

}  // namespace moe

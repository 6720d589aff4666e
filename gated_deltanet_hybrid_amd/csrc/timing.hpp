// Scoped HIP-event bracket around one kernel launch; records nothing unless timing was
// enabled with hla_timing_enable().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hla.h"

namespace hla {

class TimedLaunch {
 public:
  TimedLaunch(int32_t which, hipStream_t s);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  int32_t which_;
  hipStream_t stream_;
  hipEvent_t start_{}, stop_{};
  bool active_ = false;
};

}  // namespace hla

// Internal hooks of the opt-in per-kernel timing (profile.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace swattn {

enum KernelId {
  K_FWD_PREP = 0,
  K_FWD = 1,
  K_BWD_KSCALE = 2,
  K_BWD_DKDV = 3,
  K_BWD_DQ = 4,
  K_BWD_GATE = 5,   // the two gate-gradient kernels of the value-embedding gate
  kNumKernels = 6
};

struct ProfToken {
  int kernel;  // -1: not recording
  hipEvent_t start, stop;
  hipStream_t stream;
};

ProfToken prof_begin(int kernel, hipStream_t stream);
void prof_end(const ProfToken& t);

}  // namespace swattn

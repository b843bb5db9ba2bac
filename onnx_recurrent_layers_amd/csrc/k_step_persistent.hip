// k_step_persistent.hip -- stage 3 as one cooperative launch (placeholder).
#include "cells.h"

namespace rnnhip {

bool persistent_supported(const Problem&, int*, int*, int*) { return false; }

hipError_t launch_step_persistent(const StepArgs&, const Problem&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace rnnhip

// k_step_launch.hip -- stage 3 of a layer as one kernel launch per step
// ("Recurrent layers" page, "How a layer runs", item 3): the recurrent product
// rec = R[d] . h_prev of every active (direction, batch row), fused with the
// gate arithmetic of cells.h.  A GRU with linear_before_reset = 0 takes two
// launches per step, because its candidate product needs r*h of every unit.
//
// One wave64 per (direction, hidden unit, block of 8 batch rows) covers all
// gate rows of that unit, so the gate arithmetic stays in the wave.  Lanes walk
// k = lane, lane+64, ... in increasing order and the 64 partial sums are
// combined by a fixed xor butterfly: the summation order depends only on the
// shapes, never on scheduling (no atomics), so runs are bit-identical.
// Rows whose sequence has ended are skipped: their h stays in the state slot
// of their last step, and nothing reads it again.  Each step writes Y (and,
// after a row's last step, Y_h / Y_c) itself.
#include "step_wave.h"

namespace rnnhip {

template <typename T>
__global__ __launch_bounds__(64) void step_launch_kernel(StepArgs a, int s, int phase) {
  step_wave<T>(a, s, phase, blockIdx.x, blockIdx.y * kRows, blockIdx.z, threadIdx.x);
}

int step_generic_launches_per_step(const StepArgs& a) { return (a.cell == RNN_CELL_GRU && !a.lbr) ? 2 : 1; }

hipError_t launch_step_generic(const StepArgs& a, int step, hipStream_t s) {
  const dim3 grid(unsigned(a.H), unsigned((a.B + kRows - 1) / kRows), unsigned(a.D));
  if (grid.y > 65535) return hipErrorInvalidValue;
  const int phases = step_generic_launches_per_step(a);
  for (int ph = 0; ph < phases; ++ph) {
    if (a.dtype == RNN_DTYPE_F32)
      hipLaunchKernelGGL(step_launch_kernel<float>, grid, dim3(64), 0, s, a, step, ph);
    else
      hipLaunchKernelGGL(step_launch_kernel<half_t>, grid, dim3(64), 0, s, a, step, ph);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rnnhip

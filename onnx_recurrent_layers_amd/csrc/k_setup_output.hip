// k_setup_output.hip -- stage 2 (state setup) of a layer ("Recurrent layers"
// page, "How a layer runs") as a launch of its own, used when there is no
// projection to carry it (Seq = 0).  Stage 4 (the outputs) needs no pass of
// its own: each step writes Y and, after a row's last step, Y_h / Y_c, and
// the setup writes the outputs no step writes under the page's "Semantics"
// rules (Y zero past a row's length, zero final states for a row of length 0,
// the initial states when Seq = 0).
#include "device_common.h"

namespace rnnhip {

template <typename T>
__global__ void setup_kernel(SetupArgs a) {
  setup_state<T>(a, int(blockIdx.x), int(gridDim.x));
}

// R of f32 layers as bf16 hi and lo planes for the bf16 matrix cores of the
// per-step product (the planes are read there instead of R).
__global__ void split_r_kernel(const float* R, unsigned short* out, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    split_bf16_bits(R[i], out[i], out[n + i]);
}

static int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65536) g = 65536;
  return int(g < 1 ? 1 : g);
}

hipError_t launch_setup(const SetupArgs& a, hipStream_t s) {
  const int64_t n = int64_t(a.D) * a.B * a.H;
  if (n == 0) return hipSuccess;
  if (a.dtype == RNN_DTYPE_F32)
    hipLaunchKernelGGL(setup_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(setup_kernel<half_t>, dim3(grid_for(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_r(const void* R, unsigned short* rsplit, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(split_r_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, static_cast<const float*>(R), rsplit, n);
  return hipGetLastError();
}

}  // namespace rnnhip

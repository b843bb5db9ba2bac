// k_setup_output.hip -- stage 2 (state setup) and stage 4 (output passes) of a
// layer ("Recurrent layers" page, "How a layer runs"), with the page's
// "Semantics" rules for the outputs: Y is zero at steps past a row's length,
// Y_h / Y_c are the state after the row's last valid step, a row of length 0
// has zero final states, and Seq = 0 gives the initial states.
#include "device_common.h"

namespace rnnhip {

template <typename T>
__global__ void setup_kernel(SetupArgs a) {
  setup_state<T>(a, int(blockIdx.x), int(gridDim.x));
}

template <typename T>
__global__ void output_kernel(OutputArgs a) {
  const int64_t DBH = int64_t(a.D) * a.B * a.H;
  const int64_t nY = a.Y ? int64_t(a.S) * DBH : 0;
  const int64_t nH = a.Y_h ? DBH : 0;
  const int64_t nC = a.Y_c ? DBH : 0;
  const int64_t total = nY + nH + nC;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    if (i < nY) {
      int64_t j = i % a.H, b, d, t;
      if (a.layout == 0) {  // [S, D, B, H]
        b = (i / a.H) % a.B;
        d = (i / (int64_t(a.H) * a.B)) % a.D;
        t = i / DBH;
      } else {              // [B, S, D, H]
        d = (i / a.H) % a.D;
        t = (i / (int64_t(a.H) * a.D)) % a.S;
        b = i / (int64_t(a.H) * a.D * a.S);
      }
      const int L = row_length(a.lens, int(b), a.S, a.steps);
      float v = 0.f;
      if (t < L) {
        const int64_t s = a.dir_reverse[d] ? (L - 1 - t) : t;
        v = a.slab[(s + 1) * DBH + (d * a.B + b) * a.H + j];
      }
      static_cast<T*>(a.Y)[i] = to_elem<T>(v);
    } else {
      const int64_t k = i - nY;
      const bool is_h = k < nH;
      const int64_t e = is_h ? k : k - nH;     // index in the output's own layout
      const int64_t j = e % a.H;
      int64_t b, d;
      if (a.layout == 0) {  // [D, B, H]
        b = (e / a.H) % a.B;
        d = e / (int64_t(a.H) * a.B);
      } else {              // [B, D, H]
        d = (e / a.H) % a.D;
        b = e / (int64_t(a.H) * a.D);
      }
      const int64_t sidx = (d * a.B + b) * a.H + j;
      float v;
      if (a.S == 0) {
        v = is_h ? a.slab[sidx] : a.cell_state[sidx];
      } else {
        const int L = row_length(a.lens, int(b), a.S, a.steps);
        v = L == 0 ? 0.f : (is_h ? a.slab[int64_t(L) * DBH + sidx] : a.cell_state[sidx]);
      }
      static_cast<T*>(is_h ? a.Y_h : a.Y_c)[e] = to_elem<T>(v);
    }
  }
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

hipError_t launch_output(const OutputArgs& a, hipStream_t s) {
  const int64_t DBH = int64_t(a.D) * a.B * a.H;
  const int64_t n = (a.Y ? int64_t(a.S) * DBH : 0) + (a.Y_h ? DBH : 0) + (a.Y_c ? DBH : 0);
  if (n == 0) return hipSuccess;
  if (a.dtype == RNN_DTYPE_F32)
    hipLaunchKernelGGL(output_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(output_kernel<half_t>, dim3(grid_for(n, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rnnhip

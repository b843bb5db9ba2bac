// k_projection.hip -- stage 1 of a layer ("Recurrent layers" page, "How a
// layer runs", item 1): the input projection of every step and direction as
// one batched matrix product Xw[d] = X . W[d]^T (W read as stored, [G*H, I],
// i.e. the transposed-B form), f32 accumulation.  No bias is added here: the
// biases enter the gate sum in the page's fixed order.
//
// MI355X design: 128x128 output tiles per 256-thread workgroup (four wave64s,
// 64x64 each as 2x2 blocks of 32x32 MFMA), operands staged through LDS.
// f16 tensors use v_mfma_f32_32x32x16_f16 (f16 products are exact in f32, f32
// accumulate); f32 tensors use v_mfma_f32_32x32x2_f32.  Rows of X are gathered
// per layout so that Xw is written time-major ([D][S][B][G*H], row t*B+b).
#include "device_common.h"

namespace rnnhip {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 128, kBN = 128;

template <typename T> struct ProjCfg;
template <> struct ProjCfg<half_t> { static constexpr int BK = 32, PAD = 8; };
template <> struct ProjCfg<float> { static constexpr int BK = 16, PAD = 4; };

// Row m of the product (m = t*B + b) -> row of X in its layout.
__device__ __forceinline__ int64_t x_row(int64_t m, int64_t S, int64_t B, int layout) {
  if (layout == 0) return m;
  const int64_t t = m / B, b = m - t * B;
  return b * S + t;
}

template <typename T>
__global__ __launch_bounds__(256) void projection_kernel(ProjArgs a) {
  constexpr int BK = ProjCfg<T>::BK, LD = BK + ProjCfg<T>::PAD;
  __shared__ __attribute__((aligned(16))) T As[kBM * LD];
  __shared__ __attribute__((aligned(16))) T Bs[kBN * LD];

  const int d = blockIdx.z;
  const int64_t m0 = int64_t(blockIdx.x) * kBM;
  const int64_t n0 = int64_t(blockIdx.y) * kBN;
  // a whole tile inside a gate block nobody reads (input_forget's f) is skipped
  if (a.skip_block >= 0 && n0 >= a.skip_block * a.H && n0 + kBN <= (a.skip_block + 1) * a.H) return;

  const T* X = static_cast<const T*>(a.X);
  const T* W = static_cast<const T*>(a.W) + int64_t(d) * a.N * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int64_t k0 = 0; k0 < a.K; k0 += BK) {
    // stage A (X rows) and B (W rows) tiles; zero outside the matrices
    for (int e = tid; e < kBM * BK; e += 256) {
      const int r = e / BK, k = e % BK;
      const int64_t m = m0 + r, kk = k0 + k;
      T v = T(0.f);
      if (m < a.M && kk < a.K) v = X[x_row(m, a.S, a.B, a.layout) * a.K + kk];
      As[r * LD + k] = v;
    }
    for (int e = tid; e < kBN * BK; e += 256) {
      const int r = e / BK, k = e % BK;
      const int64_t n = n0 + r, kk = k0 + k;
      T v = T(0.f);
      if (n < a.N && kk < a.K) v = W[n * a.K + kk];
      Bs[r * LD + k] = v;
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        f16x8 av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          av[i] = *reinterpret_cast<const f16x8*>(&As[(wm * 64 + i * 32 + (lane & 31)) * LD + ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bv[j] = *reinterpret_cast<const f16x8*>(&Bs[(wn * 64 + j * 32 + (lane & 31)) * LD + ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 2) {
        float av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) av[i] = As[(wm * 64 + i * 32 + (lane & 31)) * LD + ks + (lane >> 5)];
#pragma unroll
        for (int j = 0; j < 2; ++j) bv[j] = Bs[(wn * 64 + j * 32 + (lane & 31)) * LD + ks + (lane >> 5)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
  float* out = a.xw + int64_t(d) * a.M * a.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m < a.M && n < a.N) out[m * a.N + n] = acc[i][j][r];
      }
}

hipError_t launch_projection(const ProjArgs& a, int dtype, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const int64_t mt = (a.M + kBM - 1) / kBM, nt = (a.N + kBN - 1) / kBN;
  if (mt > 0x7fffffff || nt > 65535) return hipErrorInvalidValue;
  dim3 grid(unsigned(mt), unsigned(nt), unsigned(a.D));
  if (dtype == RNN_DTYPE_F32)
    hipLaunchKernelGGL(projection_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(projection_kernel<half_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rnnhip

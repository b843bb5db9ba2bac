// k_projection.hip -- stage 1 of a layer ("Recurrent layers" page, "How a
// layer runs", item 1): the input projection of every step and direction as
// one batched matrix product Xw[d] = X . W[d]^T (W read as stored, [G*H, I],
// i.e. the transposed-B form), f32 accumulation.  No bias is added here: the
// biases enter the gate sum in the page's fixed order.  The same launch also
// carries the state setup (stage 2) in a few extra workgroups.
//
// MI355X design: BMxBN output tiles per 256-thread workgroup (four wave64s in
// 2x2, each a grid of 32x32 MFMA blocks); k chunks (64 for f16, 32 for f32)
// staged through double-buffered LDS, with the next chunk's 16-byte loads in
// flight while the matrix cores work on the current one.  f16 tensors use
// v_mfma_f32_32x32x16_f16 (f16 products are exact in f32, f32 accumulate);
// f32 tensors use v_mfma_f32_32x32x2_f32.  Rows of X are gathered per layout
// so that Xw is written time-major ([D][S][B][G*H], row t*B+b).  Tiles that
// fall entirely in a gate block nobody reads (input_forget's f) are skipped.
#include <algorithm>

#include "device_common.h"

namespace rnnhip {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct ProjCfg;
template <> struct ProjCfg<half_t> { static constexpr int BK = 64, SEG = 8; };   // 16-byte segments
template <> struct ProjCfg<float> { static constexpr int BK = 32, SEG = 4; };

template <typename T> struct Seg;
template <> struct Seg<half_t> { typedef f16x8 type; };
template <> struct Seg<float> { typedef float4 type; };

// Row m of the product (m = t*B + b) -> row of X in its layout.
__device__ __forceinline__ int64_t x_row(int64_t m, int64_t S, int64_t B, int layout) {
  if (layout == 0) return m;
  const int64_t t = m / B, b = m - t * B;
  return b * S + t;
}

template <typename T, bool VEC>
__device__ __forceinline__ typename Seg<T>::type load_seg(const T* p, int64_t k, int64_t K) {
  typedef typename Seg<T>::type V;
  constexpr int SEG = ProjCfg<T>::SEG;
  if (VEC && k + SEG <= K) return *reinterpret_cast<const V*>(p + k);
  V v;
#pragma unroll
  for (int z = 0; z < SEG; ++z) v[z] = (k + z < K) ? p[k + z] : T(0.f);
  return v;
}

template <typename T, int BM, int BN, bool VEC>
__global__ __launch_bounds__(256) void projection_kernel(ProjArgs a, SetupArgs sa, int gemm_blocks) {
  constexpr int BK = ProjCfg<T>::BK, SEG = ProjCfg<T>::SEG, LD = BK + SEG;  // padded LDS row
  constexpr int SEGROW = BK / SEG;
  constexpr int APER = BM * SEGROW / 256, BPER = BN * SEGROW / 256;
  constexpr int WM = BM / 2, WN = BN / 2;             // per-wave tile
  constexpr int IM = WM / 32, IN = WN / 32;           // 32x32 blocks per wave
  typedef typename Seg<T>::type V;
  __shared__ __attribute__((aligned(16))) T As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * LD];

  // extra workgroups: the state setup of stage 2
  if (int(blockIdx.x) >= gemm_blocks) {
    setup_state<T>(sa, int(blockIdx.x) - gemm_blocks, int(gridDim.x) - gemm_blocks);
    return;
  }
  const int64_t mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int64_t lin = blockIdx.x;
  const int64_t mi = lin % mt, ni = (lin / mt) % nt;
  const int d = int(lin / (mt * nt));
  const int64_t m0 = mi * BM, n0 = ni * BN;
  if (a.skip_block >= 0 && n0 >= a.skip_block * a.H && n0 + BN <= (a.skip_block + 1) * a.H) return;

  const T* X = static_cast<const T*>(a.X);
  const T* W = static_cast<const T*>(a.W) + int64_t(d) * a.N * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // row pointers of this thread's segments (null: outside the matrix)
  const T* ap[APER];
  const T* bp[BPER];
  int ak[APER], bk[BPER];
#pragma unroll
  for (int i = 0; i < APER; ++i) {
    const int q = tid + i * 256, r = q / SEGROW;
    ak[i] = (q % SEGROW) * SEG;
    ap[i] = (m0 + r < a.M) ? X + x_row(m0 + r, a.S, a.B, a.layout) * a.K : nullptr;
  }
#pragma unroll
  for (int i = 0; i < BPER; ++i) {
    const int q = tid + i * 256, r = q / SEGROW;
    bk[i] = (q % SEGROW) * SEG;
    bp[i] = (n0 + r < a.N) ? W + (n0 + r) * a.K : nullptr;
  }
  V ra[APER], rb[BPER];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      V z{};
      ra[i] = ap[i] ? load_seg<T, VEC>(ap[i], k0 + ak[i], a.K) : z;
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      V z{};
      rb[i] = bp[i] ? load_seg<T, VEC>(bp[i], k0 + bk[i], a.K) : z;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int q = tid + i * 256;
      *reinterpret_cast<V*>(&As[buf][(q / SEGROW) * LD + ak[i]]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + i * 256;
      *reinterpret_cast<V*>(&Bs[buf][(q / SEGROW) * LD + bk[i]]) = rb[i];
    }
  };

  f32x16 acc[IM][IN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int64_t nk = (a.K + BK - 1) / BK;
  if (nk > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int64_t kc = 0; kc < nk; ++kc) {
    const int buf = int(kc & 1);
    if (kc + 1 < nk) fetch((kc + 1) * BK);
    const T* A = As[buf];
    const T* Bm = Bs[buf];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        f16x8 av[IM], bv[IN];
#pragma unroll
        for (int i = 0; i < IM; ++i)
          av[i] = *reinterpret_cast<const f16x8*>(&A[(wm * WM + i * 32 + (lane & 31)) * LD + ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int j = 0; j < IN; ++j)
          bv[j] = *reinterpret_cast<const f16x8*>(&Bm[(wn * WN + j * 32 + (lane & 31)) * LD + ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int i = 0; i < IM; ++i)
#pragma unroll
          for (int j = 0; j < IN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 2) {
        float av[IM], bv[IN];
#pragma unroll
        for (int i = 0; i < IM; ++i) av[i] = A[(wm * WM + i * 32 + (lane & 31)) * LD + ks + (lane >> 5)];
#pragma unroll
        for (int j = 0; j < IN; ++j) bv[j] = Bm[(wn * WN + j * 32 + (lane & 31)) * LD + ks + (lane >> 5)];
#pragma unroll
        for (int i = 0; i < IM; ++i)
#pragma unroll
          for (int j = 0; j < IN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kc + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
  float* out = a.xw + int64_t(d) * a.M * a.N;
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * WN + j * 32 + (lane & 31);
        if (m < a.M && n < a.N) out[m * a.N + n] = acc[i][j][r];
      }
}

// f32 tensors on the bf16 matrix cores: each f32 value x is split into
// hi = bf16(x) and lo = bf16(x - hi) (both rounded to nearest even; x - hi is
// exact in f32) when its chunk is stored to LDS, and a product a.b is taken
// as lo_a.hi_b + hi_a.lo_b + hi_a.hi_b with v_mfma_f32_32x32x16_bf16, f32
// accumulation, in that order.  bf16 x bf16 products are exact in f32; the
// dropped lo_a.lo_b term and the split residuals are below 2^-16 of |a.b|, so
// a K-term dot product is within about 2^-16 * sum |a.b| of the f32 result.
// bf16 keeps the f32 exponent range, so no scaling is needed.  Tiles, k
// chunks and the double-buffered LDS are as in projection_kernel (BK = 32 f32
// values per chunk, stored as two bf16 planes per operand).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split_bf16(const float4 v, bf16x4& hi, bf16x4& lo) {
  const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    const __bf16 h = __bf16(x[z]);
    hi[z] = h;
    lo[z] = __bf16(x[z] - float(h));
  }
}

template <int BM, int BN, bool VEC>
__global__ __launch_bounds__(256) void projection_bf16x3_kernel(ProjArgs a, SetupArgs sa, int gemm_blocks) {
  constexpr int BK = 32, SEG = 4, LD = BK + 8;        // LDS row: 32 bf16 + 8 pad (80 bytes)
  constexpr int SEGROW = BK / SEG;
  constexpr int APER = BM * SEGROW / 256, BPER = BN * SEGROW / 256;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int IM = WM / 32, IN = WN / 32;
  __shared__ __attribute__((aligned(16))) __bf16 Ah[2][BM * LD], Al[2][BM * LD];
  __shared__ __attribute__((aligned(16))) __bf16 Bh[2][BN * LD], Bl[2][BN * LD];

  if (int(blockIdx.x) >= gemm_blocks) {
    setup_state<float>(sa, int(blockIdx.x) - gemm_blocks, int(gridDim.x) - gemm_blocks);
    return;
  }
  const int64_t mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int64_t lin = blockIdx.x;
  const int64_t mi = lin % mt, ni = (lin / mt) % nt;
  const int d = int(lin / (mt * nt));
  const int64_t m0 = mi * BM, n0 = ni * BN;
  if (a.skip_block >= 0 && n0 >= a.skip_block * a.H && n0 + BN <= (a.skip_block + 1) * a.H) return;

  const float* X = static_cast<const float*>(a.X);
  const float* W = static_cast<const float*>(a.W) + int64_t(d) * a.N * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const float* ap[APER];
  const float* bp[BPER];
  int ak[APER], bk[BPER];
#pragma unroll
  for (int i = 0; i < APER; ++i) {
    const int q = tid + i * 256, r = q / SEGROW;
    ak[i] = (q % SEGROW) * SEG;
    ap[i] = (m0 + r < a.M) ? X + x_row(m0 + r, a.S, a.B, a.layout) * a.K : nullptr;
  }
#pragma unroll
  for (int i = 0; i < BPER; ++i) {
    const int q = tid + i * 256, r = q / SEGROW;
    bk[i] = (q % SEGROW) * SEG;
    bp[i] = (n0 + r < a.N) ? W + (n0 + r) * a.K : nullptr;
  }
  float4 ra[APER], rb[BPER];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < APER; ++i) ra[i] = ap[i] ? load_seg<float, VEC>(ap[i], k0 + ak[i], a.K) : float4{};
#pragma unroll
    for (int i = 0; i < BPER; ++i) rb[i] = bp[i] ? load_seg<float, VEC>(bp[i], k0 + bk[i], a.K) : float4{};
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < APER; ++i) {
      const int q = tid + i * 256, o = (q / SEGROW) * LD + ak[i];
      bf16x4 hi, lo;
      split_bf16(ra[i], hi, lo);
      *reinterpret_cast<bf16x4*>(&Ah[buf][o]) = hi;
      *reinterpret_cast<bf16x4*>(&Al[buf][o]) = lo;
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      const int q = tid + i * 256, o = (q / SEGROW) * LD + bk[i];
      bf16x4 hi, lo;
      split_bf16(rb[i], hi, lo);
      *reinterpret_cast<bf16x4*>(&Bh[buf][o]) = hi;
      *reinterpret_cast<bf16x4*>(&Bl[buf][o]) = lo;
    }
  };

  f32x16 acc[IM][IN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int64_t nk = (a.K + BK - 1) / BK;
  if (nk > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int64_t kc = 0; kc < nk; ++kc) {
    const int buf = int(kc & 1);
    if (kc + 1 < nk) fetch((kc + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      const int ko = ks + 8 * (lane >> 5);
      bf16x8 ah[IM], al[IM], bh[IN], bl[IN];
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        const int o = (wm * WM + i * 32 + (lane & 31)) * LD + ko;
        ah[i] = *reinterpret_cast<const bf16x8*>(&Ah[buf][o]);
        al[i] = *reinterpret_cast<const bf16x8*>(&Al[buf][o]);
      }
#pragma unroll
      for (int j = 0; j < IN; ++j) {
        const int o = (wn * WN + j * 32 + (lane & 31)) * LD + ko;
        bh[j] = *reinterpret_cast<const bf16x8*>(&Bh[buf][o]);
        bl[j] = *reinterpret_cast<const bf16x8*>(&Bl[buf][o]);
      }
#pragma unroll
      for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < IN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        }
    }
    if (kc + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  float* out = a.xw + int64_t(d) * a.M * a.N;
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * WN + j * 32 + (lane & 31);
        if (m < a.M && n < a.N) out[m * a.N + n] = acc[i][j][r];
      }
}

template <int BM, int BN>
static hipError_t launch_bf16x3(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, hipStream_t s) {
  const int64_t mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int64_t gemm = (a.M > 0 && a.N > 0) ? mt * nt * a.D : 0;
  if (gemm + setup_blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bool vec = a.K % 4 == 0 && reinterpret_cast<uintptr_t>(a.X) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.W) % 16 == 0;
  const dim3 grid(unsigned(gemm + setup_blocks));
  if (vec)
    hipLaunchKernelGGL((projection_bf16x3_kernel<BM, BN, true>), grid, dim3(256), 0, s, a, sa, int(gemm));
  else
    hipLaunchKernelGGL((projection_bf16x3_kernel<BM, BN, false>), grid, dim3(256), 0, s, a, sa, int(gemm));
  return hipGetLastError();
}

template <typename T, int BM, int BN>
static hipError_t launch_tile(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, hipStream_t s) {
  const int64_t mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int64_t gemm = (a.M > 0 && a.N > 0) ? mt * nt * a.D : 0;
  if (gemm + setup_blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int seg = ProjCfg<T>::SEG;
  const bool vec = a.K % seg == 0 && reinterpret_cast<uintptr_t>(a.X) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.W) % 16 == 0;
  const dim3 grid(unsigned(gemm + setup_blocks));
  if (vec)
    hipLaunchKernelGGL((projection_kernel<T, BM, BN, true>), grid, dim3(256), 0, s, a, sa, int(gemm));
  else
    hipLaunchKernelGGL((projection_kernel<T, BM, BN, false>), grid, dim3(256), 0, s, a, sa, int(gemm));
  return hipGetLastError();
}

hipError_t launch_projection_lds(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, hipStream_t s);

hipError_t launch_projection(const ProjArgs& a, const SetupArgs& sa, int dtype, hipStream_t s) {
  const int64_t n_state = int64_t(sa.D) * sa.B * sa.H;
  const int setup_blocks = n_state > 0 ? int(std::min<int64_t>((n_state + 255) / 256, 1024)) : 0;
  // large f16 layers: 256x256 tiles loaded straight into LDS (k_projection_lds.hip)
  if (dtype == RNN_DTYPE_F16 && a.M > 0 && a.N > 0) {
    const hipError_t e = launch_projection_lds(a, sa, setup_blocks, s);
    if (e != hipErrorNotSupported) return e;
  }
  // 128x128 tiles when they still give every compute unit a workgroup, else 64x64
  const int64_t big = ((a.M + 127) / 128) * ((a.N + 127) / 128) * a.D;
  const bool use_big = big >= 256;
  if (dtype == RNN_DTYPE_F32) {
    if (a.f32_split)
      return use_big ? launch_bf16x3<128, 128>(a, sa, setup_blocks, s) : launch_bf16x3<64, 64>(a, sa, setup_blocks, s);
    return use_big ? launch_tile<float, 128, 128>(a, sa, setup_blocks, s)
                   : launch_tile<float, 64, 64>(a, sa, setup_blocks, s);
  }
  return use_big ? launch_tile<half_t, 128, 128>(a, sa, setup_blocks, s)
                 : launch_tile<half_t, 64, 64>(a, sa, setup_blocks, s);
}

}  // namespace rnnhip

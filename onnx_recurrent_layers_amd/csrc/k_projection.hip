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
#include <cstdlib>

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

// The segment of SEG elements at k of a row starting at p (zeros past K);
// elements at or past kh lie `jump` further on (a row of X in two pieces; W
// rows pass kh = K).  VEC: whole segments in one load, which the host allows
// only when no segment straddles kh.
template <typename T, bool VEC>
__device__ __forceinline__ typename Seg<T>::type load_seg(const T* p, int64_t k, int64_t K, int64_t kh,
                                                          int64_t jump) {
  typedef typename Seg<T>::type V;
  constexpr int SEG = ProjCfg<T>::SEG;
  if (VEC && k + SEG <= K) return *reinterpret_cast<const V*>(p + k + (k >= kh ? jump : 0));
  V v;
#pragma unroll
  for (int z = 0; z < SEG; ++z) v[z] = (k + z < K) ? p[k + z + (k + z >= kh ? jump : 0)] : T(0.f);
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
    ap[i] = (m0 + r < a.M) ? X + x_row_step(a, d, m0 + r) : nullptr;
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
      ra[i] = ap[i] ? load_seg<T, VEC>(ap[i], k0 + ak[i], a.K, a.xkh, a.xjump) : z;
    }
#pragma unroll
    for (int i = 0; i < BPER; ++i) {
      V z{};
      rb[i] = bp[i] ? load_seg<T, VEC>(bp[i], k0 + bk[i], a.K, a.K, 0) : z;
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
  float* out = a.xw + int64_t(d) * a.out_dstride;
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
    ap[i] = (m0 + r < a.M) ? X + x_row_step(a, d, m0 + r) : nullptr;
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
    for (int i = 0; i < APER; ++i)
      ra[i] = ap[i] ? load_seg<float, VEC>(ap[i], k0 + ak[i], a.K, a.xkh, a.xjump) : float4{};
#pragma unroll
    for (int i = 0; i < BPER; ++i) rb[i] = bp[i] ? load_seg<float, VEC>(bp[i], k0 + bk[i], a.K, a.K, 0) : float4{};
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

  float* out = a.xw + int64_t(d) * a.out_dstride;
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

// Small projections (fewer than 256 tiles of 64x64: C2's 80 x 1024 x 256 per
// direction, say) are latency-bound: the tiled kernel above walks K in eight
// or more chunks, one memory round trip each, on a quarter of the compute
// units.  Here a workgroup owns a 32x32 output tile, which gives 3 to 4 times
// as many workgroups, and its four waves split K: the K axis is cut into
// blocks of 2*NSEG segments of 16 bytes, wave w takes blocks w, w+4, ...
// Inside a block lane l reads NSEG consecutive segments of row l%32 of X (A
// operand) and of W (B operand) straight into registers, lanes 0-31 the first
// half of the block and lanes 32-63 the second; MFMA step j then pairs the two
// halves' j-th k values (32x32x2 f32) or 8-value runs (32x32x16 f16).  A and
// B use the same k assignment, so every product is a genuine X*W term, and
// the order is fixed.  No LDS staging: a block is one round of loads.  The
// four waves' partial tiles are added in wave order through LDS.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void projection_small_kernel(ProjArgs a, SetupArgs sa, int gemm_blocks) {
  constexpr int SEG = ProjCfg<T>::SEG, NSEG = 8;
  constexpr int HALF = NSEG * SEG;  // k of one half-wave in a block
  constexpr int KBLK = 2 * HALF;    // k of one block
  typedef typename Seg<T>::type V;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
  __shared__ float red[4][32][33];

  if (int(blockIdx.x) >= gemm_blocks) {
    setup_state<T>(sa, int(blockIdx.x) - gemm_blocks, int(gridDim.x) - gemm_blocks);
    return;
  }
  const int64_t mt = (a.M + 31) / 32, nt = (a.N + 31) / 32;
  const int64_t lin = blockIdx.x;
  const int64_t mi = lin % mt, ni = (lin / mt) % nt;
  const int d = int(lin / (mt * nt));
  const int64_t m0 = mi * 32, n0 = ni * 32;
  if (a.skip_block >= 0 && n0 >= a.skip_block * a.H && n0 + 32 <= (a.skip_block + 1) * a.H) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, half = lane >> 5;
  const T* X = static_cast<const T*>(a.X);
  const T* W = static_cast<const T*>(a.W) + int64_t(d) * a.N * a.K;
  // Loads are unconditional, from clamped addresses (a load under a lane
  // condition makes the compiler wait for it before issuing the next one), and
  // the values are masked where they are used.  Only k past K needs masking,
  // in both operands, so that such a product is exactly zero; a row past M or
  // N feeds only outputs that are dropped.  The mask is a bit mask, not a
  // select, which keeps the compiler from moving the loads into branches.
  const T* ap = X + x_row_step(a, d, m0 + r32 < a.M ? m0 + r32 : a.M - 1);
  const T* bp = W + (n0 + r32 < a.N ? n0 + r32 : a.N - 1) * a.K;
  // (rows of X in two pieces: elements at or past kh lie `jump` further on;
  // W passes kh = K)
  auto seg = [&](const T* p, int64_t k, int64_t kh, int64_t jump) {
    if constexpr (VEC) {  // K is a whole number of segments, none straddles kh
      const int64_t kk = k < a.K ? k : 0;
      return *reinterpret_cast<const u32x4*>(p + kk + (kk >= kh ? jump : 0));
    } else if constexpr (sizeof(T) == 4) {
      u32x4 u;
#pragma unroll
      for (int z = 0; z < SEG; ++z) {
        const int64_t kk = k + z < a.K ? k + z : a.K - 1;
        u[z] = reinterpret_cast<const unsigned*>(p)[kk + (kk >= kh ? jump : 0)];
      }
      return u;
    } else {
      u16x8 u;
#pragma unroll
      for (int z = 0; z < SEG; ++z) {
        const int64_t kk = k + z < a.K ? k + z : a.K - 1;
        u[z] = reinterpret_cast<const unsigned short*>(p)[kk + (kk >= kh ? jump : 0)];
      }
      return __builtin_bit_cast(u32x4, u);
    }
  };
  // mask of the 32-bit words of the segment at k: all ones where k is inside K
  auto kmask = [&](int64_t k) {
    u32x4 m;
    if constexpr (VEC) {
      m = u32x4(0u - unsigned(k < a.K));
    } else if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int z = 0; z < 4; ++z) m[z] = 0u - unsigned(k + z < a.K);
    } else {
#pragma unroll
      for (int z = 0; z < 4; ++z)
        m[z] = ((0u - unsigned(k + 2 * z < a.K)) & 0xffffu) | ((0u - unsigned(k + 2 * z + 1 < a.K)) & 0xffff0000u);
    }
    return m;
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // One round of loads per block.  For K up to 256 f32 or 512 f16 values
  // every wave has at most one block, so the tile takes one memory round
  // trip.  (Prefetching the next block into a second register set was undone
  // by the compiler, which moved those loads past the loop's exit test to
  // where they are used.)
  const int64_t nblk = (a.K + KBLK - 1) / KBLK;
  for (int64_t blk = wave; blk < nblk; blk += 4) {
    const int64_t k0 = blk * KBLK + half * HALF;
    u32x4 ra[NSEG], rb[NSEG];
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      ra[i] = seg(ap, k0 + i * SEG, a.xkh, a.xjump);
      rb[i] = seg(bp, k0 + i * SEG, a.K, 0);
    }
    // keep the scheduler from moving each load down to its use
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      const u32x4 m = kmask(k0 + i * SEG);
      const V va = __builtin_bit_cast(V, ra[i] & m), vb = __builtin_bit_cast(V, rb[i] & m);
      if constexpr (sizeof(T) == 2) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, vb, acc, 0, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < SEG; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], vb[e], acc, 0, 0, 0);
      }
    }
  }

  // 32x32 accumulator layout: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * half + (r & 3)][r32] = acc[r];
  __syncthreads();
  const int nw = int(nblk < 4 ? nblk : 4);  // waves that own a block
  float* out = a.xw + int64_t(d) * a.out_dstride;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q, row = e >> 5, col = e & 31;
    const int64_t m = m0 + row, n = n0 + col;
    if (m < a.M && n < a.N) {
      float v = red[0][row][col];
      for (int w = 1; w < nw; ++w) v += red[w][row][col];
      out[m * a.N + n] = v;
    }
  }
}

template <typename T>
static hipError_t launch_small(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, hipStream_t s) {
  const int64_t mt = (a.M + 31) / 32, nt = (a.N + 31) / 32;
  const int64_t gemm = (a.M > 0 && a.N > 0) ? mt * nt * a.D : 0;
  if (gemm + setup_blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int seg = ProjCfg<T>::SEG;
  const bool vec = a.K % seg == 0 && a.xkh % seg == 0 && a.xjump % seg == 0 &&
                   reinterpret_cast<uintptr_t>(a.X) % 16 == 0 && reinterpret_cast<uintptr_t>(a.W) % 16 == 0;
  const dim3 grid(unsigned(gemm + setup_blocks));
  if (vec)
    hipLaunchKernelGGL((projection_small_kernel<T, true>), grid, dim3(256), 0, s, a, sa, int(gemm));
  else
    hipLaunchKernelGGL((projection_small_kernel<T, false>), grid, dim3(256), 0, s, a, sa, int(gemm));
  return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_bf16x3(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, hipStream_t s) {
  const int64_t mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int64_t gemm = (a.M > 0 && a.N > 0) ? mt * nt * a.D : 0;
  if (gemm + setup_blocks > 0x7fffffff) return hipErrorInvalidValue;
  const bool vec = a.K % 4 == 0 && a.xkh % 4 == 0 && a.xjump % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(a.X) % 16 == 0 && reinterpret_cast<uintptr_t>(a.W) % 16 == 0;
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
  const bool vec = a.K % seg == 0 && a.xkh % seg == 0 && a.xjump % seg == 0 &&
                   reinterpret_cast<uintptr_t>(a.X) % 16 == 0 && reinterpret_cast<uintptr_t>(a.W) % 16 == 0;
  const dim3 grid(unsigned(gemm + setup_blocks));
  if (vec)
    hipLaunchKernelGGL((projection_kernel<T, BM, BN, true>), grid, dim3(256), 0, s, a, sa, int(gemm));
  else
    hipLaunchKernelGGL((projection_kernel<T, BM, BN, false>), grid, dim3(256), 0, s, a, sa, int(gemm));
  return hipGetLastError();
}

hipError_t launch_projection_lds(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, int dtype,
                                 hipStream_t s);

hipError_t launch_projection(const ProjArgs& a, const SetupArgs& sa, int dtype, hipStream_t s) {
  const int64_t n_state = int64_t(sa.D) * sa.B * sa.H;
  const int setup_blocks = n_state > 0 ? int(std::min<int64_t>((n_state + 255) / 256, 1024)) : 0;
  // large f16 layers, and large f32 layers on the bf16 matrix cores: 256x256
  // tiles loaded straight into LDS (k_projection_lds.hip)
  if ((dtype == RNN_DTYPE_F16 || (dtype == RNN_DTYPE_F32 && a.f32_split)) && a.M > 0 && a.N > 0) {
    const hipError_t e = launch_projection_lds(a, sa, setup_blocks, dtype, s);
    if (e != hipErrorNotSupported) return e;
  }
  // 128x128 tiles when they still give every compute unit a workgroup, else
  // 64x64; below 256 tiles of 64x64 the latency-bound small kernel
  const int64_t big = ((a.M + 127) / 128) * ((a.N + 127) / 128) * a.D;
  const bool use_big = big >= 256;
  const int64_t mid = ((a.M + 63) / 64) * ((a.N + 63) / 64) * a.D;
  bool small = mid < 256;
  if (const char* e = std::getenv("RNN_SMALL_PROJECTION")) small = std::atoi(e) != 0;  // forces it on (1) or off (0)
  if (small && !(dtype == RNN_DTYPE_F32 && a.f32_split))
    return dtype == RNN_DTYPE_F32 ? launch_small<float>(a, sa, setup_blocks, s)
                                  : launch_small<half_t>(a, sa, setup_blocks, s);
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

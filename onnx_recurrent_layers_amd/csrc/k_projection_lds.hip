// k_projection_lds.hip -- stage 1 of a layer ("Recurrent layers" page, "How a
// layer runs", item 1) for large f16 layers: Xw[d] = X . W[d]^T with f32
// accumulation, as the other projection kernel computes it, in 256x256 tiles
// whose operands go from global memory straight into LDS.
//
// A workgroup of four waves owns a 256x256 output tile; each wave a 128x128
// quarter of it as 4x4 blocks of v_mfma_f32_32x32x16_f16 (f16 products are
// exact in f32).  k advances in chunks of 32; four chunks are resident in LDS,
// three of them in flight while the matrix cores work on the fourth.  Each
// chunk is loaded with buffer loads that write LDS directly: a segment
// outside the matrices (rows past M or N, k past K) gets an offset past the
// resource and reads as zero, so there are no bounds branches and every wave
// issues the same number of loads per chunk (the wait for a chunk is a fixed
// count).  Rows are 64 bytes (four 16-byte segments); segment s of row r sits
// in slot s ^ ((r >> 2) & 3), which puts the 16 rows of one operand read in
// different bank groups.  Inside a chunk lane group g of an operand takes k
// 16g..16g+15 (for both operands, so each dot product is the same sum).
//
// f32 layers whose projection runs on the bf16 matrix cores (three split
// products) use the same tiles with f32 operands: a 64-byte row then holds 16
// values, so a chunk covers k 16 and has the same LDS layout, loads and waits.
// Each lane reads the 8 values of its lane group (k 8g..8g+7) and splits them
// on the way into registers, hi = bf16(x) and lo = bf16(x - hi) (round to
// nearest even; x - hi is exact in f32), and each 32x32 block takes
// lo_x.hi_w + hi_x.lo_w + hi_x.hi_w with v_mfma_f32_32x32x16_bf16, f32
// accumulation: bf16 products are exact in f32, and what the split drops is
// below 2^-16 of each |x.w|.  Splitting as the operands are read, not as they
// are stored, is what lets them go straight into LDS.
//
// The grid is laid out for the eight XCDs: workgroup i runs on XCD i % 8, and
// the tiles of one XCD are consecutive in n within an m row, so neighbouring
// tiles of an XCD share their X panel in that XCD's L2.  Column tiles inside
// a gate block nobody reads (input_forget's f) are not computed.  Extra
// workgroups at the end of the grid run the state setup (stage 2).
#include <algorithm>
#include <cstdlib>

#include "device_common.h"

namespace rnnhip {

namespace {

typedef _Float16 hx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bx8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;          // rows and columns of an output tile
constexpr int kRowBytes = 64;       // bytes of one operand row of a chunk: k 32 (f16) or 16 (f32)
constexpr int kNS = 4;              // chunks resident
constexpr int kOpBytes = kTile * kRowBytes;  // one operand of one chunk (16 KiB)
constexpr int kLoads = kOpBytes / 1024 / 4; // loads per wave per operand per chunk (4)
constexpr unsigned kOOB = 0x80000000u;      // beyond every resource used here
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, 32-bit data format (gfx9 family)

constexpr int waitcnt_imm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

template <int VM>
__device__ __forceinline__ void chunk_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling of one chunk's instructions: its D operand reads first, then
// the L loads of a later chunk spread between its M matrix-core products (a
// wave issues in order: loads grouped ahead of the products would hold the
// products back while the memory unit accepts them).
template <int D, int L, int M>
__device__ __forceinline__ void interleave_chunk() {
  __builtin_amdgcn_sched_group_barrier(0x100, D, 0);   // LDS reads
#pragma unroll
  for (int g = 0; g < L; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);              // a memory load
    __builtin_amdgcn_sched_group_barrier(0x008, (M + L - 1) / L, 0);   // matrix-core products
  }
}

// hi = bf16(x), lo = bf16(x - hi) of eight values
__device__ __forceinline__ void split8(const f32x4 p, const f32x4 q, bx8& hi, bx8& lo) {
  const float x[8] = {p[0], p[1], p[2], p[3], q[0], q[1], q[2], q[3]};
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    const __bf16 h = __bf16(x[z]);
    hi[z] = h;
    lo[z] = __bf16(x[z] - float(h));
  }
}

}  // namespace

struct TileMap {
  int mt, nct, tiles_per_dir, per_xcd, sb0, nskip;
};

// T = half_t: f16 operands; T = float: f32 operands split into bf16 halves.
template <typename T>
__global__ __launch_bounds__(256) void projection_lds_kernel(ProjArgs a, SetupArgs sa, TileMap tm, int gemm_blocks) {
  constexpr int ES = int(sizeof(T));          // element bytes
  constexpr int KC = kRowBytes / ES;          // k per chunk
  constexpr int SEGE = 16 / ES;               // elements of a 16-byte segment
  // one LDS object per operand of each resident chunk (the compiler then
  // keeps its waits for the loads into one chunk apart from the reads of
  // another)
  __shared__ __attribute__((aligned(1024))) unsigned char xa0[kOpBytes], xa1[kOpBytes], xa2[kOpBytes], xa3[kOpBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char wb0[kOpBytes], wb1[kOpBytes], wb2[kOpBytes], wb3[kOpBytes];

  if (int(blockIdx.x) >= gemm_blocks) {
    setup_state<T>(sa, int(blockIdx.x) - gemm_blocks, int(gridDim.x) - gemm_blocks);
    return;
  }
  // XCD-aware tile order: workgroup i -> tile (i % 8) * per_xcd + i / 8
  const int t = int(blockIdx.x & 7) * tm.per_xcd + int(blockIdx.x >> 3);
  if (t >= tm.tiles_per_dir * a.D) return;
  const int d = t / tm.tiles_per_dir, r = t - d * tm.tiles_per_dir;
  const int mi = r / tm.nct, ci = r - mi * tm.nct;
  const int ni = ci < tm.sb0 ? ci : ci + tm.nskip;   // skip the unread gate block's column tiles
  const int64_t m0 = int64_t(mi) * kTile, n0 = int64_t(ni) * kTile;
  const int K = int(a.K);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.X), 0, int(a.S * a.B * a.K * ES), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(a.W) + int64_t(d) * a.N * a.K), 0, int(a.N * a.K * ES), kRsrcWord3);

  // this lane's rows: load i of the wave covers tile rows (wave*kLoads + i)*16 .. +16,
  // lane l row +l/4, slot l%4 holding segment slot ^ ((row >> 2) & 3)
  unsigned xrow[kLoads], wrow[kLoads];
  int seg[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int row = (wave * kLoads + i) * 16 + (lane >> 2);
    seg[i] = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t m = m0 + row, n = n0 + row;
    xrow[i] = m < a.M ? unsigned(x_row_step(a, d, m) * ES) : kOOB;
    wrow[i] = n < a.N ? unsigned(n * K * ES) : kOOB;
  }
  // X column of element k of a row (32-bit: every offset fits the resource)
  const int xkh = int(a.xkh);
  const unsigned xjump = unsigned(a.xjump);
  auto fetch = [&](int kc, unsigned char* sa_, unsigned char* sb_) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int k = kc * KC + seg[i] * SEGE;
      const unsigned xc = unsigned(k) + (k >= xkh ? xjump : 0u);
      // a row outside the matrix starts at the out-of-range marker, so row + k stays out of range
      const unsigned ox = k < K ? xrow[i] + xc * unsigned(ES) : kOOB;
      const unsigned ow = k < K ? wrow[i] + unsigned(k) * unsigned(ES) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, RNN_LDS_PTR(sa_ + (wave * kLoads + i) * 1024), 16, ox, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, RNN_LDS_PTR(sb_ + (wave * kLoads + i) * 1024), 16, ow, 0, 0, 0);
    }
  };
  auto slot_a = [&](int i) -> unsigned char* { return i == 0 ? xa0 : i == 1 ? xa1 : i == 2 ? xa2 : xa3; };
  auto slot_b = [&](int i) -> unsigned char* { return i == 0 ? wb0 : i == 1 ? wb1 : i == 2 ? wb2 : wb3; };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, g = lane >> 5;
  const int nk = (K + KC - 1) / KC;
#pragma unroll
  for (int c = 0; c < kNS - 1; ++c) fetch(c, slot_a(c), slot_b(c));
  // chunk kc lives in slot kc % 4; the loop is unrolled over the slots so that
  // each slot is a fixed LDS object.  Chunks past the end load zeros.
  for (int kc0 = 0; kc0 < nk; kc0 += kNS) {
#pragma unroll
    for (int u = 0; u < kNS; ++u) {
      const int kc = kc0 + u;
      chunk_barrier<(kNS - 2) * 2 * kLoads>();   // chunk kc landed for every wave; chunk kc - 1 is read
      fetch(kc + kNS - 1, slot_a((u + kNS - 1) % kNS), slot_b((u + kNS - 1) % kNS));
      const unsigned char* As = slot_a(u);
      const unsigned char* Bs = slot_b(u);
      if constexpr (ES == 4) {
        // lane group g: segments 2g and 2g+1 of each row (k 8g..8g+7)
        bx8 ah[4], al[4], bh[4], bl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 128 + i * 32 + r32;
          const unsigned char* rp = As + row * 64;
          const int sw = (row >> 2) & 3;
          split8(*reinterpret_cast<const f32x4*>(rp + (((2 * g) ^ sw) << 4)),
                 *reinterpret_cast<const f32x4*>(rp + (((2 * g + 1) ^ sw) << 4)), ah[i], al[i]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wn * 128 + j * 32 + r32;
          const unsigned char* rp = Bs + row * 64;
          const int sw = (row >> 2) & 3;
          split8(*reinterpret_cast<const f32x4*>(rp + (((2 * g) ^ sw) << 4)),
                 *reinterpret_cast<const f32x4*>(rp + (((2 * g + 1) ^ sw) << 4)), bh[j], bl[j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[j], al[i], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bl[j], ah[i], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bh[j], ah[i], acc[i][j], 0, 0, 0);
          }
        interleave_chunk<16, 2 * kLoads, 48>();
        continue;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int s = 2 * g + kk;
        hx8 av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 128 + i * 32 + r32;
          av[i] = *reinterpret_cast<const hx8*>(As + row * 64 + ((s ^ ((row >> 2) & 3)) << 4));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wn * 128 + j * 32 + r32;
          bv[j] = *reinterpret_cast<const hx8*>(Bs + row * 64 + ((s ^ ((row >> 2) & 3)) << 4));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[j], av[i], acc[i][j], 0, 0, 0);
      }
      interleave_chunk<16, 2 * kLoads, 32>();
    }
  }
  chunk_barrier<0>();   // the loads past the end have landed before the workgroup ends

  // Each product block is taken transposed (W rows as the first operand), so
  // that the 32x32 accumulator layout, element e of lane l at row
  // 8*(e/4) + 4*(l/32) + e%4 and column l%32, puts four consecutive output
  // columns n (block rows) of one output row m (block column) in elements
  // 4t..4t+3 of a lane: one 16-byte store each when Xw rows are whole 16-byte
  // groups.
  float* out = a.xw + int64_t(d) * a.out_dstride;
  const bool vec = (a.N & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + i * 32 + r32;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t n = n0 + wn * 128 + j * 32 + 8 * t + 4 * g;
        if (m >= a.M) continue;
        if (vec) {
          if (n < a.N)
            *reinterpret_cast<f32x4*>(out + m * a.N + n) =
                f32x4{acc[i][j][4 * t], acc[i][j][4 * t + 1], acc[i][j][4 * t + 2], acc[i][j][4 * t + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < a.N) out[m * a.N + n + e] = acc[i][j][4 * t + e];
        }
      }
  }
}

// Takes the layer when the operands are rows of whole 16-byte segments (f16,
// or f32 split into bf16 halves), every byte offset fits 31 bits and the
// tiles fill the chip; otherwise reports hipErrorNotSupported and the caller
// uses the other kernels.
hipError_t launch_projection_lds(const ProjArgs& a, const SetupArgs& sa, int setup_blocks, int dtype,
                                 hipStream_t s) {
  const int es = dtype == RNN_DTYPE_F32 ? 4 : 2;
  const int sege = 16 / es;
  if (a.K % sege != 0 || a.xkh % sege != 0 || a.xjump % sege != 0 || reinterpret_cast<uintptr_t>(a.X) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(a.W) % 16 != 0)
    return hipErrorNotSupported;
  if (a.S * a.B * a.K * es >= int64_t(kOOB) || a.N * a.K * es >= int64_t(kOOB)) return hipErrorNotSupported;
  TileMap tm{};
  tm.mt = int((a.M + kTile - 1) / kTile);
  const int nt = int((a.N + kTile - 1) / kTile);
  tm.sb0 = nt;
  tm.nskip = 0;
  if (a.skip_block >= 0 && a.H % kTile == 0) {   // the unread block is whole column tiles
    tm.sb0 = int(a.skip_block * a.H / kTile);
    tm.nskip = int(a.H / kTile);
  }
  tm.nct = nt - tm.nskip;
  tm.tiles_per_dir = tm.mt * tm.nct;
  const int64_t tiles = int64_t(tm.tiles_per_dir) * a.D;
  // too few tiles: the 128-wide kernel fills the chip better.  RNN_PROJ_LDS_MIN_TILES
  // lowers the bar, so that tests reach this kernel on small layers.
  int64_t min_tiles = 512;
  if (const char* e = std::getenv("RNN_PROJ_LDS_MIN_TILES")) min_tiles = std::atoll(e);
  if (tiles < min_tiles) return hipErrorNotSupported;
  tm.per_xcd = int((tiles + 7) / 8);
  const int gemm_blocks = 8 * tm.per_xcd;
  if (int64_t(gemm_blocks) + setup_blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (dtype == RNN_DTYPE_F32)
    hipLaunchKernelGGL(projection_lds_kernel<float>, dim3(unsigned(gemm_blocks + setup_blocks)), dim3(256), 0, s, a,
                       sa, tm, gemm_blocks);
  else
    hipLaunchKernelGGL(projection_lds_kernel<half_t>, dim3(unsigned(gemm_blocks + setup_blocks)), dim3(256), 0, s, a,
                       sa, tm, gemm_blocks);
  return hipGetLastError();
}

}  // namespace rnnhip

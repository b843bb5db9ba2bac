// k_step_mfma.hip -- stage 3 of a layer ("Recurrent layers" page, "How a
// layer runs", item 3) for larger batches: one launch per step (two for a GRU
// with linear_before_reset = 0), each computing the recurrent product of the
// step as a matrix product on the matrix cores and finishing the gate
// arithmetic of cells.h in the epilogue.
//
// A workgroup owns a tile of BM batch rows x UJ hidden units of one direction
// and all Gp gate blocks of those units, so the gate arithmetic needs no data
// from other workgroups: the product tile is [BM] x [Gp*UJ] over K = H, with
// A = h_prev rows (f32) and B = R rows (f32, or f16 widened exactly).
// v_mfma_f32_16x16x4_f32 keeps exact f32 products with f32 accumulation;
// the k order inside a workgroup is fixed (chunks of 64 in increasing order,
// the instruction's own order within a chunk), so runs are bit-identical.
// Operand chunks are staged through LDS, the next chunk is fetched into
// registers while the current one feeds the matrix cores.
#include <cstdio>
#include <cstdlib>

#include "step_mfma.h"

namespace rnnhip {

constexpr int kBK = 64;          // k chunk
constexpr int kLDA = kBK + 4;    // padded LDS row (floats)
constexpr int kPF = 3;           // k chunks in flight
constexpr int kSeg = 4;          // elements per load segment (16 bytes of f32 h; 8 bytes of f16 R, 16 of f32 R)

// Four consecutive elements as f32 (vector load when aligned, else four loads).
template <bool VEC>
__device__ __forceinline__ float4 load4(const float* p) {
  if constexpr (VEC) return *reinterpret_cast<const float4*>(p);
  else return make_float4(p[0], p[1], p[2], p[3]);
}
template <bool VEC>
__device__ __forceinline__ float4 load4(const half_t* p) {
  if constexpr (VEC) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = *reinterpret_cast<const h4*>(p);
    return make_float4(float(v[0]), float(v[1]), float(v[2]), float(v[3]));
  } else {
    return make_float4(float(p[0]), float(p[1]), float(p[2]), float(p[3]));
  }
}

template <typename T, int BM, bool VEC>
__global__ __launch_bounds__(kMThreads) void step_mfma_kernel(MfmaStepArgs m) {
  const StepArgs& a = m.a;
  const int H = a.H, B = a.B, G = a.G, S = a.S;
  const int s = m.step;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.x * m.UJ;
  const int b0 = blockIdx.y * BM;
  const int d = blockIdx.z;
  const int UJ = m.UJ, NC = m.Gp * UJ;

  // rows of this tile that are still running at this step
  __shared__ int len_s[BM];
  __shared__ int any_s;
  if (tid == 0) any_s = 0;
  __syncthreads();
  for (int r = tid; r < BM; r += kMThreads) {
    const int b = b0 + r;
    len_s[r] = b < B ? row_length(a.lens, b, S, a.steps) : 0;
    if (s < len_s[r]) atomicOr(&any_s, 1);
  }
  __syncthreads();
  if (!any_s) return;

  __shared__ __attribute__((aligned(16))) float As[2][BM * kLDA];
  __shared__ __attribute__((aligned(16))) float Bs[2][kMaxNC * kLDA];
  __shared__ float rec[BM * (kMaxNC + 1)];

  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  const bool cand_phase = a.cell == RNN_CELL_GRU && !a.lbr && m.phase == 1;
  const float* hsrc = cand_phase ? a.rhbuf + dBH : a.hbuf + int64_t(s & 1) * DBH + dBH;
  const T* Rd = static_cast<const T*>(a.R) + int64_t(d) * G * H * H;

  // Staging: segment q of a chunk is row q / (kBK/kSeg), elements
  // kSeg*(q % (kBK/kSeg)) .. +kSeg.  Each thread keeps the row pointers of its
  // segments for the whole k loop.  Rows beyond the tile, ended batch rows
  // and k beyond H read as zero (H is padded to the chunk by the valid mask).
  constexpr int kSegRow = kBK / kSeg;
  constexpr int kAPer = (BM * kSegRow + kMThreads - 1) / kMThreads;
  constexpr int kBPer = (kMaxNC * kSegRow + kMThreads - 1) / kMThreads;
  const float* aptr[kAPer];
  const T* bptr[kBPer];
  int aoff[kAPer], boff[kBPer];
#pragma unroll
  for (int i = 0; i < kAPer; ++i) {
    const int q = tid + i * kMThreads;
    const int r = q / kSegRow;
    aoff[i] = (q % kSegRow) * kSeg;
    const bool ok = q < BM * kSegRow && b0 + r < B && s < len_s[r];
    aptr[i] = ok ? hsrc + int64_t(b0 + r) * H : nullptr;
  }
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int q = tid + i * kMThreads;
    const int c = q / kSegRow;
    boff[i] = (q % kSegRow) * kSeg;
    bptr[i] = nullptr;
    if (q < NC * kSegRow) {
      const int gi = c / UJ, u = c - gi * UJ;
      if (j0 + u < H) bptr[i] = Rd + int64_t(gate_block(m, gi) * H + j0 + u) * H;
    }
  }
  float4 ring_a[kPF][kAPer], ring_b[kPF][kBPer];
  auto fetch = [&](int k0, float4* ra, float4* rb) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int k = k0 + aoff[i];
      ra[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (aptr[i]) {
        if (k + kSeg <= H) ra[i] = load4<true>(aptr[i] + k);
        else {
          float t4[4] = {0.f, 0.f, 0.f, 0.f};
          for (int z = 0; z < kSeg && k + z < H; ++z) t4[z] = aptr[i][k + z];
          ra[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int k = k0 + boff[i];
      rb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bptr[i]) {
        if (k + kSeg <= H) rb[i] = load4<VEC>(bptr[i] + k);
        else {
          float t4[4] = {0.f, 0.f, 0.f, 0.f};
          for (int z = 0; z < kSeg && k + z < H; ++z) t4[z] = static_cast<float>(bptr[i][k + z]);
          rb[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
        }
      }
    }
  };
  auto stash = [&](int buf, const float4* ra, const float4* rb) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int q = tid + i * kMThreads;
      if (q < BM * kSegRow) *reinterpret_cast<float4*>(&As[buf][(q / kSegRow) * kLDA + aoff[i]]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int q = tid + i * kMThreads;
      if (q < NC * kSegRow) *reinterpret_cast<float4*>(&Bs[buf][(q / kSegRow) * kLDA + boff[i]]) = rb[i];
    }
  };

  // 16x16 output blocks: wave w owns column blocks w, w+4 (all row blocks of
  // the tile), so its matrix-core instructions alternate between independent
  // accumulators and share each loaded B operand across the row blocks
  constexpr int NBI = BM / 16;
  constexpr int CB = kMaxNC / 16 / 4;
  const int ncb = NC / 16;
  f32x4 acc[CB][NBI];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) acc[cb][bi] = f32x4{0.f, 0.f, 0.f, 0.f};

  // k loop with kPF chunks in flight: chunk c lives in ring slot c % kPF from
  // its fetch (iteration c - kPF) until it is staged in LDS (iteration c - 1)
  const int nk = (H + kBK - 1) / kBK;
#pragma unroll
  for (int u = 0; u < kPF; ++u)
    if (u < nk) fetch(u * kBK, ring_a[u], ring_b[u]);
  stash(0, ring_a[0], ring_b[0]);
  __syncthreads();
  for (int kc0 = 0; kc0 < nk; kc0 += kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      const int kc = kc0 + u;
      if (kc >= nk) break;
      const int buf = kc & 1;
      const float* A = As[buf];
      const float* Bm = Bs[buf];
      float av[NBI][kBK / 4];
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
        for (int kk = 0; kk < kBK / 4; ++kk) av[bi][kk] = A[(bi * 16 + (lane & 15)) * kLDA + 4 * kk + (lane >> 4)];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int ci = wave + 4 * cb;
        if (ci >= ncb) break;
        float bv[kBK / 4];
#pragma unroll
        for (int kk = 0; kk < kBK / 4; ++kk) bv[kk] = Bm[(ci * 16 + (lane & 15)) * kLDA + 4 * kk + (lane >> 4)];
#pragma unroll
        for (int kk = 0; kk < kBK / 4; ++kk)
#pragma unroll
          for (int bi = 0; bi < NBI; ++bi)
            acc[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[bi][kk], bv[kk], acc[cb][bi], 0, 0, 0);
      }
      const int nx = (u + 1) % kPF;
      if (kc + 1 < nk) stash(buf ^ 1, ring_a[nx], ring_b[nx]);
      // slot u held chunk kc, staged an iteration ago: it receives chunk kc + kPF
      if (kc + kPF < nk) fetch((kc + kPF) * kBK, ring_a[u], ring_b[u]);
      __syncthreads();
    }
  }

  // accumulator layout of 16x16x4: element i of lane l is row 4*(l/16) + i, column l%16
  constexpr int LDR = kMaxNC + 1;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int ci = wave + 4 * cb;
    if (ci >= ncb) break;
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rec[(bi * 16 + 4 * (lane >> 4) + i) * LDR + ci * 16 + (lane & 15)] = acc[cb][bi][i];
  }
  __syncthreads();

  mfma_epilogue<T, BM>(m, rec, len_s, b0, j0, d);
}

// f16 R on the f16 matrix cores.  R is exact in f16; each f32 value of h is
// split into hi = f16(h) and lo = f16(h - hi), and the product is taken as
// R.hi + R.lo with v_mfma_f32_16x16x32_f16 (f16 products are exact in f32,
// f32 accumulation; the two sums are kept apart and added once at the end), so
// the only loss is lo's own rounding, about 2^-22 of |h|.
// Used when every activation is the ONNX default, which keeps |h| within the
// f16 range (|h| <= max(1, |initial h|)).
constexpr int kBK16 = 128;           // k chunk (f16 path)
constexpr int kLDH = kBK16 + 8;      // padded LDS row (halves)

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));

template <int BM, bool VEC>
__global__ __launch_bounds__(kMThreads) void step_mfma_h16_kernel(MfmaStepArgs m) {
  const StepArgs& a = m.a;
  const int H = a.H, B = a.B, G = a.G, S = a.S;
  const int s = m.step;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.x * m.UJ;
  const int b0 = blockIdx.y * BM;
  const int d = blockIdx.z;
  const int UJ = m.UJ, NC = m.Gp * UJ;

  __shared__ int len_s[BM];
  __shared__ int any_s;
  if (tid == 0) any_s = 0;
  __syncthreads();
  for (int r = tid; r < BM; r += kMThreads) {
    const int b = b0 + r;
    len_s[r] = b < B ? row_length(a.lens, b, S, a.steps) : 0;
    if (s < len_s[r]) atomicOr(&any_s, 1);
  }
  __syncthreads();
  if (!any_s) return;

  // staging buffers; the product tile rec reuses their space after the k loop
  constexpr int kAHalves = BM * kLDH, kBHalves = kMaxNC * kLDH;
  constexpr int kPool = (4 * kAHalves + 2 * kBHalves) * 2;
  static_assert(BM * (kMaxNC + 1) * 4 <= kPool, "product tile must fit in the staging space");
  __shared__ __attribute__((aligned(16))) unsigned char pool[kPool];
  half_t (*Ahi)[kAHalves] = reinterpret_cast<half_t (*)[kAHalves]>(pool);
  half_t (*Alo)[kAHalves] = reinterpret_cast<half_t (*)[kAHalves]>(pool + 2 * kAHalves * 2);
  half_t (*Bh)[kBHalves] = reinterpret_cast<half_t (*)[kBHalves]>(pool + 4 * kAHalves * 2);
  float* rec = reinterpret_cast<float*>(pool);

  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  const bool cand_phase = a.cell == RNN_CELL_GRU && !a.lbr && m.phase == 1;
  const float* hsrc = cand_phase ? a.rhbuf + dBH : a.hbuf + int64_t(s & 1) * DBH + dBH;
  const half_t* Rd = static_cast<const half_t*>(a.R) + int64_t(d) * G * H * H;

  // A: segments of 4 f32 (16 bytes); B: segments of 8 halves (16 bytes)
  constexpr int kASegRow = kBK16 / 4, kBSegRow = kBK16 / 8;
  constexpr int kAPer = (BM * kASegRow + kMThreads - 1) / kMThreads;
  constexpr int kBPer = (kMaxNC * kBSegRow + kMThreads - 1) / kMThreads;
  const float* aptr[kAPer];
  const half_t* bptr[kBPer];
  int aoff[kAPer], boff[kBPer];
#pragma unroll
  for (int i = 0; i < kAPer; ++i) {
    const int q = tid + i * kMThreads;
    const int r = q / kASegRow;
    aoff[i] = (q % kASegRow) * 4;
    const bool ok = q < BM * kASegRow && b0 + r < B && s < len_s[r];
    aptr[i] = ok ? hsrc + int64_t(b0 + r) * H : nullptr;
  }
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int q = tid + i * kMThreads;
    const int c = q / kBSegRow;
    boff[i] = (q % kBSegRow) * 8;
    bptr[i] = nullptr;
    if (q < NC * kBSegRow) {
      const int gi = c / UJ, u = c - gi * UJ;
      if (j0 + u < H) bptr[i] = Rd + int64_t(gate_block(m, gi) * H + j0 + u) * H;
    }
  }
  float4 ring_a[kPF][kAPer];
  h16x8 ring_b[kPF][kBPer];
  auto fetch = [&](int k0, float4* ra, h16x8* rb) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int k = k0 + aoff[i];
      ra[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (aptr[i]) {
        if (k + 4 <= H) ra[i] = *reinterpret_cast<const float4*>(aptr[i] + k);
        else {
          float t4[4] = {0.f, 0.f, 0.f, 0.f};
          for (int z = 0; z < 4 && k + z < H; ++z) t4[z] = aptr[i][k + z];
          ra[i] = make_float4(t4[0], t4[1], t4[2], t4[3]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int k = k0 + boff[i];
      h16x8 v;
#pragma unroll
      for (int z = 0; z < 8; ++z) v[z] = half_t(0.f);
      if (bptr[i]) {
        if (VEC && k + 8 <= H) v = *reinterpret_cast<const h16x8*>(bptr[i] + k);
        else
          for (int z = 0; z < 8 && k + z < H; ++z) v[z] = bptr[i][k + z];
      }
      rb[i] = v;
    }
  };
  auto stash = [&](int buf, const float4* ra, const h16x8* rb) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int q = tid + i * kMThreads;
      if (q < BM * kASegRow) {
        const float x[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
        h16x4 hi, lo;
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          hi[z] = half_t(x[z]);
          lo[z] = half_t(x[z] - float(hi[z]));
        }
        const int off = (q / kASegRow) * kLDH + aoff[i];
        *reinterpret_cast<h16x4*>(&Ahi[buf][off]) = hi;
        *reinterpret_cast<h16x4*>(&Alo[buf][off]) = lo;
      }
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) {
      const int q = tid + i * kMThreads;
      if (q < NC * kBSegRow) *reinterpret_cast<h16x8*>(&Bh[buf][(q / kBSegRow) * kLDH + boff[i]]) = rb[i];
    }
  };

  // wave w owns column blocks w, w+4 and all row blocks; the hi and lo
  // products accumulate separately (independent chains) and are added at the end
  constexpr int NBI = BM / 16;
  constexpr int CB = kMaxNC / 16 / 4;
  const int ncb = NC / 16;
  f32x4 acc_hi[CB][NBI], acc_lo[CB][NBI];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) acc_hi[cb][bi] = acc_lo[cb][bi] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (H + kBK16 - 1) / kBK16;
#pragma unroll
  for (int u = 0; u < kPF; ++u)
    if (u < nk) fetch(u * kBK16, ring_a[u], ring_b[u]);
  stash(0, ring_a[0], ring_b[0]);
  __syncthreads();
  for (int kc0 = 0; kc0 < nk; kc0 += kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      const int kc = kc0 + u;
      if (kc >= nk) break;
      const int buf = kc & 1;
      constexpr int KS = kBK16 / 32;
      h16x8 ah[NBI][KS], al[NBI][KS];
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int ao = (bi * 16 + (lane & 15)) * kLDH + 8 * (lane >> 4) + 32 * kk;
          ah[bi][kk] = *reinterpret_cast<const h16x8*>(&Ahi[buf][ao]);
          al[bi][kk] = *reinterpret_cast<const h16x8*>(&Alo[buf][ao]);
        }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int ci = wave + 4 * cb;
        if (ci >= ncb) break;
        h16x8 bv[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          bv[kk] = *reinterpret_cast<const h16x8*>(&Bh[buf][(ci * 16 + (lane & 15)) * kLDH + 8 * (lane >> 4) + 32 * kk]);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
          for (int bi = 0; bi < NBI; ++bi) {
            acc_hi[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[bi][kk], bv[kk], acc_hi[cb][bi], 0, 0, 0);
            acc_lo[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[bi][kk], bv[kk], acc_lo[cb][bi], 0, 0, 0);
          }
      }
      const int nx = (u + 1) % kPF;
      if (kc + 1 < nk) stash(buf ^ 1, ring_a[nx], ring_b[nx]);
      // slot u held chunk kc, staged an iteration ago: it receives chunk kc + kPF
      if (kc + kPF < nk) fetch((kc + kPF) * kBK16, ring_a[u], ring_b[u]);
      __syncthreads();
    }
  }

  // accumulator layout of the 16x16 MFMA: element i of lane l is row 4*(l/16) + i, column l%16
  constexpr int LDR = kMaxNC + 1;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int ci = wave + 4 * cb;
    if (ci >= ncb) break;
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rec[(bi * 16 + 4 * (lane >> 4) + i) * LDR + ci * 16 + (lane & 15)] = acc_hi[cb][bi][i] + acc_lo[cb][bi][i];
  }
  __syncthreads();
  mfma_epilogue<half_t, BM>(m, rec, len_s, b0, j0, d);
}

// Tile shape (BM batch rows, UJ units): the largest tile that still gives at
// least 256 workgroups, so every compute unit has work.  RNN_MFMA_TILE=BMxUJ
// (BM, UJ in 16, 32, 64; Gp*UJ <= 128) overrides the choice, so that tests
// can reach every tile on small layers.
void mfma_tile(int B, int H, int D, int Gp, int* bm, int* uj) {
  if (const char* e = std::getenv("RNN_MFMA_TILE")) {
    int fb = 0, fu = 0;
    if (std::sscanf(e, "%dx%d", &fb, &fu) == 2 && (fb == 16 || fb == 32 || fb == 64) &&
        (fu == 16 || fu == 32 || fu == 64) && Gp * fu <= kMaxNC) {
      *bm = fb;
      *uj = fu;
      return;
    }
  }
  static const int cand[][2] = {{64, 64}, {64, 32}, {32, 32}, {32, 16}, {16, 16}};
  for (const auto& c : cand) {
    if (Gp * c[1] > kMaxNC) continue;
    const long wgs = long((B + c[0] - 1) / c[0]) * ((H + c[1] - 1) / c[1]) * D;
    *bm = c[0];
    *uj = c[1];
    if (wgs >= 256) return;
  }
}

// Batches above eight (the small-batch engine takes eight and fewer): 16-row
// blocks, the rows past the batch read as zeros and their outputs dropped.
bool mfma_step_supported(const Problem& p) { return p.B >= 9; }

template <typename T, int BM>
static hipError_t launch_bm(const MfmaStepArgs& m, int H, int B, int D, hipStream_t s) {
  const dim3 grid(unsigned((H + m.UJ - 1) / m.UJ), unsigned((B + BM - 1) / BM), unsigned(D));
  if (grid.y > 65535) return hipErrorInvalidValue;
  // vector loads of R need every row start aligned to a whole segment
  const bool vec = (reinterpret_cast<uintptr_t>(m.a.R) % (kSeg * sizeof(T))) == 0 && H % kSeg == 0;
  if (vec)
    hipLaunchKernelGGL((step_mfma_kernel<T, BM, true>), grid, dim3(kMThreads), 0, s, m);
  else
    hipLaunchKernelGGL((step_mfma_kernel<T, BM, false>), grid, dim3(kMThreads), 0, s, m);
  return hipGetLastError();
}

template <int BM>
static hipError_t launch_h16(const MfmaStepArgs& m, int H, int B, int D, hipStream_t s) {
  const dim3 grid(unsigned((H + m.UJ - 1) / m.UJ), unsigned((B + BM - 1) / BM), unsigned(D));
  if (grid.y > 65535) return hipErrorInvalidValue;
  const bool vec = (reinterpret_cast<uintptr_t>(m.a.R) % 16) == 0 && H % 8 == 0;
  if (vec)
    hipLaunchKernelGGL((step_mfma_h16_kernel<BM, true>), grid, dim3(kMThreads), 0, s, m);
  else
    hipLaunchKernelGGL((step_mfma_h16_kernel<BM, false>), grid, dim3(kMThreads), 0, s, m);
  return hipGetLastError();
}

// Arguments of phase `ph` of a step (a GRU with linear_before_reset = 0 has
// two: z and r, then the candidate) and the tile's batch rows.
static MfmaStepArgs phase_args(const StepArgs& a, const Problem& p, int step, int ph, int* bm) {
  const bool skip_f = a.cell == RNN_CELL_LSTM && a.input_forget;
  const bool two_phase = a.cell == RNN_CELL_GRU && !a.lbr;
  MfmaStepArgs m{};
  m.a = a;
  m.step = step;
  m.phase = ph;
  int gi = 0;
  for (int g = 0; g < a.G; ++g) {
    if (skip_f && g == 2) continue;
    if (two_phase && ph == 0 && g == 2) continue;
    if (two_phase && ph == 1 && g != 2) continue;
    m.gate_of[gi++] = g;
  }
  m.Gp = gi;
  *bm = p.mfma_bm;
  m.UJ = p.mfma_uj;
  return m;
}

// Mode of the matrix-core step: 2 (f32 on the bf16 matrix cores, chosen when
// the problem is created), 1 (f16 tensors, default activations), 0 (f32).
static int step_mode(const Problem& p) {
  return p.f32_split_step ? 2 : (p.desc.dtype == RNN_DTYPE_F16 && p.def_acts) ? 1 : 0;
}

hipError_t launch_step_mfma(const StepArgs& a, const Problem& p, int step, hipStream_t s) {
  const bool two_phase = a.cell == RNN_CELL_GRU && !a.lbr;
  for (int ph = 0; ph < (two_phase ? 2 : 1); ++ph) {
    int bm = 16;
    const MfmaStepArgs m = phase_args(a, p, step, ph, &bm);
    hipError_t e;
    const bool h16 = a.dtype == RNN_DTYPE_F16 && p.def_acts;
    const int mode = step_mode(p);
    if (mode == 2 || ((h16 || a.dtype == RNN_DTYPE_F32) && step_dma_supported(a, mode))) {
      e = launch_step_dma(m, bm, mode, s);
    } else if (h16) {
      e = bm == 64 ? launch_h16<64>(m, a.H, a.B, a.D, s)
                   : bm == 32 ? launch_h16<32>(m, a.H, a.B, a.D, s) : launch_h16<16>(m, a.H, a.B, a.D, s);
    } else if (a.dtype == RNN_DTYPE_F32) {
      e = bm == 64 ? launch_bm<float, 64>(m, a.H, a.B, a.D, s)
                   : bm == 32 ? launch_bm<float, 32>(m, a.H, a.B, a.D, s) : launch_bm<float, 16>(m, a.H, a.B, a.D, s);
    } else {
      e = bm == 64 ? launch_bm<half_t, 64>(m, a.H, a.B, a.D, s)
                   : bm == 32 ? launch_bm<half_t, 32>(m, a.H, a.B, a.D, s) : launch_bm<half_t, 16>(m, a.H, a.B, a.D, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The persistent form of the matrix-core step takes a problem when the
// direct-to-LDS kernel takes its shape in its mode and the tiles fit the chip
// one workgroup per compute unit (its LDS allows no more).  R's alignment is
// only known at encode time: launch_step_mfma_persistent reports
// hipErrorNotSupported when it rules the kernel out, and the caller then
// launches per step.
bool mfma_persistent_supported(const Problem& p, int* tiles_out) {
  if (!mfma_step_supported(p) || p.S < 1 || p.steps < 1) return false;
  const int mode = step_mode(p);
  if (mode == 0 && p.desc.dtype == RNN_DTYPE_F16) return false;   // f16 R widened: the register-staged kernel
  StepArgs t{};
  t.G = p.G;
  t.D = p.D;
  t.H = int(p.H);
  t.B = int(p.B);
  if (!step_dma_supported(t, mode)) return false;
  const int bm = p.mfma_bm, uj = p.mfma_uj;
  const int64_t tiles = ((p.H + uj - 1) / uj) * ((p.B + bm - 1) / bm) * p.D;
  if (tiles > kPersistentMfmaTiles) return false;
  *tiles_out = int(tiles);
  return true;
}

hipError_t launch_step_mfma_persistent(const StepArgs& a, const Problem& p, int* flags, int* status, hipStream_t s) {
  const int mode = step_mode(p);
  if (mode != 2 && !step_dma_supported(a, mode)) return hipErrorNotSupported;
  const int P = (a.cell == RNN_CELL_GRU && !a.lbr) ? 2 : 1;
  MfmaStepArgs ph[2];
  int bm = 16;
  for (int k = 0; k < P; ++k) ph[k] = phase_args(a, p, 0, k, &bm);
  return launch_step_dma_persistent(ph, P, bm, mode, flags, status, s);
}

}  // namespace rnnhip

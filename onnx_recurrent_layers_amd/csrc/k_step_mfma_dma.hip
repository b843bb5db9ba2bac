// k_step_mfma_dma.hip -- the matrix-core step (stage 3 of a layer,
// "Recurrent layers" page, "How a layer runs", item 3) for hidden sizes that
// are whole 16-byte segments: h rows and R rows go from global memory straight
// into LDS with buffer loads carrying the LDS bit, several k chunks ahead of
// the matrix cores, so no register staging and no per-element bounds branches.
//
// Tile and arithmetic are those of the other matrix-core step: a workgroup
// owns BM batch rows x UJ units of one direction with all Gp gate blocks of
// those units (product tile [BM] x [Gp*UJ], K = H), and finishes the gate
// arithmetic itself.  Three modes:
//   mode 0, f32 tensors: v_mfma_f32_16x16x4_f32 on f32 h and f32 R;
//   mode 1, f16 tensors with the default activations: h as f16 halves
//     hi = f16(h) and lo = f16(h - hi) (written by the step that produced h),
//     R.hi + R.lo on v_mfma_f32_16x16x32_f16 with separate f32 accumulators
//     (f16 products are exact in f32);
//   mode 2, large f32 layers: h and R as bf16 hi/lo planes (R split once per
//     layer, h by the step that produces it), each product taken as
//     lo_h.hi_R + hi_h.lo_R + hi_h.hi_R on v_mfma_f32_16x16x32_bf16 with one
//     f32 accumulator: bf16 x bf16 products are exact in f32, and what the
//     split drops is below 2^-16 of each |h.R|.
// The k order is fixed (chunks in increasing order, a fixed order within a
// chunk), so runs are bit-identical.
//
// Loads: one buffer resource per operand (h of this direction, R of this
// direction).  A segment that lies outside the tile (rows past the batch or
// the tile's gate rows, k past H) gets an offset beyond the resource's size,
// which the hardware answers with zeros and no memory traffic.  Each wave
// issues the same number of loads per chunk, so the wait for a chunk is a
// fixed vector-memory count.
//
// LDS layout of a chunk: rows of 16-byte segments, unpadded; the segment of
// logical index s of row r is stored at slot s ^ w(r & 15), w(r) = r for
// rows of 16 segments and r with bit 0 copied to bit 4 for the 32-segment h
// rows of the f16 mode, so that the 32 lanes of a half-wave operand read land
// in 32 different 16-byte bank groups.  The k index is permuted inside a
// chunk (step kk of lane group q takes segment 4kk + q), identically for h
// and R, so each lane reads whole 16-byte segments; a sum over a permuted k
// range is the same sum.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "residency.h"
#include "step_mfma.h"

namespace rnnhip {

typedef _Float16 hx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bx8 __attribute__((ext_vector_type(8)));


constexpr unsigned kOutOfRange = 0x80000000u;   // beyond every resource size used here
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format (gfx9 family)
constexpr int kLdsBudget = 144 * 1024;          // staging bytes per workgroup
// R resident in LDS (persistent form, f16 mode): the tile's R rows for every
// k chunk, loaded once per layer; the chunk slots then carry h alone.
constexpr int kRresBytes = 104 * 1024;

// s_waitcnt immediate of the gfx9 encoding: vector-memory count vm (6 bits,
// split), export count left open, LDS count lgkm.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Wait until at most VM of this wave's vector-memory loads are outstanding and
// its LDS accesses are done, then meet the other waves.  The empty asm
// statements keep the compiler from moving memory accesses across.
template <int VM>
__device__ __forceinline__ void chunk_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Slot of segment s of LDS row r is s ^ row_swizzle(r & 15) (see above).
template <int MODE>
__device__ __forceinline__ int row_swizzle(int r) {
  return MODE == 1 ? r | ((r & 1) << 4) : r;
}

// Scheduling of one chunk's instructions: its D operand reads first, then
// the L loads of a later chunk spread between its M matrix-core products (a
// wave issues in order, so loads grouped ahead of the products hold the
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

template <int MODE> struct DmaGeo;
template <> struct DmaGeo<0> {           // f32 h, f32 R
  typedef float RT;
  static constexpr int KC = 64;          // k per chunk
  static constexpr int ASEGS = 16;       // 16-byte segments per h row of a chunk
  static constexpr int BELEMS = 4;       // R elements per segment
};
template <> struct DmaGeo<1> {           // f16 halves of h, f16 R
  typedef half_t RT;
  static constexpr int KC = 128;
  static constexpr int ASEGS = 32;       // a row of a chunk: 16 hi segments, then 16 lo segments
  static constexpr int BELEMS = 8;
};
template <> struct DmaGeo<2> {           // bf16 hi/lo planes of h and R (f32 tensors)
  typedef float RT;
  static constexpr int KC = 64;          // a row of a chunk: 8 hi segments, then 8 lo segments
  static constexpr int ASEGS = 16;
  static constexpr int BELEMS = 8;
};

template <int MODE, int BM, int CB, bool RR = false>
struct DmaCfg {
  typedef DmaGeo<MODE> Geo;
  static constexpr int A_BYTES = BM * Geo::ASEGS * 16;
  static constexpr int B_BYTES = RR ? 0 : CB * 4 * 16 * 256;    // 16 rows x 16 segments per column block
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int REC = BM * (kMaxNC + 1) * 4;             // product tile, over slot 0
  static constexpr int BUDGET = kLdsBudget - (RR ? kRresBytes : 0);
  static constexpr int NS0 = (BUDGET - (REC > STAGE ? REC - STAGE : 0)) / STAGE;
  static constexpr int NS = NS0 > 4 ? 4 : NS0;                  // chunks resident (NS - 1 in flight)
  static constexpr int LA = A_BYTES / 1024 / 4;                 // h loads per wave per chunk
  static constexpr int LB = RR ? 0 : 4 * CB;                    // R loads per wave per chunk
  static constexpr int L = LA + LB;
  static_assert(NS >= 2, "two chunks must fit in LDS");
  static_assert((A_BYTES / 1024) % 4 == 0, "h loads must split evenly over the four waves");
  static_assert((NS - 2) * L < 64, "wait count must fit the counter");
};

// Operands of the gate arithmetic of one (batch row, unit) element besides
// its recurrent products.  They do not depend on the product, so the first
// element of each thread is gathered before the k loop and its loads overlap
// the matrix work.
struct EpiIn {
  float xv[4];     // Xw of the computed gate blocks
  unsigned wb[4];  // Wb of those blocks as loaded (0 without B); widened at use,
  unsigned rb[4];  //   so that waiting for the loads is left to the arithmetic
  unsigned pp[3];  // P_i, P_o, P_f (LSTM), likewise
  float cprev;     // LSTM cell state
  float hprev;     // GRU previous hidden state
  float z;         // GRU linear_before_reset = 0, second pass: z of the first
  int len;         // the row's length
  bool live;       // the element exists and its row still runs at this step
};

// Everything the gate arithmetic of one direction needs, read out of the
// launch arguments once at the start (uniform values).  The arithmetic then
// touches the argument block nowhere: when many inlined copies of it index
// the block, the compiler stops reading the block in place and copies it to
// scratch memory.
struct EpiCtx {
  __amdgpu_buffer_rsrc_t bias, peep;   // absent vector: size 0, loads return zeros without traffic
  const float* xw;      // the projection slab of this step and direction, [B][G*H]
  const float* hprev;   // h of this step, [B][H]
  float* hnext;         // h of the next step, [B][H]
  bool h32;             // hnext is written: its readers are the f32 mode's product and the GRU gates;
                        // the other cells of the split modes read h only as 16-bit halves
  void* Y;              // outputs (or null), written as the step finishes each element
  void* Y_h;
  void* Y_c;
  float* cst;           // LSTM cell state, [B][H]
  float* zbuf;          // GRU z of the first pass, [B][H]
  float* rhbuf;         // GRU r*h, [B][H]
  unsigned short* hsn;  // mode 2: h of the next step as bf16 hi/lo planes (lo at +DBH), or null
  unsigned short* rhs;  // mode 2: GRU r*h as bf16 hi/lo planes, or null
  int64_t DBH;
  float clip;
  int H, B, GH, s, cell, lbr, phase, input_forget, has_p, rev, Gp;
  int S, D, d, layout;
  bool coh;             // persistent launch: state read and written at device scope
  int split_kind;       // of hsn / rhs: 1 f16 halves, 2 bf16 halves
  int gate[4];
  Act act[3];
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

template <typename RT>
__device__ __forceinline__ EpiCtx epi_context(const MfmaStepArgs& m, int d, int step, bool coh) {
  const StepArgs& a = m.a;
  EpiCtx c;
  c.H = a.H;
  c.B = a.B;
  c.GH = a.G * a.H;
  c.s = step;
  c.coh = coh;
  c.cell = a.cell;
  c.lbr = a.lbr;
  c.phase = m.phase;
  c.input_forget = a.input_forget;
  c.has_p = a.P != nullptr;
  c.rev = uniform(a.dir_reverse[d]);
  c.Gp = m.Gp;
  c.clip = a.clip;
#pragma unroll
  for (int k = 0; k < 4; ++k) c.gate[k] = uniform(m.gate_of[k]);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int i = d * a.slots + (k < a.slots ? k : 0);
    c.act[k].kind = uniform(a.act[i].kind);
    c.act[k].alpha = uniform(a.act[i].alpha);
    c.act[k].beta = uniform(a.act[i].beta);
  }
  const int64_t DBH = int64_t(a.D) * a.B * a.H, dBH = int64_t(d) * a.B * a.H;
  c.xw = xw_slab(a, d, step);
  c.hprev = a.hbuf + int64_t(step & 1) * DBH + dBH;
  c.hnext = a.hbuf + int64_t((step + 1) & 1) * DBH + dBH;
  c.Y = a.Y;
  c.Y_h = a.Y_h;
  c.Y_c = a.Y_c;
  c.S = a.S;
  c.D = a.D;
  c.d = d;
  c.layout = a.layout;
  c.cst = a.cell_state + dBH;
  c.DBH = DBH;
  c.hsn = a.hsplit ? a.hsplit + int64_t((step + 1) & 1) * 2 * DBH + dBH : nullptr;
  // (the persistent form keeps the store: without it C4's shape measured
  // slower, its schedule being what it is)
  c.h32 = coh || !c.hsn || a.cell == RNN_CELL_GRU;
  c.rhs = a.rhsplit ? a.rhsplit + dBH : nullptr;
  c.split_kind = a.split_kind;
  c.zbuf = a.zbuf + dBH;
  c.rhbuf = a.rhbuf + dBH;
  const RT* bias = a.bias ? static_cast<const RT*>(a.bias) + int64_t(d) * 2 * c.GH : nullptr;
  const RT* P = a.P ? static_cast<const RT*>(a.P) + int64_t(d) * 3 * a.H : nullptr;
  c.bias = __builtin_amdgcn_make_buffer_rsrc(const_cast<RT*>(bias), 0, bias ? 2 * c.GH * int(sizeof(RT)) : 0, kRsrcWord3);
  c.peep = __builtin_amdgcn_make_buffer_rsrc(const_cast<RT*>(P), 0, P ? 3 * a.H * int(sizeof(RT)) : 0, kRsrcWord3);
  return c;
}

// State that a launch both writes and reads (h, c, z, r*h and their bf16
// planes).  In a persistent launch it goes through device scope (cache
// policy sc1): other workgroups, on other XCDs, read h between steps, and a
// workgroup's own values come back to it through caches that other traffic
// went through.  A per-step launch needs nothing of the kind: kernel
// boundaries order and publish everything.
__device__ __forceinline__ float st_ld(const float* p, bool coh) {
  return coh ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
}
__device__ __forceinline__ void st_st(float* p, float v, bool coh) {
  if (coh) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
__device__ __forceinline__ void st_split(unsigned short* p, int64_t plane, float v, bool coh, int kind) {
  unsigned short hi, lo;
  split_bits(kind, v, hi, lo);
  if (coh) {
    __hip_atomic_store(p, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + plane, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    p[0] = hi;
    p[plane] = lo;
  }
}

// f16 elements are loaded as the aligned dword that holds them (the vectors
// have an even length), so that no conversion sits at the load; widen() picks
// the half by the parity of the element index.
template <typename RT>
__device__ __forceinline__ unsigned res_load(__amdgpu_buffer_rsrc_t r, int idx) {
  if constexpr (sizeof(RT) == 2) return __builtin_amdgcn_raw_buffer_load_b32(r, (idx * 2) & ~3, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, 0);
}

template <typename RT>
__device__ __forceinline__ float widen(unsigned v, int odd) {
  if constexpr (sizeof(RT) == 2) return float(__builtin_bit_cast(half_t, (unsigned short)(v >> (odd * 16))));
  else return __builtin_bit_cast(float, v);
}

// Element e of the tile is row e >> ujs, unit e & (UJ - 1); elements from
// n_el on do not exist.
template <typename RT, bool INIT = false>
__device__ __forceinline__ void epi_gather(const EpiCtx& c, const int* len_s, int e, int n_el, int ujs, int b0, int j0,
                                           EpiIn& o) {
  const int H = c.H, s = c.s;
  const int r = e >> ujs, u = e & ((1 << ujs) - 1);
  const int b = b0 + r, j = j0 + u;
  const int L = e < n_el ? len_s[r] : 0;
  o.len = L;
  o.live = b < c.B && j < H && s < L;
  // INIT: every field defined on every path, so that the struct stays in
  // registers.  In the persistent kernel, fields left unset on some paths
  // kept the state loads in scratch memory, with a wait for each right where
  // it was issued (C4 1.71 -> 1.61 ms with INIT); in the per-step kernel
  // the same initialisation cost C5 2 %.
  if constexpr (INIT) {
    o.cprev = 0.f;
    o.hprev = 0.f;
    o.z = 0.f;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      o.xv[gi] = 0.f;
      o.wb[gi] = 0u;
      o.rb[gi] = 0u;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) o.pp[k] = 0u;
  }
  if (j >= H) return;
  // the unit's biases and peepholes, also for a row that does not run: the
  // thread's later elements (same unit) take them from here
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    if (gi >= c.Gp) break;
    const int n = c.gate[gi] * H + j;
    o.wb[gi] = res_load<RT>(c.bias, n);
    o.rb[gi] = res_load<RT>(c.bias, c.GH + n);
  }
  if (c.cell == RNN_CELL_LSTM) {
#pragma unroll
    for (int k = 0; k < 3; ++k) o.pp[k] = res_load<RT>(c.peep, k * H + j);
  }
  if (!o.live) return;
  const float* xw = c.xw + int64_t(b) * c.GH;
  const int64_t si = int64_t(b) * H + j;
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    if (gi >= c.Gp) break;
    o.xv[gi] = xw[c.gate[gi] * H + j];
  }
  if (c.cell == RNN_CELL_LSTM) {
    o.cprev = st_ld(c.cst + si, c.coh);
  } else if (c.cell == RNN_CELL_GRU) {
    o.hprev = st_ld(c.hprev + si, c.coh);
    if (!c.lbr && c.phase == 1) o.z = st_ld(c.zbuf + si, c.coh);
  }
}

// h of the next step: f32, and in mode 2 also its bf16 planes.
__device__ __forceinline__ void epi_put_h(const EpiCtx& c, int64_t si, float h) {
  if (c.h32) st_st(c.hnext + si, h, c.coh);
  if (c.hsn) st_split(c.hsn + si, c.DBH, h, c.coh, c.split_kind);
}

// Y of one finished element and, after its row's last step, Y_h / Y_c.
template <typename RT>
__device__ __forceinline__ void epi_outputs(const EpiCtx& c, int b, int j, int L, float h, float cc) {
  const int t = c.rev ? (L - 1 - c.s) : c.s;
  if (c.Y) static_cast<RT*>(c.Y)[y_index(c.layout, c.S, c.D, c.B, c.H, t, c.d, b, j)] = to_elem<RT>(h);
  if (c.s == L - 1) {
    const int64_t si = state_index(c.layout, c.D, c.B, c.H, c.d, b, j);
    if (c.Y_h) static_cast<RT*>(c.Y_h)[si] = to_elem<RT>(h);
    if (c.Y_c) static_cast<RT*>(c.Y_c)[si] = to_elem<RT>(cc);
  }
}

// Gate arithmetic of one gathered element with its products rrow[gi*UJ + u],
// in the order of cells.h.
template <typename RT, bool DEF>
__device__ __forceinline__ void epi_finish(const EpiCtx& c, const EpiIn& o, const float* rec, int e, int ujs, int b0,
                                           int j0) {
  if (!o.live) return;
  constexpr int LDR = kMaxNC + 1;
  const int UJ = 1 << ujs;
  const int r = e >> ujs, u = e & (UJ - 1);
  const int b = b0 + r, j = j0 + u;
  const int64_t si = int64_t(b) * c.H + j;
  const float* rrow = rec + r * LDR + u;
  const Act* acts = c.act;
  const int odd = j & 1;   // every bias and peephole index of unit j has the parity of j (H is even)
  auto pre = [&](int gi) {
    return pre_sum(o.xv[gi], rrow[gi * UJ], widen<RT>(o.wb[gi], odd), widen<RT>(o.rb[gi], odd));
  };
  if (c.cell == RNN_CELL_LSTM) {
    float p4[4];
    p4[0] = pre(0);
    p4[1] = pre(1);
    if (c.input_forget) {            // computed blocks i, o, c
      p4[2] = 0.f;
      p4[3] = pre(2);
    } else {
      p4[2] = pre(2);
      p4[3] = pre(3);
    }
    float h, cc;
    const float pp[3] = {widen<RT>(o.pp[0], odd), widen<RT>(o.pp[1], odd), widen<RT>(o.pp[2], odd)};
    if (c.has_p)   // two calls, so that the peephole array stays in registers
      lstm_unit<DEF>(p4, pp, o.cprev, c.clip, c.input_forget, acts, &h, &cc);
    else
      lstm_unit<DEF>(p4, nullptr, o.cprev, c.clip, c.input_forget, acts, &h, &cc);
    st_st(c.cst + si, cc, c.coh);
    epi_put_h(c, si, h);
    epi_outputs<RT>(c, b, j, o.len, h, cc);
  } else if (c.cell == RNN_CELL_GRU) {
    if (c.lbr) {
      // linear_before_reset = 1: h~ = g(xw_h + r * (rec_h + Rb_h) + Wb_h)
      const float z = gru_gate<DEF>(pre(0), c.clip, acts);
      const float rg = gru_gate<DEF>(pre(1), c.clip, acts);
      const float ph = (o.xv[2] + rg * (rrow[2 * UJ] + widen<RT>(o.rb[2], odd))) + widen<RT>(o.wb[2], odd);
      const float h = gru_unit<DEF>(z, ph, o.hprev, c.clip, acts);
      epi_put_h(c, si, h);
      epi_outputs<RT>(c, b, j, o.len, h, 0.f);
    } else if (c.phase == 0) {
      const float z = gru_gate<DEF>(pre(0), c.clip, acts);
      const float rg = gru_gate<DEF>(pre(1), c.clip, acts);
      st_st(c.zbuf + si, z, c.coh);
      const float rh = rg * o.hprev;
      st_st(c.rhbuf + si, rh, c.coh);
      if (c.rhs) st_split(c.rhs + si, c.DBH, rh, c.coh, c.split_kind);
    } else {
      // linear_before_reset = 0: h~ = g(((xw_h + R_h.(r*h)) + Wb_h) + Rb_h)
      const float h = gru_unit<DEF>(o.z, pre(0), o.hprev, c.clip, acts);
      epi_put_h(c, si, h);
      epi_outputs<RT>(c, b, j, o.len, h, 0.f);
    }
  } else {
    const float h = rnn_unit<DEF>(pre(0), c.clip, acts);
    epi_put_h(c, si, h);
    epi_outputs<RT>(c, b, j, o.len, h, 0.f);
  }
}

constexpr int kMaxEl = 64 * 64 / kMThreads;   // elements per thread of the largest tile (64 rows x 64 units)

// Per-element planes of the elements after each thread's first: Xw of the Gp
// computed blocks, then the state the cell reads (LSTM c, GRU h), then the
// GRU z of the first pass.  Each plane holds n_el floats, element e at e.
__host__ __device__ constexpr int epi_state_planes(int cell, int lbr, int phase) {
  return cell == RNN_CELL_LSTM ? 1 : cell == RNN_CELL_GRU ? 1 + (!lbr && phase == 1) : 0;
}

// Load the planes of elements tid + k*256, k = 1..E-1, straight into LDS
// (every load in flight at once, no registers).  Lane l of a wave writes 4
// bytes at its instruction's base + 4*l, which is element e's slot since the
// wave's 64 elements are consecutive.  Elements that do not run load a valid
// dummy address.
// VEC (the per-step kernel) takes 16-byte loads where it can; the persistent
// kernel keeps the one-value form (its code size and registers measured
// better without the second form).
template <bool VEC>
__device__ __forceinline__ void epi_tile_issue(const EpiCtx& c, const int* len_s, float* planes, int n_el, int ujs,
                                               int b0, int j0) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int ns = epi_state_planes(c.cell, c.lbr, c.phase);
  if (VEC && (c.H & 3) == 0 && uint64_t(c.B) * uint64_t(c.GH) * 4u < uint64_t(kOutOfRange)) {
    // Four consecutive elements (one row, four units) per lane and 16 bytes
    // per load: load w of the workgroup covers elements 256 (w + 1) ..
    // 256 (w + 2) - 1, lane l of it elements + 4l .. + 4l + 3.  An element
    // group that does not run (or reaches past H) reads as zeros.
    const int lane = tid & 63;
    const unsigned bh = unsigned(c.B) * unsigned(c.H) * 4u;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(c.xw), 0, int(unsigned(c.B) * unsigned(c.GH) * 4u), kRsrcWord3);
    const float* st = c.cell == RNN_CELL_LSTM ? c.cst : c.hprev;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(st), 0, int(bh), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(c.zbuf, 0, int(bh), kRsrcWord3);
    const int nw = n_el / kMThreads - 1;   // loads of the workgroup
    for (int w = wave; w < nw; w += kMThreads / 64) {
      const int e = (w + 1) * kMThreads + 4 * lane;
      const int r = e >> ujs, b = b0 + r;
      const int j = j0 + (e & ((1 << ujs) - 1));
      const bool live = b < c.B && j + 3 < c.H && c.s < len_s[r];
      float* dst = planes + (w + 1) * kMThreads;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        if (gi < c.Gp) {
          const unsigned off = live ? (unsigned(b) * unsigned(c.GH) + unsigned(c.gate[gi] * c.H + j)) * 4u : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, RNN_LDS_PTR(dst + gi * n_el), 16, off, 0, 0, 0);
        }
      const unsigned so = live ? (unsigned(b) * unsigned(c.H) + unsigned(j)) * 4u : kOutOfRange;
      if (ns > 0) {
        if (c.coh) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, RNN_LDS_PTR(dst + c.Gp * n_el), 16, so, 0, 0, 16);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, RNN_LDS_PTR(dst + c.Gp * n_el), 16, so, 0, 0, 0);
      }
      if (ns > 1) {
        if (c.coh) __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, RNN_LDS_PTR(dst + (c.Gp + 1) * n_el), 16, so, 0, 0, 16);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, RNN_LDS_PTR(dst + (c.Gp + 1) * n_el), 16, so, 0, 0, 0);
      }
    }
    return;
  }
  const int E = n_el / kMThreads;   // at most kMaxEl
  const int j = j0 + (tid & ((1 << ujs) - 1));   // the same unit for every element of this thread
  // the rows' lengths first, so that the loads below issue back to back
  // instead of each behind an LDS read
  int Ls[kMaxEl];
#pragma unroll
  for (int k = 1; k < kMaxEl; ++k) Ls[k] = k < E ? len_s[(tid + k * kMThreads) >> ujs] : 0;
#pragma unroll
  for (int k = 1; k < kMaxEl; ++k) {
    if (k >= E) break;
    const int e = tid + k * kMThreads;
    const int r = e >> ujs, b = b0 + r;
    const int L = Ls[k];
    const bool live = b < c.B && j < c.H && c.s < L;
    const int64_t row = live ? int64_t(b) * c.GH + j : 0;
    const int64_t si = live ? int64_t(b) * c.H + j : 0;
    float* dst = planes + k * kMThreads + wave * 64;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)   // fixed indices keep the context in registers
      if (gi < c.Gp)
        __builtin_amdgcn_global_load_lds(RNN_GLOBAL_PTR(c.xw + row + (live ? c.gate[gi] * c.H : 0)),
                                         RNN_LDS_PTR(dst + gi * n_el), 4, 0, 0);
    if (ns > 0) {
      const float* st = c.cell == RNN_CELL_LSTM ? c.cst : c.hprev;
      if (c.coh)
        __builtin_amdgcn_global_load_lds(RNN_GLOBAL_PTR(st + si), RNN_LDS_PTR(dst + c.Gp * n_el), 4, 0, 16);
      else
        __builtin_amdgcn_global_load_lds(RNN_GLOBAL_PTR(st + si), RNN_LDS_PTR(dst + c.Gp * n_el), 4, 0, 0);
    }
    if (ns > 1) {
      if (c.coh)
        __builtin_amdgcn_global_load_lds(RNN_GLOBAL_PTR(c.zbuf + si), RNN_LDS_PTR(dst + (c.Gp + 1) * n_el), 4, 0, 16);
      else
        __builtin_amdgcn_global_load_lds(RNN_GLOBAL_PTR(c.zbuf + si), RNN_LDS_PTR(dst + (c.Gp + 1) * n_el), 4, 0, 0);
    }
  }
}

// The elements after each thread's first of a plain RNN cell with a
// non-default activation, its kind fixed at compile time: the same
// arithmetic as epi_finish, without the activation's branches per element.
template <typename RT, int K>
__device__ __forceinline__ void rnn_tile_finish(const EpiCtx& c, const EpiIn& first, const int* len_s, const float* rec,
                                                const float* planes, int n_el, int ujs, int b0, int j0) {
  constexpr int LDR = kMaxNC + 1;
  const int tid = threadIdx.x;
  const int E = n_el / kMThreads;
  const int UJ = 1 << ujs;
  const int u = tid & (UJ - 1), j = j0 + u;
  const int odd = j & 1;
  const float wb = widen<RT>(first.wb[0], odd), rb = widen<RT>(first.rb[0], odd);
  const float al = c.act[0].alpha, be = c.act[0].beta;
  const bool quads = !c.coh && (c.H & 3) == 0 && (reinterpret_cast<uintptr_t>(c.hnext) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(c.hsn) & 7) == 0;
  if (quads) {
    // Four consecutive units of a row per thread and pass: the elements from
    // row 256/UJ on (the rows of each thread's first element done), quad q of
    // them at row 256/UJ + q/QR, units 4(q % QR) ..; a thread keeps its four
    // units (256 is a multiple of QR), so it loads their biases once.  One
    // 16-byte LDS read for their Xw, and h, its halves and Y written with
    // one store each per quad; the arithmetic per element is that of the
    // loop below.
    const int QR = UJ >> 2;
    const int uq = 4 * (tid & (QR - 1)), jq = j0 + uq;
    const int r0 = kMThreads >> ujs;
    const int nq = (n_el - kMThreads) >> 2;
    float wq[4], rq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = c.gate[0] * c.H + jq + i, odd = (jq + i) & 1;
      wq[i] = jq + i < c.H ? widen<RT>(res_load<RT>(c.bias, n), odd) : 0.f;
      rq[i] = jq + i < c.H ? widen<RT>(res_load<RT>(c.bias, c.GH + n), odd) : 0.f;
    }
    const bool yvec = c.Y && (reinterpret_cast<uintptr_t>(c.Y) & (4 * sizeof(RT) - 1)) == 0;
    for (int q = tid; q < nq; q += kMThreads) {
      const int r = r0 + q / QR, b = b0 + r;
      const int L = len_s[r];
      if (!(b < c.B && jq < c.H && c.s < L)) continue;
      const f32x4 xq = *reinterpret_cast<const f32x4*>(planes + (r << ujs) + uq);
      const float* rr = rec + r * LDR + uq;
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[i] = activate_k<K>(al, be, clipf(pre_sum(xq[i], rr[i], wq[i], rq[i]), c.clip));
      const int64_t si = int64_t(b) * c.H + jq;
      if (c.h32) *reinterpret_cast<f32x4*>(c.hnext + si) = f32x4{h[0], h[1], h[2], h[3]};
      if (c.hsn) {
        unsigned short hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_bits(c.split_kind, h[i], hi[i], lo[i]);
        typedef unsigned short us4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<us4*>(c.hsn + si) = us4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<us4*>(c.hsn + si + c.DBH) = us4{lo[0], lo[1], lo[2], lo[3]};
      }
      if (yvec) {
        const int t = c.rev ? (L - 1 - c.s) : c.s;
        RT* y = static_cast<RT*>(c.Y) + y_index(c.layout, c.S, c.D, c.B, c.H, t, c.d, b, jq);
        if constexpr (sizeof(RT) == 4) {
          *reinterpret_cast<f32x4*>(y) = f32x4{h[0], h[1], h[2], h[3]};
        } else {
          typedef _Float16 h4v __attribute__((ext_vector_type(4)));
          *reinterpret_cast<h4v*>(y) = h4v{_Float16(h[0]), _Float16(h[1]), _Float16(h[2]), _Float16(h[3])};
        }
        if (c.s == L - 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t hi2 = state_index(c.layout, c.D, c.B, c.H, c.d, b, jq + i);
            if (c.Y_h) static_cast<RT*>(c.Y_h)[hi2] = to_elem<RT>(h[i]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) epi_outputs<RT>(c, b, jq + i, L, h[i], 0.f);
      }
    }
    return;
  }
  for (int k = 1; k < E; ++k) {
    const int e = tid + k * kMThreads;
    const int r = e >> ujs, b = b0 + r;
    const int L = len_s[r];
    if (!(b < c.B && j < c.H && c.s < L)) continue;
    const float pre = pre_sum(planes[e], rec[r * LDR + u], wb, rb);
    const float h = activate_k<K>(al, be, clipf(pre, c.clip));
    epi_put_h(c, int64_t(b) * c.H + j, h);
    epi_outputs<RT>(c, b, j, L, h, 0.f);
  }
}

// Gate arithmetic of elements k = 1..E-1 from the planes; biases and
// peepholes are those of the thread's first element (same unit).
template <typename RT, bool DEF, bool SPEC = false>
__device__ __forceinline__ void epi_tile_finish(const EpiCtx& c, const EpiIn& first, const int* len_s, const float* rec,
                                                const float* planes, int n_el, int ujs, int b0, int j0) {
  // SPEC (the per-step kernel): a plain RNN cell takes a loop compiled for
  // its activation kind
  if constexpr (SPEC && !DEF) {
    if (c.cell == RNN_CELL_RNN) {
#define RNN_TILE_CASE(K) \
  case K: rnn_tile_finish<RT, K>(c, first, len_s, rec, planes, n_el, ujs, b0, j0); return;
      switch (c.act[0].kind) {
        RNN_TILE_CASE(RNN_ACT_RELU)
        RNN_TILE_CASE(RNN_ACT_TANH)
        RNN_TILE_CASE(RNN_ACT_SIGMOID)
        RNN_TILE_CASE(RNN_ACT_AFFINE)
        RNN_TILE_CASE(RNN_ACT_LEAKY_RELU)
        RNN_TILE_CASE(RNN_ACT_THRESHOLDED_RELU)
        RNN_TILE_CASE(RNN_ACT_SCALED_TANH)
        RNN_TILE_CASE(RNN_ACT_HARD_SIGMOID)
        RNN_TILE_CASE(RNN_ACT_ELU)
        RNN_TILE_CASE(RNN_ACT_SOFTSIGN)
        RNN_TILE_CASE(RNN_ACT_SOFTPLUS)
        default: break;
      }
#undef RNN_TILE_CASE
    }
  }
  const int tid = threadIdx.x;
  const int E = n_el / kMThreads;
  const int j = j0 + (tid & ((1 << ujs) - 1));
  for (int k = 1; k < E; ++k) {
    const int e = tid + k * kMThreads;
    const int r = e >> ujs, b = b0 + r;
    EpiIn o = first;
    o.len = len_s[r];
    o.live = b < c.B && j < c.H && c.s < o.len;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
      if (gi < c.Gp) o.xv[gi] = planes[gi * n_el + e];
    const float sv = planes[c.Gp * n_el + e];
    o.cprev = sv;
    o.hprev = sv;
    o.z = planes[(c.Gp + 1) * n_el + e];
    epi_finish<RT, DEF>(c, o, rec, e, ujs, b0, j0);
  }
}

// One step (one phase of a two-phase GRU step) of tile (tx, ty, tz): units
// tx*UJ.., batch rows ty*BM.., direction tz.  Run by a per-step launch (PERS =
// false) or inside the persistent kernel below (each workgroup its own tile;
// in the fallback one workgroup every tile of a group in turn).  RR: the
// tile's R rows stay in LDS for the whole layer (loaded at step 0, or at
// every call when `reload_r`; the persistent form in f16 mode with one phase
// per step only).
template <int MODE, int BM, int CB, bool PERS, bool RR = false>
__device__ __forceinline__ void dma_step(const MfmaStepArgs& m, int s, int tx, int ty, int tz, bool reload_r = false) {
  static_assert(!RR || (PERS && MODE == 1), "resident R: persistent form, f16 mode");
  typedef DmaCfg<MODE, BM, CB, RR> C;
  typedef typename C::Geo Geo;
  typedef typename Geo::RT RT;
  constexpr int KC = Geo::KC, ASEGS = Geo::ASEGS, BELEMS = Geo::BELEMS;
  constexpr int NS = C::NS, L = C::L, LA = C::LA;
  constexpr int NBI = BM / 16;
  // one LDS object per resident chunk: the compiler then tells the loads
  // into one chunk from the reads of another and waits only for the former
  constexpr int REC_BYTES = BM * (kMaxNC + 1) * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[C::STAGE > REC_BYTES ? C::STAGE : REC_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[NS > 2 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[NS > 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char rres[RR ? kRresBytes : 16];
  __shared__ int len_s[BM];
  __shared__ int any_s;

  const StepArgs& a = m.a;
  const int H = a.H, B = a.B, G = a.G, S = a.S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = tx * m.UJ;
  const int b0 = ty * BM;
  const int d = tz;
  const int UJ = m.UJ, ncb = (m.Gp * UJ) >> 4;
  const int ujs = __builtin_ctz(unsigned(UJ));   // UJ is a power of two

  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  const bool cand_phase = a.cell == RNN_CELL_GRU && !a.lbr && m.phase == 1;
  // operand resources.  Modes 1 and 2 read h as 16-bit planes: the hi plane
  // of this direction, with the lo plane `plane_a` bytes further on, and the
  // resource reaching to the end of this direction's lo plane; mode 2 reads
  // R likewise (`plane_b`).
  __amdgpu_buffer_rsrc_t ra, rb;
  unsigned plane_a = 0, plane_b = 0;
  if constexpr (MODE >= 1) {
    const unsigned short* hs2 = cand_phase ? a.rhsplit + dBH : a.hsplit + int64_t(s & 1) * 2 * DBH + dBH;
    plane_a = unsigned(DBH) * 2u;
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(hs2), 0,
                                           int(plane_a + unsigned(B) * unsigned(H) * 2u), kRsrcWord3);
  } else {
    const float* hsrc = cand_phase ? a.rhbuf + dBH : a.hbuf + int64_t(s & 1) * DBH + dBH;
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(hsrc), 0, int(unsigned(B) * unsigned(H) * 4u),
                                           kRsrcWord3);
  }
  if constexpr (MODE == 2) {
    const unsigned short* rs2 = a.rsplit + int64_t(d) * G * H * H;
    plane_b = unsigned(a.D) * unsigned(G) * unsigned(H) * unsigned(H) * 2u;
    rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(rs2), 0,
                                           int(plane_b + unsigned(G) * unsigned(H) * unsigned(H) * 2u), kRsrcWord3);
  } else {
    const RT* Rd = static_cast<const RT*>(a.R) + int64_t(d) * G * H * H;
    rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<RT*>(Rd), 0,
                                           int(unsigned(G) * unsigned(H) * unsigned(H) * unsigned(sizeof(RT))),
                                           kRsrcWord3);
  }
  constexpr unsigned AES = MODE >= 1 ? 2u : 4u;              // bytes of an element of h as loaded
  constexpr unsigned BES = MODE == 2 ? 2u : unsigned(sizeof(RT));  // ... of R

  // h segments of this lane: load i of the wave fills LDS bytes
  // [(wave*LA + i) * 1024, +1024) of the chunk, lane l the 16 bytes at 16*l
  unsigned arow[LA];
  int aseg[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int p = (wave * LA + i) * 64 + lane;
    const int r = p / ASEGS;
    aseg[i] = (p % ASEGS) ^ row_swizzle<MODE>(r & 15);
    arow[i] = b0 + r < B ? unsigned(b0 + r) * unsigned(H) * AES : kOutOfRange;
  }
  // R segments: wave w owns column blocks w and w + 4 (CB of them); load i of
  // a block fills its rows 4i..4i+3
  unsigned brow[CB][4];
  const int bseg0 = lane & 15;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = wave + 4 * cb;
      const int c = ci * 16 + 4 * i + (lane >> 4);
      const int gi = c >> ujs, u = c & (UJ - 1);
      const bool ok = ci < ncb && j0 + u < H;
      brow[cb][i] = ok ? unsigned(gate_block(m, gi) * H + j0 + u) * unsigned(H) * BES : kOutOfRange;
    }
  auto slot = [&](int i) -> unsigned char* { return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3; };
  const int nk = (H + KC - 1) / KC;
  auto fetch = [&](int kc, unsigned char* st) {
    const int k0 = kc * KC;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      // a row outside the tile starts at the out-of-range marker, so row + k stays out of range
      unsigned off;
      if constexpr (MODE >= 1) {   // logical segment: plane (hi, lo) and 8-element k group
        constexpr int SPP = ASEGS / 2;   // segments of one plane
        const int k = k0 + (aseg[i] % SPP) * 8;
        off = k < H ? arow[i] + unsigned(aseg[i] / SPP) * plane_a + unsigned(k) * 2u : kOutOfRange;
      } else {
        const int k = k0 + aseg[i] * 4;
        off = k < H ? arow[i] + unsigned(k) * 4u : kOutOfRange;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, RNN_LDS_PTR(st + (wave * LA + i) * 1024), 16, off, 0, 0,
                                               PERS ? 16 : 0);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * i + (lane >> 4);
        unsigned off;
        if constexpr (MODE == 2) {
          const int ls = bseg0 ^ rr;
          const int k = k0 + (ls & 7) * 8;
          off = k < H ? brow[cb][i] + (ls >> 3) * plane_b + unsigned(k) * 2u : kOutOfRange;
        } else {
          const int k = k0 + (bseg0 ^ rr) * BELEMS;
          off = k < H ? brow[cb][i] + unsigned(k) * BES : kOutOfRange;
        }
        if constexpr (!RR)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rb, RNN_LDS_PTR(st + C::A_BYTES + ((wave + 4 * cb) * 16 + 4 * i) * 256), 16, off, 0, 0, 0);
      }
  };
  // resident R: chunk kc, column block ci at rres + (kc * ncb + ci) * 4096, in
  // the layout of a chunk's R part; loaded before the first chunks, so the
  // chunk waits (the counter retires in order) cover it
  if constexpr (RR) {
    if (s == 0 || reload_r) {
      for (int kc = 0; kc < nk; ++kc)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int ci = wave + 4 * cb;
          if (ci >= ncb) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = 4 * i + (lane >> 4);
            const int k = kc * KC + (bseg0 ^ rr) * BELEMS;
            const unsigned off = k < H ? brow[cb][i] + unsigned(k) * BES : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, RNN_LDS_PTR(rres + ((kc * ncb + ci) * 16 + 4 * i) * 256), 16,
                                                     off, 0, 0, 0);
          }
        }
    }
  }

  // lengths of the tile's rows (wave 0); the load overlaps the first chunks
  int lv = 0;
  if (wave == 0 && lane < BM && b0 + lane < B) lv = a.lens ? a.lens[b0 + lane] : S;

#pragma unroll
  for (int c = 0; c < NS - 1; ++c) fetch(c, slot(c));

  if (wave == 0) {
    const int L_ = lv < 0 ? 0 : (lv > S ? S : lv);
    const int Lr = L_ < a.steps ? L_ : a.steps;
    if (lane < BM) len_s[lane] = Lr;
    const unsigned long long live = __ballot(lane < BM && s < Lr);
    if (lane == 0) any_s = live != 0ull;
  }

  const int q = lane >> 4, r16 = lane & 15;
  f32x4 acc[CB][NBI];
  f32x4 acc_lo[MODE == 1 ? CB : 1][MODE == 1 ? NBI : 1];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) acc[cb][bi] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == 1) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi) acc_lo[cb][bi] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  chunk_barrier<(NS - 1) * L>();      // the lengths are visible
  if (!any_s) {                       // every row of the tile has ended
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    return;
  }
  const EpiCtx ctx = epi_context<RT>(m, d, s, PERS);
  const int n_el = BM * UJ;   // a multiple of the workgroup size
  EpiIn first;
  epi_gather<RT, PERS>(ctx, len_s, tid, n_el, ujs, b0, j0, first);

  // chunk kc lives in slot kc % NS; the loop is unrolled over the slots so
  // that every slot is a fixed LDS object.  The chunk count is rounded up to
  // whole rounds of NS: chunks past the end hold zeros and add nothing.
  for (int kc0 = 0; kc0 < nk; kc0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
    const int kc = kc0 + u;
    chunk_barrier<(NS - 2) * L>();   // chunk kc has landed for every wave; chunk kc - 1 is read
    fetch(kc + NS - 1, slot((u + NS - 1) % NS));   // the slot chunk kc - 1 used; past the end: zeros
    const unsigned char* st = slot(u);
    const unsigned char* Bs = st + C::A_BYTES;
    if constexpr (MODE == 0) {
      // operands are read as whole vectors (a split read loses the LDS
      // object the compiler needs to keep its waits narrow)
      f32x4 bq[CB][4];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bq[cb][j] = *reinterpret_cast<const f32x4*>(
              Bs + ((wave + 4 * cb) * 16 + r16) * 256 + (((4 * j + q) ^ r16) << 4));
      f32x4 aq[NBI][4];
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          aq[bi][j] = *reinterpret_cast<const f32x4*>(st + (bi * 16 + r16) * 256 + (((4 * j + q) ^ r16) << 4));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int bi = 0; bi < NBI; ++bi)
              acc[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[bi][j][e], bq[cb][j][e], acc[cb][bi], 0, 0, 0);
      interleave_chunk<4 * CB + 4 * NBI, L, 16 * CB * NBI>();
    } else if constexpr (MODE == 2) {
      // step kk takes the 8-element k groups 4kk + q of both planes, the same
      // groups for h and R
      bx8 bh[CB][2], bl[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const unsigned char* row = Bs + ((wave + 4 * cb) * 16 + r16) * 256;
          bh[cb][kk] = *reinterpret_cast<const bx8*>(row + (((4 * kk + q) ^ r16) << 4));
          bl[cb][kk] = *reinterpret_cast<const bx8*>(row + (((8 + 4 * kk + q) ^ r16) << 4));
        }
      bx8 ah[NBI][2], al[NBI][2];
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const unsigned char* row = st + (bi * 16 + r16) * 256;
          ah[bi][kk] = *reinterpret_cast<const bx8*>(row + (((4 * kk + q) ^ r16) << 4));
          al[bi][kk] = *reinterpret_cast<const bx8*>(row + (((8 + 4 * kk + q) ^ r16) << 4));
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int bi = 0; bi < NBI; ++bi) {
            acc[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[bi][kk], bh[cb][kk], acc[cb][bi], 0, 0, 0);
            acc[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[bi][kk], bl[cb][kk], acc[cb][bi], 0, 0, 0);
            acc[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[bi][kk], bh[cb][kk], acc[cb][bi], 0, 0, 0);
          }
      interleave_chunk<4 * CB + 4 * NBI, L, 6 * CB * NBI>();
    } else {
      hx8 bv[CB][4];
      // resident R: this chunk's blocks (chunks past the end read the last
      // one, against zero h; a block past the tile reads block 0, dropped)
      const unsigned char* Rb = Bs;
      if constexpr (RR) Rb = rres + (kc < nk ? kc : nk - 1) * ncb * 4096;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int ci = RR && wave + 4 * cb >= ncb ? 0 : wave + 4 * cb;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          bv[cb][kk] = *reinterpret_cast<const hx8*>(Rb + (ci * 16 + r16) * 256 + (((4 * kk + q) ^ r16) << 4));
      }
      // step kk takes the 8-element k group 4kk + q of both halves of h and
      // of R (the same k for both operands)
      hx8 ah[NBI][4], al[NBI][4];
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const unsigned char* row = st + (bi * 16 + r16) * 512;
          ah[bi][kk] = *reinterpret_cast<const hx8*>(row + (((4 * kk + q) ^ row_swizzle<1>(r16)) << 4));
          al[bi][kk] = *reinterpret_cast<const hx8*>(row + (((16 + 4 * kk + q) ^ row_swizzle<1>(r16)) << 4));
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int bi = 0; bi < NBI; ++bi) {
            acc[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[bi][kk], bv[cb][kk], acc[cb][bi], 0, 0, 0);
            acc_lo[cb][bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[bi][kk], bv[cb][kk], acc_lo[cb][bi], 0, 0, 0);
          }
      interleave_chunk<4 * CB + 8 * NBI, L, 8 * CB * NBI>();
    }
    }
  }
  // the loads past the last chunk still write LDS: let them land before reuse
  chunk_barrier<0>();

  // accumulator layout of the 16x16 products: element i of lane l is row
  // 4*(l/16) + i, column l%16; column blocks past the tile are dropped
  float* rec = reinterpret_cast<float*>(st0);
  constexpr int LDR = kMaxNC + 1;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int ci = wave + 4 * cb;
    if (ci >= ncb) break;
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[cb][bi][i];
        if constexpr (MODE == 1) v += acc_lo[cb][bi][i];
        rec[(bi * 16 + 4 * q + i) * LDR + ci * 16 + r16] = v;
      }
  }
  __syncthreads();

  // gate arithmetic: the first element from its early gather; the others
  // from planes loaded into slot 1 (the host picks a column split whose
  // slot holds them), all loads in flight together
  constexpr bool DEF = MODE == 1;
  float* planes = reinterpret_cast<float*>(st1);
  if (n_el > kMThreads) epi_tile_issue<!PERS>(ctx, len_s, planes, n_el, ujs, b0, j0);
  epi_finish<RT, DEF>(ctx, first, rec, tid, ujs, b0, j0);
  if (n_el > kMThreads) {
    __syncthreads();   // waits for this wave's loads, then for the other waves
    epi_tile_finish<RT, DEF, !PERS>(ctx, first, len_s, rec, planes, n_el, ujs, b0, j0);
  }
}

template <int MODE, int BM, int CB>
__global__ __launch_bounds__(kMThreads) void step_dma_kernel(MfmaStepArgs m) {
  dma_step<MODE, BM, CB, false>(m, m.step, int(blockIdx.x), int(blockIdx.y), int(blockIdx.z));
}

// Every step in one launch (all tiles resident together, settled as in
// residency.h).  A workgroup keeps its tile for the whole layer, so the R rows it streams stay
// in its XCD's L2 from one step to the next instead of being fetched again
// after each kernel boundary.  Between phases, each workgroup publishes the
// count of phases it has finished in its own flag (a device-scope store after
// all its state stores have completed) and waits until every workgroup of its
// batch tile and direction, the ones whose h rows it reads, has published the
// count it needs.  Those are also the only readers of the h rows it writes,
// so a slot of h is never rewritten while a reader still needs it.  Every
// wait has a safety bound: a stuck run sets the status word and ends.
struct PersDmaArgs {
  MfmaStepArgs ph[2];   // per phase (a GRU with linear_before_reset = 0 has two)
  int P;                // phases per step
  int* flags;           // one per workgroup: phases finished; zeroed by the state setup
  int* status;          // [0] set to 1 if a wait ran past its bound; [1], [2] residency (residency.h)
  int fallback;         // > 0: take the fallback with this many workgroups (tests)
  int gx, gy, gz;       // the tile grid: unit tiles, batch tiles, directions
};

constexpr long kFlagSpinLimit = 1l << 22;

template <int MODE, int BM, int CB, bool RR>
__global__ __launch_bounds__(kMThreads) void step_dma_pers_kernel(PersDmaArgs p) {
  // launched plainly: every workgroup running (GO), or every workgroup exits
  // and the fallback kernel that follows runs the layer (residency.h)
  __shared__ int coop_dec;
  if (threadIdx.x == 0) {
    const int t = arrive_ticket(p.status + 1);
    coop_dec = arrive_decide(p.status + 1, int(gridDim.x * gridDim.y * gridDim.z), p.fallback, t);
  }
  __syncthreads();
  if (__builtin_expect(coop_dec != 1, 0)) return;
  const int steps = p.ph[0].a.steps, P = p.P;
  __shared__ int abort_s;
  const int gx = int(gridDim.x);
  const int row = int(blockIdx.y + gridDim.y * blockIdx.z);   // batch tile and direction
  const int me = int(blockIdx.x) + gx * row;
  const int* peers = p.flags + gx * row;
  if (threadIdx.x == 0) abort_s = 0;
  __syncthreads();
  for (int s = 0; s < steps; ++s)
    for (int ph = 0; ph < P; ++ph) {
      const int want = s * P + ph;
      if (want > 0) {
        if (threadIdx.x < 64) {
          for (int x = int(threadIdx.x); x < gx; x += 64) {
            long spin = 0;
            while (__hip_atomic_load(peers + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want)
              if (++spin > kFlagSpinLimit) {
                abort_s = 1;
                break;
              }
          }
        }
        __syncthreads();
        if (abort_s) {
          if (threadIdx.x == 0) __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
      }
      if (ph == 0) dma_step<MODE, BM, CB, true, RR>(p.ph[0], s, int(blockIdx.x), int(blockIdx.y), int(blockIdx.z));
      else dma_step<MODE, BM, CB, true, RR>(p.ph[1], s, int(blockIdx.x), int(blockIdx.y), int(blockIdx.z));
      // every state store of this workgroup has completed before the flag
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(p.flags + me, want + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Enqueued right after step_dma_pers_kernel, one workgroup per group of
// tiles (one batch tile of one direction): on GO it exits at once; on ABORT
// with count k, workgroups 0..k-1 take the groups g = w, w+k, ... and run
// every tile of a group in turn, step by step and phase by phase, through the
// same tile body as the fast path, so the results are bit-identical.  The
// tiles of one group depend only on one another, and one workgroup's own
// stores are complete (and so visible to its later loads) after each tile's
// final wait.  It waits on no other workgroup.
template <int MODE, int BM, int CB, bool RR>
__global__ __launch_bounds__(kMThreads) void step_dma_fallback_kernel(PersDmaArgs p) {
  __shared__ int dec;
  if (threadIdx.x == 0) dec = __hip_atomic_load(p.status + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (dec < 2) return;
  const int cnt = dec >> 8;
  const int steps = p.ph[0].a.steps, P = p.P;
  const int groups = p.gy * p.gz;
  if (int(blockIdx.x) >= cnt) return;
  for (int g = int(blockIdx.x); g < groups; g += cnt)
    for (int s = 0; s < steps; ++s)
      for (int ph = 0; ph < P; ++ph)
        for (int x = 0; x < p.gx; ++x) {
          if (ph == 0) dma_step<MODE, BM, CB, true, RR>(p.ph[0], s, x, g % p.gy, g / p.gy, true);
          else dma_step<MODE, BM, CB, true, RR>(p.ph[1], s, x, g % p.gy, g / p.gy, true);
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
          __syncthreads();
        }
}

template <int MODE, int BM, int CB>
static hipError_t launch_cfg(const MfmaStepArgs& m, hipStream_t s) {
  const StepArgs& a = m.a;
  const dim3 grid(unsigned((a.H + m.UJ - 1) / m.UJ), unsigned((a.B + BM - 1) / BM), unsigned(a.D));
  if (grid.y > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((step_dma_kernel<MODE, BM, CB>), grid, dim3(kMThreads), 0, s, m);
  return hipGetLastError();
}

// Column split: one 16-column block per wave when the tile has at most four,
// else two; two also when slot 1 of the one-block layout cannot hold the
// epilogue planes.
template <int MODE, int BM>
static hipError_t launch_bm(const MfmaStepArgs& m, hipStream_t s) {
  const int ncb = (m.Gp * m.UJ) >> 4;
  const int planes = (m.Gp + epi_state_planes(m.a.cell, m.a.lbr, m.phase)) * BM * m.UJ * 4;
  if (ncb <= 4 && planes <= DmaCfg<MODE, BM, 1>::STAGE) return launch_cfg<MODE, BM, 1>(m, s);
  if (planes > DmaCfg<MODE, BM, 2>::STAGE) return hipErrorInvalidValue;
  return launch_cfg<MODE, BM, 2>(m, s);
}

// The persistent form: one column split for both phases (the wider one).
template <int MODE, int BM, int CB, bool RR = false>
static hipError_t launch_pers_cfg(const PersDmaArgs& pa, hipStream_t s) {
  const StepArgs& a = pa.ph[0].a;
  const dim3 grid(unsigned((a.H + pa.ph[0].UJ - 1) / pa.ph[0].UJ), unsigned((a.B + BM - 1) / BM), unsigned(a.D));
  auto kern = step_dma_pers_kernel<MODE, BM, CB, RR>;
  PersDmaArgs arg = pa;
  arg.gx = int(grid.x);
  arg.gy = int(grid.y);
  arg.gz = int(grid.z);
  // A plain launch after a host check that every workgroup fits on the device
  // at once; the kernel settles residency itself (residency.h).
  // RNN_COOPERATIVE_LAUNCH=1 takes the cooperative launch instead.
  const char* coop_env = std::getenv("RNN_COOPERATIVE_LAUNCH");
  hipError_t e;
  if (!(coop_env && coop_env[0] == '1')) {
    int per_cu = 0, dev = 0, cus = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kMThreads,
                                                           0)) != hipSuccess)
      return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if (int64_t(per_cu) * cus < int64_t(grid.x) * grid.y * grid.z) return hipErrorCooperativeLaunchTooLarge;
    hipLaunchKernelGGL(kern, grid, dim3(kMThreads), 0, s, arg);
    e = hipGetLastError();
  } else {
    void* args[] = {&arg};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), grid, dim3(kMThreads), args, 0u, s);
  }
  if (e != hipSuccess) return e;
  // the fallback (it exits at once unless the decision was ABORT)
  hipLaunchKernelGGL((step_dma_fallback_kernel<MODE, BM, CB, RR>), dim3(grid.y * grid.z), dim3(kMThreads), 0, s, arg);
  return hipGetLastError();
}

// Resident R (f16 mode, one phase per step, 16 or 32 batch rows): the
// tile's R rows for every k chunk fit kRresBytes, and the epilogue planes fit
// a slot that holds h alone.  RNN_MFMA_RRES=0 turns it off.
template <int MODE, int BM>
static bool rres_fits(const PersDmaArgs& pa, int* cb) {
  if constexpr (MODE != 1 || BM > 32) {
    return false;
  } else {
    if (const char* e = std::getenv("RNN_MFMA_RRES"))
      if (std::atoi(e) == 0) return false;
    if (pa.P != 1) return false;
    const MfmaStepArgs& m = pa.ph[0];
    const int ncb = (m.Gp * m.UJ) >> 4;
    const int nk = (m.a.H + DmaGeo<1>::KC - 1) / DmaGeo<1>::KC;
    if (int64_t(nk) * ncb * 4096 > kRresBytes || ncb > 8) return false;
    const int planes = (m.Gp + epi_state_planes(m.a.cell, m.a.lbr, m.phase)) * BM * m.UJ * 4;
    *cb = ncb > 4 ? 2 : 1;
    return planes <= (*cb == 1 ? DmaCfg<1, BM, 1, true>::STAGE : DmaCfg<1, BM, 2, true>::STAGE);
  }
}

template <int MODE, int BM>
static hipError_t launch_pers_bm(const PersDmaArgs& pa, hipStream_t s) {
  int cb = 1;
  if constexpr (MODE == 1 && BM <= 32) {
    if (rres_fits<MODE, BM>(pa, &cb))
      return cb == 1 ? launch_pers_cfg<MODE, BM, 1, true>(pa, s) : launch_pers_cfg<MODE, BM, 2, true>(pa, s);
  }
  bool two = false;
  for (int ph = 0; ph < pa.P; ++ph) {
    const MfmaStepArgs& m = pa.ph[ph];
    const int ncb = (m.Gp * m.UJ) >> 4;
    const int planes = (m.Gp + epi_state_planes(m.a.cell, m.a.lbr, m.phase)) * BM * m.UJ * 4;
    if (ncb > 4 || planes > DmaCfg<MODE, BM, 1>::STAGE) two = true;
    if (planes > DmaCfg<MODE, BM, 2>::STAGE) return hipErrorNotSupported;
  }
  return two ? launch_pers_cfg<MODE, BM, 2>(pa, s) : launch_pers_cfg<MODE, BM, 1>(pa, s);
}

hipError_t launch_step_dma_persistent(const MfmaStepArgs* ph, int P, int bm, int mode, int* flags, int* status,
                                      hipStream_t s) {
  PersDmaArgs pa{};
  pa.ph[0] = ph[0];
  pa.ph[1] = P > 1 ? ph[1] : ph[0];
  pa.P = P;
  pa.flags = flags;
  pa.status = status;
  // the fallback reads the tensors as f16 in mode 1 and as f32 otherwise
  if ((mode == 1) != (ph[0].a.dtype == RNN_DTYPE_F16)) return hipErrorNotSupported;
  if (const char* e = std::getenv("RNN_PERSISTENT_FALLBACK")) pa.fallback = std::max(0, std::atoi(e));
  if (mode == 1)
    return bm == 64 ? launch_pers_bm<1, 64>(pa, s) : bm == 32 ? launch_pers_bm<1, 32>(pa, s)
                                                      : launch_pers_bm<1, 16>(pa, s);
  if (mode == 2)
    return bm == 64 ? launch_pers_bm<2, 64>(pa, s) : bm == 32 ? launch_pers_bm<2, 32>(pa, s)
                                                      : launch_pers_bm<2, 16>(pa, s);
  return bm == 64 ? launch_pers_bm<0, 64>(pa, s) : bm == 32 ? launch_pers_bm<0, 32>(pa, s)
                                                    : launch_pers_bm<0, 16>(pa, s);
}

bool step_dma_supported(const StepArgs& a, int mode) {
  if (mode == 2) {
    // bf16 planes in the state scratch (16-byte aligned rows when H is a
    // multiple of 8); every offset plus a plane, and the out-of-range marker
    // above them, fits 31 bits
    if (a.H % 8 != 0) return false;
    const uint64_t r = uint64_t(a.G) * a.H * a.H;
    if ((uint64_t(a.D) + 1) * r * 2 >= kOutOfRange) return false;
    if ((uint64_t(a.D) + 1) * a.B * a.H * 2 >= kOutOfRange) return false;
    return true;
  }
  const bool h16 = mode == 1;
  const int seg = h16 ? 8 : 4;   // elements of a 16-byte segment of R
  const uint64_t esize = h16 ? 2 : 4;
  if (a.H % seg != 0 || reinterpret_cast<uintptr_t>(a.R) % 16 != 0) return false;
  // every offset, and the out-of-range marker above them, fits 32 bits (mode
  // 1: h as two f16 planes, an offset plus a plane)
  if (uint64_t(a.G) * a.H * a.H * esize >= kOutOfRange) return false;
  if (uint64_t(a.B) * a.H * 4 >= kOutOfRange) return false;
  if (h16 && (uint64_t(a.D) + 1) * a.B * a.H * 2 >= kOutOfRange) return false;
  return true;
}

hipError_t launch_step_dma(const MfmaStepArgs& m, int bm, int mode, hipStream_t s) {
  if (mode == 1)
    return bm == 64 ? launch_bm<1, 64>(m, s) : bm == 32 ? launch_bm<1, 32>(m, s) : launch_bm<1, 16>(m, s);
  if (mode == 2)
    return bm == 64 ? launch_bm<2, 64>(m, s) : bm == 32 ? launch_bm<2, 32>(m, s) : launch_bm<2, 16>(m, s);
  return bm == 64 ? launch_bm<0, 64>(m, s) : bm == 32 ? launch_bm<0, 32>(m, s) : launch_bm<0, 16>(m, s);
}

}  // namespace rnnhip

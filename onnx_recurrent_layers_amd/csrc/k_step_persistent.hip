// k_step_persistent.hip -- stage 3 of a layer ("Recurrent layers" page, "How a
// layer runs", item 3) for small batches as ONE launch that walks every step,
// followed directly by the page's output rules ("Semantics").
//
// Why not a pass per step: the page avoids a grid-wide dependency because its
// APIs cannot guarantee co-resident workgroups ("Why a pass per step").  Here
// each workgroup keeps its share of R resident in LDS for the whole layer and
// the steps are ordered by per-value handshakes instead of kernel boundaries.
// The page's own one-workgroup-per-direction attempt lost because every step's
// R went through one compute unit; here R is spread over up to 256 compute
// units.
//
// Residency: HIP's cooperative launch guarantees co-resident workgroups, but
// on this runtime it costs about 18 us per launch (a sixteenth of a 80-step
// layer).  So the grid is launched plainly (after a host check that it fits
// the device) and the workgroups first agree whether all of them are running:
// each takes an arrival ticket; the first to see every ticket taken records
// GO, and one that waits past a short window records ABORT with the number of
// tickets taken by then (one compare-and-swap decides).  On GO the fast path
// below runs.  On ABORT (the device was partly held by other work) every
// workgroup exits, and the fallback kernel that the host enqueues right after
// this one (it exits at once on GO) runs the layer one direction per
// workgroup, taking the place of each workgroup of the direction in turn with
// the same arithmetic: slower, but bit-identical, and never a wait on a
// workgroup that may not be scheduled.  The fallback lives in its own kernel
// because inlined here it cost the fast path 2-3 % (C3: 877 against 859 us).
//
// Exchange: the hidden state of step s travels as 64-bit words
// (tag = step << 32 | f32 bits) stored and loaded with agent-scope relaxed
// atomics.  A reader spins until the word carries the tag it expects, so each
// value carries its own validity: no barrier, no fence, no counter.  Two slots
// (parity of the step) suffice: a workgroup can only overwrite a slot after
// every workgroup of its direction has published the next step, which each of
// them does only after it finished reading that slot.  The state setup that
// precedes this kernel on the stream writes step 0's words and invalidates the
// other slot, so words left by an earlier call are never taken for new ones.
//
// Determinism: each dot product is summed by fixed lanes in a fixed order and
// combined by a fixed xor butterfly; nothing depends on timing.
#include <algorithm>
#include <cstdlib>

#include "residency.h"

namespace rnnhip {

constexpr int kPThreads = 256;
constexpr int kMaxNB = 8;              // batch rows handled by this engine
constexpr long kSpinLimit = 1l << 22;  // safety bound on one wait (several seconds); never reached normally

struct PersArgs {
  StepArgs a;
  int U;            // units per workgroup
  int WPD;          // workgroups per direction
  int NR;           // R rows per workgroup = Gp * U
  int Gp;           // gate blocks computed (an LSTM with input_forget skips f)
  int gate_of[4];   // gate block index of each computed block
  int cand;         // GRU linear_before_reset = 0: index (in gate_of) of the candidate block, else -1
  int layout;
  const void* init_h;
  const void* init_c;
  void* Y;
  void* Y_h;
  void* Y_c;
  int* status;      // [0] set to 1 if a wait ran past the safety bound; [1] arrival tickets, [2] residency decision
  int fallback;     // > 0: take the fallback with this many workgroups (tests); 0: decide by arrival
};

__device__ __forceinline__ unsigned long long tagged(unsigned tag, float v) {
  return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
}

__device__ __forceinline__ unsigned long long load_word(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_word(unsigned long long* p, unsigned tag, float v) {
  __hip_atomic_store(p, tagged(tag, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy the words of step `tag` of every active batch row of one direction
// (src: [B][H]) into the workgroup's copy of h, waiting for each word to carry
// the tag.  That copy is hs[k][NB] in f32 for the vector-ALU products, or two
// f16 planes [NB][HS] (hi = f16(h), lo = f16(h - hi)) for the matrix-core
// products.  A thread keeps up to kChunk loads in flight and re-polls only
// stale words.
// issue() sends the first loads; complete() waits.  Memory operations issued
// between the two (output stores, the projection prefetch) are not waited for:
// the load counter retires in order, so only earlier operations delay a wait.
constexpr int kChunk = 24;
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left open
constexpr int kPollThreads = kPThreads - 64;  // waves 1..3 poll; wave 0 computes gates and does the other memory traffic

struct WordPoll {
  unsigned long long v[kChunk];
  bool want[kChunk];
};

// Where this thread's word slots of one chunk land: offset k*NB + b (f32
// copy) or b*HS + k (f16 planes) of the copy, and the batch row b (offset
// -1: no word).  Computed once; integer division by a runtime H costs tens of
// instructions, far too much to redo every step.
struct WordMap {
  int off[kChunk];
  int row[kChunk];
};

template <int NB, bool MF>
__device__ __forceinline__ void map_words(WordMap& m, int base, int H, int HS) {
  const int n = NB * H;
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    const int e = base + i * kPollThreads;
    const int b = e / H;
    m.off[i] = e < n ? (MF ? b * HS + (e - b * H) : (e - b * H) * NB + b) : -1;
    m.row[i] = b;
  }
}

// One value of h into the workgroup's copy: f32, or the hi/lo f16 pair (the
// lo plane starts `lo` halves after the hi plane).
template <bool MF>
__device__ __forceinline__ void store_h(void* hs, int off, int lo, float v) {
  if constexpr (MF) {
    half_t* h16 = static_cast<half_t*>(hs);
    const half_t hi = half_t(v);
    h16[off] = hi;
    h16[off + lo] = half_t(v - float(hi));
  } else {
    static_cast<float*>(hs)[off] = v;
  }
}

__device__ __forceinline__ void poll_issue(WordPoll& w, const WordMap& m, const unsigned long long* src, int base,
                                           unsigned amask) {
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    w.want[i] = m.off[i] >= 0 && ((amask >> m.row[i]) & 1u);
    if (w.want[i]) w.v[i] = load_word(src + base + i * kPollThreads);
  }
}

// Returns non-zero when the safety bound was hit.
template <bool MF>
__device__ __forceinline__ int poll_complete(WordPoll& w, const WordMap& m, const unsigned long long* src, int base,
                                             void* hs, int lo, unsigned tag) {
  int fail = 0;
  for (long round = 0;; ++round) {
    bool pending = false;
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (w.want[i] && static_cast<unsigned>(w.v[i] >> 32) != tag) pending = true;
    if (!pending) break;
    if (round > kSpinLimit) {
      fail = 1;
      break;
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (w.want[i] && static_cast<unsigned>(w.v[i] >> 32) != tag) w.v[i] = load_word(src + base + i * kPollThreads);
  }
#pragma unroll
  for (int i = 0; i < kChunk; ++i)
    if (w.want[i]) store_h<MF>(hs, m.off[i], lo, __uint_as_float(static_cast<unsigned>(w.v[i])));
  return fail;
}

// Staggered polling, for a few words per polling thread (the words
// ptid + i * kPollThreads): two batches of loads of the thread's words
// are kept in flight, the second issued about half a load round trip after
// the first; each batch is checked when it returns and reissued at once, so a
// word that lands is seen within about half a round trip instead of a whole
// one.  The loads are unconditional (a slot without a wanted word loads word
// 0 and ignores it), which keeps each batch's wait an exact count of the
// younger batch.  On C2 this took the layer from 269 to 199 us; a pause
// between the rounds of a single batch made it slower, so what counts is how
// soon a landed word is seen.  With many words per thread the doubled polling
// traffic swamps the memory system (22 words per thread: 3.6 times slower),
// and variants for more slots cost every kernel registers, so larger layers
// keep one batch at a time.
// s_sleep units of 64 cycles: about 0.9 us.  The optimum is narrow: biLSTM
// seq 80 batch 1 hidden 256 f32 took 194.5, 186.8, 180.1, 178.8 and 182.6 us
// of steps at 28, 30, 32, 34 and 36.
constexpr int kPollStagger = 34;
constexpr int kPollDelayMF = 24;   // before the first poll of the matrix-core form: about 0.64 us

// One batch row of up to 2 * kPollThreads units (the f32 copy of h is then
// h itself): polling thread t watches words t and t + kPollThreads.
__device__ __forceinline__ int stage_words_row(const unsigned long long* src, float* hs, unsigned tag, int H,
                                               unsigned amask, int ptid) {
  const int e0 = ptid, e1 = ptid + kPollThreads;
  const bool w0 = e0 < H && (amask & 1u), w1 = e1 < H && (amask & 1u);
  const unsigned long long* p0 = src + (w0 ? e0 : 0);
  const unsigned long long* p1 = src + (w1 ? e1 : 0);
  unsigned long long a0 = load_word(p0), a1 = load_word(p1);
  __builtin_amdgcn_s_sleep(kPollStagger);
  unsigned long long b0 = load_word(p0), b1 = load_word(p1);
  bool d0 = !w0, d1 = !w1;
  unsigned v0 = 0, v1 = 0;
  int fail = 0;
  for (long round = 0;; ++round) {
    if (!d0 && static_cast<unsigned>(a0 >> 32) == tag) {
      v0 = static_cast<unsigned>(a0);
      d0 = true;
    }
    if (!d1 && static_cast<unsigned>(a1 >> 32) == tag) {
      v1 = static_cast<unsigned>(a1);
      d1 = true;
    }
    if (d0 && d1) break;
    a0 = load_word(p0);
    a1 = load_word(p1);
    if (!d0 && static_cast<unsigned>(b0 >> 32) == tag) {
      v0 = static_cast<unsigned>(b0);
      d0 = true;
    }
    if (!d1 && static_cast<unsigned>(b1 >> 32) == tag) {
      v1 = static_cast<unsigned>(b1);
      d1 = true;
    }
    if (d0 && d1) break;
    b0 = load_word(p0);
    b1 = load_word(p1);
    if (round > kSpinLimit) {
      fail = 1;
      break;
    }
  }
  if (w0) hs[e0] = __uint_as_float(v0);
  if (w1) hs[e1] = __uint_as_float(v1);
  return fail;
}

// Whole stage, run by the polling waves only (ptid = thread index among
// them): staggered polling for one batch row of up to 384 units;
// otherwise the first chunk from the precomputed map `m0` and further chunks
// mapped on the fly, one batch of loads at a time.
template <int NB, bool MF>
__device__ __forceinline__ int stage_words(const unsigned long long* src, void* hs, unsigned tag, int H, int HS,
                                           unsigned amask, const WordMap& m0, int ptid) {
  // (compiled for one batch row only: any inlined variant moves the code and
  // registers of the other instances too, and cost C3 5 %)
  if constexpr (NB == 1 && !MF)
    if (H <= 2 * kPollThreads) return stage_words_row(src, static_cast<float*>(hs), tag, H, amask, ptid);
  int fail = 0;
  const int lo = NB * HS;
  WordPoll w;
  // with the matrix-core products, a first poll about 0.64 us late sees more
  // words landed (biGRU seq 128 batch 8 hidden 512 f16 at about 16 R rows per
  // workgroup: steps 976 us without the pause, 855 at 0.43 us, 849 at 0.64 us,
  // 890 at 0.85 us; with linear_before_reset = 1: 574, 495, 473, 477 us)
  if constexpr (MF) __builtin_amdgcn_s_sleep(kPollDelayMF);
  poll_issue(w, m0, src, ptid, amask);
  fail |= poll_complete<MF>(w, m0, src, ptid, hs, lo, tag);
  for (int base = ptid + kPollThreads * kChunk; base < NB * H; base += kPollThreads * kChunk) {
    WordMap m;
    map_words<NB, MF>(m, base, H, HS);
    poll_issue(w, m, src, base, amask);
    fail |= poll_complete<MF>(w, m, src, base, hs, lo, tag);
  }
  // Every load above has been consumed; this wait (free: nothing is
  // outstanding) tells the compiler so.  Without it the word registers of
  // words a thread did not want count as possibly still loading, and where
  // the polling waves' path joins wave 0's the compiler then waits for all
  // of wave 0's memory operations before reusing those registers, the
  // exchange store included.
  if constexpr (MF) __builtin_amdgcn_s_waitcnt(kWaitVm0);
  return fail;
}

// Workgroup barrier that orders LDS only: global loads (the projection
// prefetch) and stores (outputs, exchange words) stay in flight across it,
// where __syncthreads would wait for every outstanding memory operation.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the 8 lanes of an aligned lane group with DPP moves (xor 1, xor 2,
// then the half-row mirror); every lane of the group ends with the same total.
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

// Four consecutive elements of an LDS row, widened to f32.
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const half_t* p) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 v = *reinterpret_cast<const h4*>(p);
  return make_float4(float(v[0]), float(v[1]), float(v[2]), float(v[3]));
}

// rec[r][b] = sum_k Rl[r][k] * hs[k][b] for rows r in [r_lo, r_hi).  Groups
// of 8 lanes own a row (two rows at a time for more loads in flight); lane c
// of a group sums the chunks k = 4c..4c+3, 4c+32..4c+35, ... in increasing
// order, and sum8 combines the eight partial sums in a fixed tree.  Rows and
// hs are zero-padded to H4 (a multiple of 32), which adds exact zeros.
template <typename T, int NB>
__device__ __forceinline__ void products_ksplit(const T* Rl, int RS, const float* hs, float* rec, int NRNB, int r_lo,
                                                int r_hi, int H4) {
  // two groups per row: group rg takes row r_lo + rg % 16 and the 32-wide k
  // chunks of parity rg / 16; the two partial sums go to rec and rec + NRNB,
  // and the gate code adds them in that order
  const int c = threadIdx.x & 7, rg = threadIdx.x >> 3;
  const int r0 = r_lo + (rg & 15), half = rg >> 4;
  if (r0 >= r_hi) return;
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  const T* row = Rl + r0 * RS;
#pragma unroll 4
  for (int k0 = 4 * c + 32 * half; k0 < H4; k0 += 64) {
    const float4 a0 = ld4(row + k0);
    const float* hk = hs + k0 * NB;
    float hv[4 * NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const float4 v = ld4(hk + 4 * q);
      hv[4 * q] = v.x;
      hv[4 * q + 1] = v.y;
      hv[4 * q + 2] = v.z;
      hv[4 * q + 3] = v.w;
    }
    const float ra0[4] = {a0.x, a0.y, a0.z, a0.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[b] += ra0[i] * hv[i * NB + b];
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float v = sum8(acc[b]);
    if (c == b) rec[half * NRNB + r0 * NB + b] = v;
  }
}

template <typename T, int NB>
__device__ __forceinline__ void products(const T* Rl, int RS, const float* hs, float* rec, int r_lo, int r_hi,
                                         int H4) {
  const int c = threadIdx.x & 7, rg = threadIdx.x >> 3;
  constexpr int kGroups = kPThreads / 8;
  for (int r0 = r_lo + rg; r0 < r_hi; r0 += 2 * kGroups) {
    const int r1 = r0 + kGroups;
    const bool two = r1 < r_hi;
    float acc0[NB], acc1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = 0.f;
    const T* row0 = Rl + r0 * RS;
    const T* row1 = Rl + (two ? r1 : r0) * RS;
#pragma unroll 4
    for (int k0 = 4 * c; k0 < H4; k0 += 32) {
      const float4 a0 = ld4(row0 + k0);
      const float4 a1 = ld4(row1 + k0);
      const float* hk = hs + k0 * NB;
      float hv[4 * NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const float4 v = ld4(hk + 4 * q);
        hv[4 * q] = v.x;
        hv[4 * q + 1] = v.y;
        hv[4 * q + 2] = v.z;
        hv[4 * q + 3] = v.w;
      }
      const float ra0[4] = {a0.x, a0.y, a0.z, a0.w};
      const float ra1[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          acc0[b] += ra0[i] * hv[i * NB + b];
          acc1[b] += ra1[i] * hv[i * NB + b];
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v0 = sum8(acc0[b]);
      const float v1 = sum8(acc1[b]);
      if (c == b) {
        rec[r0 * NB + b] = v0;
        if (two) rec[r1 * NB + b] = v1;
      }
    }
  }
}

// Matrix-core variant of the products, for f16 R with the default
// activations (h then stays within f16 range) and four or more batch rows.
// R rows are the A operand, h the B operand as its hi and lo halves, each on
// v_mfma_f32_16x16x32_f16 with f32 accumulation.  Wave w takes the 32-wide k
// chunks w, w+4, ... of every 16-row block and writes its partial sums to
// red[w][r][b]; the gate code adds the four partials in wave order.
// Operand layout of the 16x16x32 product: lane l supplies row (A) or column
// (B) l%16 with the 8 consecutive k from 8*(l/16); element i of the
// accumulator of lane l is row 4*(l/16) + i, column l%16.  Columns at or past
// NB repeat real columns and are dropped; rows past r_hi are clamped to the
// last resident row and dropped.
typedef _Float16 hx8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NB, int NRB>
__device__ __forceinline__ void mfma_blocks(const half_t* Rl, int RS, const half_t* hhi, int HS, float* red, int r_lo,
                                            int r_hi, int NR, int H4) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  f32x4 acc[NRB], accl[NRB];
  const half_t* arow[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    acc[rb] = accl[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    arow[rb] = Rl + min(r_lo + 16 * rb + r16, NR - 1) * RS + 8 * q;
  }
  const half_t* bh = hhi + (r16 & (NB - 1)) * HS + 8 * q;
  const half_t* bl = bh + NB * HS;
  for (int kc = 32 * wave; kc < H4; kc += 128) {
    const hx8 vh = *reinterpret_cast<const hx8*>(bh + kc);
    const hx8 vl = *reinterpret_cast<const hx8*>(bl + kc);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const hx8 av = *reinterpret_cast<const hx8*>(arow[rb] + kc);
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, vh, acc[rb], 0, 0, 0);
      accl[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, vl, accl[rb], 0, 0, 0);
    }
  }
  if (r16 < NB) {
    float* out = red + wave * NR * NB + r16;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r_lo + 16 * rb + 4 * q + i;
        if (r < r_hi) out[r * NB] = acc[rb][i] + accl[rb][i];
      }
  }
}

template <int NB>
__device__ __forceinline__ void products_mfma(const half_t* Rl, int RS, const half_t* hhi, int HS, float* red,
                                              int r_lo, int r_hi, int NR, int H4) {
  switch ((r_hi - r_lo + 15) >> 4) {  // 16-row blocks: at most 4, since NB >= 4 allows 16 units, 64 rows
    case 1: mfma_blocks<NB, 1>(Rl, RS, hhi, HS, red, r_lo, r_hi, NR, H4); break;
    case 2: mfma_blocks<NB, 2>(Rl, RS, hhi, HS, red, r_lo, r_hi, NR, H4); break;
    case 3: mfma_blocks<NB, 3>(Rl, RS, hhi, HS, red, r_lo, r_hi, NR, H4); break;
    default: mfma_blocks<NB, 4>(Rl, RS, hhi, HS, red, r_lo, r_hi, NR, H4); break;
  }
}

// Which products a kernel instance uses (host and device agree on it).
template <typename T, int NB, bool DEF>
constexpr bool mfma_products() {
  return sizeof(T) == 2 && DEF && NB >= 4;
}

// The R rows of the units u0 .. u0+Uw-1 of direction d (every computed gate
// block) into LDS: row gi*U + uu holds R[d][gate_of[gi]*H + u0 + uu][0..H),
// zero past H up to H4 and for uu >= Uw.
template <typename T>
__device__ __forceinline__ void load_rows(const PersArgs& p, T* Rl, int RS, int d, int u0, int Uw, int H4) {
  const int H = p.a.H;
  const T* Rd = static_cast<const T*>(p.a.R) + int64_t(d) * p.a.G * H * H;
  for (int e = threadIdx.x; e < p.NR * H4; e += kPThreads) {
    const int r = e / H4, k = e - r * H4;
    const int gi = r / p.U, uu = r - gi * p.U;
    Rl[r * RS + k] = (uu < Uw && k < H) ? Rd[int64_t(p.gate_of[gi] * H + u0 + uu) * H + k] : T(0.f);
  }
}

// Gate arithmetic of one (unit, batch row) element in the step's first (or
// only) phase, in the order of cells.h: the fallback's copy of the fast path's
// inline gate code, the same expressions over the same helpers (the fast path
// keeps its inline form, which measured 1.5-2 % faster per step); a GPU test
// requires the two paths' outputs bit for bit equal.  rec_of(gi) is
// the recurrent sum of computed gate block gi; xv, wb, rb hold the
// projection and biases of gate block g at index g.  Returns the new h
// (LSTM, RNN, GRU with linear_before_reset = 1; c is updated in place); for
// a GRU with linear_before_reset = 0 (cand >= 0) it leaves z and r*h for the
// second phase and returns 0.
template <bool DEF, typename RecOf>
__device__ __forceinline__ float gates_first(const StepArgs& a, int cand, const Act* acts, const float* xv,
                                             RecOf rec_of, const float* wb, const float* rb, const float* peep,
                                             float& c, float hown, float& z, float& rh) {
  auto pre = [&](int gi, int g) { return pre_sum(xv[g], rec_of(gi), wb[g], rb[g]); };
  float hnew = 0.f;
  if (a.cell == RNN_CELL_LSTM) {
    float p4[4];
    p4[0] = pre(0, 0);
    p4[1] = pre(1, 1);
    if (a.input_forget) {
      p4[2] = 0.f;
      p4[3] = pre(2, 3);
    } else {
      p4[2] = pre(2, 2);
      p4[3] = pre(3, 3);
    }
    lstm_unit<DEF>(p4, a.P ? peep : nullptr, c, a.clip, a.input_forget, acts, &hnew, &c);
  } else if (a.cell == RNN_CELL_GRU) {
    z = gru_gate<DEF>(pre(0, 0), a.clip, acts);
    const float r = gru_gate<DEF>(pre(1, 1), a.clip, acts);
    if (cand < 0) {
      // linear_before_reset = 1: h~ = g(xw_h + r * (rec_h + Rb_h) + Wb_h)
      const float ph = (xv[2] + r * (rec_of(2) + rb[2])) + wb[2];
      hnew = gru_unit<DEF>(z, ph, hown, a.clip, acts);
    } else {
      rh = r * hown;
    }
  } else {
    hnew = rnn_unit<DEF>(pre(0, 0), a.clip, acts);
  }
  return hnew;
}

// Second phase of a GRU step with linear_before_reset = 0:
// h~ = g(((xw_h + R_h.(r*h)) + Wb_h) + Rb_h), h = (1 - z)*h~ + z*h.
template <bool DEF>
__device__ __forceinline__ float gates_cand(const StepArgs& a, const Act* acts, float xw_h, float rec_h, float wb_h,
                                            float rb_h, float z, float hown) {
  const float ph = pre_sum(xw_h, rec_h, wb_h, rb_h);
  return gru_unit<DEF>(z, ph, hown, a.clip, acts);
}

// The layer's direction d by one workgroup alone, for the fallback of the
// residency decision (not every workgroup of the grid is running, so none may
// wait on another).  The workgroup takes the place of each workgroup of the
// direction in turn, every step: it loads that workgroup's R rows into the
// same LDS layout, stages the same exchange words (already published, so the
// polls return at once), runs the same products and the same gate code, and
// publishes the same words.  Every result is therefore bit-identical to the
// fast path.  What the fast path keeps in registers across steps comes from
// memory instead: the cell state (cell_state, initialised by the state
// setup), the own h (the exchange word the unit published, or step 0's word
// from the setup) and a GRU's z between its two phases (zbuf).  Returns
// non-zero when a wait ran past its safety bound.
template <typename T, int NB, bool DEF>
__device__ __forceinline__ int fallback_blocks(const PersArgs& p, int d, unsigned char* smem) {
  const StepArgs& a = p.a;
  const int H = a.H, B = a.B, S = a.S, G = a.G;
  const int tid = threadIdx.x;
  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  const int GH = G * H;
  const int H4 = (H + 31) & ~31;
  const int RS = H4 + 8;
  constexpr bool MF = mfma_products<T, NB, DEF>();
  const int HS = H4 + 8;
  T* Rl = reinterpret_cast<T*>(smem);
  const size_t r_bytes = (size_t(p.NR) * RS * sizeof(T) + 15) & ~size_t(15);
  void* hs = smem + r_bytes;
  float* rec = reinterpret_cast<float*>(smem + r_bytes + (MF ? size_t(4) * NB * HS : size_t(4) * NB * H4));
  const int NRNB = p.NR * NB;
  const bool ksplit = !MF && p.NR <= 16 && H4 >= 64;
  auto recv = [&](int r, int b) {
    const int i = r * NB + b;
    if constexpr (MF) return ((rec[i] + rec[NRNB + i]) + rec[2 * NRNB + i]) + rec[3 * NRNB + i];
    else return ksplit ? rec[i] + rec[NRNB + i] : rec[i];
  };
  auto run_products = [&](int r_lo, int r_hi) {
    if constexpr (MF)
      products_mfma<NB>(reinterpret_cast<const half_t*>(Rl), RS, static_cast<const half_t*>(hs), HS, rec, r_lo, r_hi,
                        p.NR, H4);
    else if (ksplit)
      products_ksplit<T, NB>(Rl, RS, static_cast<const float*>(hs), rec, NRNB, r_lo, r_hi, H4);
    else
      products<T, NB>(Rl, RS, static_cast<const float*>(hs), rec, r_lo, r_hi, H4);
  };
  if constexpr (MF) {
    for (int e = tid; e < 2 * NB * HS; e += kPThreads) static_cast<half_t*>(hs)[e] = half_t(0.f);
  } else {
    for (int e = NB * H + tid; e < NB * H4; e += kPThreads) static_cast<float*>(hs)[e] = 0.f;
  }
  int maxL = 0;
  unsigned lens_left[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    lens_left[b] = b < B ? unsigned(row_length(a.lens, b, S, a.steps)) : 0u;
    maxL = max(maxL, int(lens_left[b]));
  }
  const int g_uu = tid / NB, g_b = tid % NB;
  int L = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (g_b == b) L = int(lens_left[b]);
  const Act* acts = a.act + d * a.slots;
  const T* bias = a.bias ? static_cast<const T*>(a.bias) + int64_t(d) * 2 * GH : nullptr;
  const bool rev = a.dir_reverse[d] != 0;
  const bool poller = tid >= kPThreads - kPollThreads;
  const int ptid = tid - (kPThreads - kPollThreads);
  WordMap wmap;
  if (poller) map_words<NB, MF>(wmap, ptid, H, HS);
  const int phases = p.cand >= 0 ? 2 : 1;
  const int nrows_main = p.cand >= 0 ? p.cand * p.U : p.NR;
  __shared__ int fb_fail;
  if (tid == 0) fb_fail = 0;
  for (int s = 0; s < maxL; ++s) {
    unsigned amask = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) amask |= (unsigned(s) < lens_left[b] ? 1u : 0u) << b;
    for (int ph = 0; ph < phases; ++ph)
      for (int vb = 0; vb < p.WPD; ++vb) {
        const int u0 = vb * p.U;
        const int Uw = min(p.U, H - u0);
        __syncthreads();   // the previous block is done with the LDS
        load_rows<T>(p, Rl, RS, d, u0, Uw, H4);
        if (poller) {
          const unsigned long long* src = (ph == 0 ? a.xch : a.xch2) + (s & 1) * DBH + dBH;
          if (stage_words<NB, MF>(src, hs, unsigned(s), H, HS, amask, wmap, ptid)) fb_fail = 1;
        }
        __syncthreads();
        if (fb_fail) return 1;
        run_products(ph == 0 ? 0 : nrows_main, ph == 0 ? nrows_main : p.NR);
        __syncthreads();
        const int j = u0 + g_uu;
        if (!(g_uu < Uw && g_b < B && s < L)) continue;
        const int64_t si = dBH + int64_t(g_b) * H + j;
        const int t = rev ? L - 1 - s : s;
        const float* xw = xw_dir(a, d) + (int64_t(s) * B + g_b) * GH + j;
        float xv[4] = {0.f, 0.f, 0.f, 0.f}, wb[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f};
        float peep[3] = {0.f, 0.f, 0.f};
        for (int g = 0; g < G; ++g) {
          if (!(a.input_forget && g == 2)) xv[g] = xw[g * H];
          if (bias) {
            wb[g] = ld(bias, g * H + j);
            rb[g] = ld(bias, GH + g * H + j);
          }
        }
        if (a.P) {
          const T* P = static_cast<const T*>(a.P) + int64_t(d) * 3 * H;
          peep[0] = ld(P, j);
          peep[1] = ld(P, H + j);
          peep[2] = ld(P, 2 * H + j);
        }
        const float hown = __uint_as_float(static_cast<unsigned>(load_word(a.xch + (s & 1) * DBH + si)));
        float hnew, c = 0.f;
        if (ph == 0) {
          float z = 0.f, rh = 0.f;
          if (a.cell == RNN_CELL_LSTM) c = a.cell_state[si];
          hnew = gates_first<DEF>(a, p.cand, acts, xv, [&](int gi) { return recv(gi * p.U + g_uu, g_b); }, wb, rb,
                                  peep, c, hown, z, rh);
          if (a.cell == RNN_CELL_LSTM) a.cell_state[si] = c;
          if (p.cand >= 0) {
            a.zbuf[si] = z;
            put_word(a.xch2 + (s & 1) * DBH + si, unsigned(s), rh);
            continue;
          }
        } else {
          hnew = gates_cand<DEF>(a, acts, xv[2], recv(p.cand * p.U + g_uu, g_b), wb[2], rb[2], a.zbuf[si], hown);
        }
        put_word(a.xch + ((s + 1) & 1) * DBH + si, unsigned(s + 1), hnew);
        if (p.Y)
          static_cast<T*>(p.Y)[y_index(p.layout, S, a.D, B, H, t, d, g_b, j)] = to_elem<T>(hnew);
        if (s == L - 1) {
          const int64_t oi = state_index(p.layout, a.D, B, H, d, g_b, j);
          if (p.Y_h) static_cast<T*>(p.Y_h)[oi] = to_elem<T>(hnew);
          if (p.Y_c) static_cast<T*>(p.Y_c)[oi] = to_elem<T>(c);
        }
      }
  }
  __syncthreads();
  return 0;
}

template <typename T, int NB, bool DEF>
__global__ __launch_bounds__(kPThreads) void persistent_kernel(PersArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const StepArgs& a = p.a;
  const int H = a.H, B = a.B, S = a.S, G = a.G;
  const int tid = threadIdx.x;
  const int d = blockIdx.x / p.WPD;
  const int u0 = (blockIdx.x % p.WPD) * p.U;
  const int Uw = min(p.U, H - u0);  // units of this workgroup (the last one may have fewer)
  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  const int GH = G * H;
  const int H4 = (H + 31) & ~31;     // rows and h padded with zeros to a multiple of 32
  const int RS = H4 + 8;             // LDS row stride: the rows a wave reads start in different banks
  constexpr bool MF = mfma_products<T, NB, DEF>();
  const int HS = H4 + 8;             // row stride of the f16 planes of h

  // arrival ticket now, the residency decision after the R rows are loaded
  int ticket = 0;
  if (tid == 0) ticket = arrive_ticket(p.status + 1);

  // LDS: R rows | copy of h | recurrent sums (f32 [NR][NB], or the four
  // partials [4][NR][NB] of the matrix-core products)
  T* Rl = reinterpret_cast<T*>(smem);
  const size_t r_bytes = (size_t(p.NR) * RS * sizeof(T) + 15) & ~size_t(15);
  void* hs = smem + r_bytes;
  float* rec = reinterpret_cast<float*>(smem + r_bytes + (MF ? size_t(4) * NB * HS : size_t(4) * NB * H4));
  const int NRNB = p.NR * NB;
  // the vector-ALU products with at most 16 rows leave half the lane groups
  // idle: then two groups share each row, one per parity of the 32-wide k
  // chunks (C2: 204 -> 187 us per layer, the recognizer shape 48/8/192/96:
  // 214 -> 193 us; needs two chunks at least)
  const bool ksplit = !MF && p.NR <= 16 && H4 >= 64;
  // recurrent sum of row r, batch row b
  auto recv = [&](int r, int b) {
    const int i = r * NB + b;
    if constexpr (MF) return ((rec[i] + rec[NRNB + i]) + rec[2 * NRNB + i]) + rec[3 * NRNB + i];
    else return ksplit ? rec[i] + rec[NRNB + i] : rec[i];
  };

  // R rows of this workgroup's units, resident for the whole layer
  const T* Rd = static_cast<const T*>(a.R) + int64_t(d) * GH * H;
  for (int e = tid; e < p.NR * H4; e += kPThreads) {
    const int r = e / H4, k = e - r * H4;
    const int gi = r / p.U, uu = r - gi * p.U;
    Rl[r * RS + k] = (uu < Uw && k < H) ? Rd[int64_t(p.gate_of[gi] * H + u0 + uu) * H + k] : T(0.f);
  }
  // padded tail of h stays zero (the f16 planes are cleared whole: columns of
  // absent batch rows feed only dropped outputs, but must not hold Inf or NaN)
  if constexpr (MF) {
    for (int e = tid; e < 2 * NB * HS; e += kPThreads) static_cast<half_t*>(hs)[e] = half_t(0.f);
  } else {
    for (int e = NB * H + tid; e < NB * H4; e += kPThreads) static_cast<float*>(hs)[e] = 0.f;
  }

  // every workgroup running, or the fallback kernel that follows this one
  __shared__ int coop_dec;
  if (tid == 0) coop_dec = arrive_decide(p.status + 1, int(gridDim.x), p.fallback, ticket);
  __syncthreads();
  if (__builtin_expect(coop_dec != 1, 0)) return;

  int maxL = 0;
  unsigned lens_left[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    lens_left[b] = b < B ? unsigned(row_length(a.lens, b, S, a.steps)) : 0u;
    maxL = max(maxL, int(lens_left[b]));
  }

  // gate thread: (unit u0 + uu, batch row b)
  const int g_uu = tid / NB, g_b = tid % NB;
  const bool gthread = g_uu < Uw && g_b < B;
  const int j = u0 + g_uu;
  int L = 0;
  float c = 0.f, hown = 0.f;
  const Act* acts = a.act + d * a.slots;
  const T* bias = a.bias ? static_cast<const T*>(a.bias) + int64_t(d) * 2 * GH : nullptr;
  float wb[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f}, peep[3] = {0.f, 0.f, 0.f};
  const int64_t sidx = p.layout == 0 ? (dBH + int64_t(g_b) * H + j) : ((int64_t(g_b) * a.D + d) * H + j);
  const bool rev = a.dir_reverse[d] != 0;
  if (gthread) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (g_b == b) L = int(lens_left[b]);
    hown = p.init_h ? ld(static_cast<const T*>(p.init_h), sidx) : 0.f;
    c = p.init_c ? ld(static_cast<const T*>(p.init_c), sidx) : 0.f;
    if (bias)
      for (int g = 0; g < G; ++g) {
        wb[g] = ld(bias, g * H + j);
        rb[g] = ld(bias, GH + g * H + j);
      }
    if (a.P) {
      const T* P = static_cast<const T*>(a.P) + int64_t(d) * 3 * H;
      peep[0] = ld(P, j);
      peep[1] = ld(P, H + j);
      peep[2] = ld(P, 2 * H + j);
    }
    // (the outputs no step writes, Y past the length and the final states of
    // an empty row, are written by the state setup)
  }
  __shared__ int abort_flag;
  if (tid == 0) abort_flag = 0;
  __syncthreads();

  int abort_run = 0;
  const int nrows_main = p.cand >= 0 ? p.cand * p.U : p.NR;  // rows of the first product
  // this thread's slice of the projection for one step.  Vector-ALU
  // products: prefetched one step ahead by wave 0 while the other waves poll
  // (HBM latency is about a step long).  Matrix-core products: loaded at the
  // end of the step before, after the exchange store, and first read by the
  // next gate arithmetic, after the next stage wait: by then every memory
  // operation of the wave issued before it has completed, so the wait for
  // these registers costs nothing.  There the loads are unconditional (a
  // lane with no element of its own, a gate block that does not exist or a
  // step past the row's length loads an element that exists and ignores
  // it): a load under a lane condition makes the compiler copy the
  // registers and wait for every memory operation issued after it, the
  // exchange stores included, whose completion takes a long trip.
  const int64_t xw_stride = int64_t(B) * GH;   // one step's slab
  const float* xw_me = xw_dir(a, d) + int64_t(min(g_b, B - 1)) * GH + min(j, H - 1);
  auto fetch_xw = [&](int step, float* out) {
    if constexpr (MF) {
      const int st = max(0, min(step, L - 1));
      const float* xw = xw_me + st * xw_stride;
#pragma unroll
      for (int g = 0; g < 4; ++g) out[g] = xw[min(g, G - 1) * H];
    } else if (gthread && step < L) {
      const float* xw = xw_me + step * xw_stride;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g < G && !(a.input_forget && g == 2)) out[g] = xw[g * H];
    }
  };
  const bool poller = tid >= kPThreads - kPollThreads;
  const int ptid = tid - (kPThreads - kPollThreads);
  WordMap wmap;
  if (poller) map_words<NB, MF>(wmap, ptid, H, HS);
  float xv[4] = {0.f, 0.f, 0.f, 0.f}, xnext[4] = {0.f, 0.f, 0.f, 0.f};
  fetch_xw(0, MF ? xv : xnext);
  // output of the previous step, stored after the next step's word loads are issued
  float y_prev = 0.f;
  int64_t yi_prev = -1;
  auto store_y = [&]() {
    if (yi_prev >= 0) static_cast<T*>(p.Y)[yi_prev] = to_elem<T>(y_prev);
    yi_prev = -1;
  };
  auto run_products = [&](int r_lo, int r_hi) {
    if constexpr (MF)
      products_mfma<NB>(reinterpret_cast<const half_t*>(Rl), RS, static_cast<const half_t*>(hs), HS, rec, r_lo, r_hi,
                        p.NR, H4);
    else if (ksplit)
      products_ksplit<T, NB>(Rl, RS, static_cast<const float*>(hs), rec, NRNB, r_lo, r_hi, H4);
    else
      products<T, NB>(Rl, RS, static_cast<const float*>(hs), rec, r_lo, r_hi, H4);
  };
  for (int s = 0; s < maxL; ++s) {
    unsigned amask = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) amask |= (unsigned(s) < lens_left[b] ? 1u : 0u) << b;

    const bool live = gthread && s < L;
    const int t = rev ? L - 1 - s : s;

    // 1. h of step s, every unit of this direction, active rows only (polling
    // waves); meanwhile wave 0 stores the previous output.
    int fail = 0;
    if (poller) {
      fail = stage_words<NB, MF>(a.xch + (s & 1) * DBH + dBH, hs, unsigned(s), H, HS, amask, wmap, ptid);
    } else {
      store_y();
      if constexpr (!MF) {
#pragma unroll
        for (int g = 0; g < 4; ++g) xv[g] = xnext[g];
        fetch_xw(s + 1, xnext);
      }
    }
    if (fail) abort_flag = 1;
    lds_barrier();
    if ((abort_run = abort_flag) != 0) break;

    // 2. recurrent products of this workgroup's rows
    run_products(0, nrows_main);
    lds_barrier();

    // 3. gate arithmetic
    float hnew = 0.f, z = 0.f;
    if (live) {
      auto pre = [&](int gi, int g) { return pre_sum(xv[g], recv(gi * p.U + g_uu, g_b), wb[g], rb[g]); };
      if (a.cell == RNN_CELL_LSTM) {
        float p4[4];
        p4[0] = pre(0, 0);
        p4[1] = pre(1, 1);
        if (a.input_forget) {
          p4[2] = 0.f;
          p4[3] = pre(2, 3);
        } else {
          p4[2] = pre(2, 2);
          p4[3] = pre(3, 3);
        }
        lstm_unit<DEF>(p4, a.P ? peep : nullptr, c, a.clip, a.input_forget, acts, &hnew, &c);
      } else if (a.cell == RNN_CELL_GRU) {
        z = gru_gate<DEF>(pre(0, 0), a.clip, acts);
        const float r = gru_gate<DEF>(pre(1, 1), a.clip, acts);
        if (p.cand < 0) {
          // linear_before_reset = 1: h~ = g(xw_h + r * (rec_h + Rb_h) + Wb_h)
          const float ph = (xv[2] + r * (recv(2 * p.U + g_uu, g_b) + rb[2])) + wb[2];
          hnew = gru_unit<DEF>(z, ph, hown, a.clip, acts);
        } else {
          put_word(a.xch2 + (s & 1) * DBH + dBH + int64_t(g_b) * H + j, unsigned(s), r * hown);
        }
      } else {
        hnew = rnn_unit<DEF>(pre(0, 0), a.clip, acts);
      }
    }

    if (p.cand >= 0) {
      // GRU, linear_before_reset = 0: the candidate needs r*h of every unit
      if (poller &&
          stage_words<NB, MF>(a.xch2 + (s & 1) * DBH + dBH, hs, unsigned(s), H, HS, amask, wmap, ptid))
        abort_flag = 1;
      lds_barrier();
      if ((abort_run = abort_flag) != 0) break;
      run_products(p.cand * p.U, p.NR);
      lds_barrier();
      if (live) {
        // h~ = g(((xw_h + R_h.(r*h)) + Wb_h) + Rb_h)
        const float ph = pre_sum(xv[2], recv(p.cand * p.U + g_uu, g_b), wb[2], rb[2]);
        hnew = gru_unit<DEF>(z, ph, hown, a.clip, acts);
      }
    }

    if (live) {
      put_word(a.xch + ((s + 1) & 1) * DBH + dBH + int64_t(g_b) * H + j, unsigned(s + 1), hnew);
      hown = hnew;
      if (p.Y) {
        yi_prev = p.layout == 0 ? ((int64_t(t) * a.D + d) * B + g_b) * H + j
                                : ((int64_t(g_b) * S + t) * a.D + d) * H + j;
        y_prev = hnew;
      }
      if (s == L - 1) {
        if (p.Y_h) static_cast<T*>(p.Y_h)[sidx] = to_elem<T>(hnew);
        if (p.Y_c) static_cast<T*>(p.Y_c)[sidx] = to_elem<T>(c);
      }
    }
    // 4. the projection of step s+1, after the exchange store has gone out
    if (MF && !poller) fetch_xw(s + 1, xv);
  }
  if (!abort_run && p.Y) store_y();
  if (abort_run && tid == 0) atomicExch(p.status, 1);
}

// Enqueued right after persistent_kernel, one workgroup per direction: on GO
// (the decision word is final once that kernel has ended) it exits at once;
// on ABORT with count k, workgroups 0..k-1 run the directions d = w, w+k, ...
// (fallback_blocks).  It waits on no other workgroup.
template <typename T, int NB, bool DEF>
__global__ __launch_bounds__(kPThreads) void persistent_fallback_kernel(PersArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int dec;
  if (threadIdx.x == 0) dec = __hip_atomic_load(p.status + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (dec < 2) return;
  const int cnt = dec >> 8;
  if (int(blockIdx.x) >= cnt) return;
  int fail = 0;
  for (int dd = blockIdx.x; dd < p.a.D && !fail; dd += cnt) fail = fallback_blocks<T, NB, DEF>(p, dd, smem);
  if (fail && threadIdx.x == 0) atomicExch(p.status, 1);
}

namespace {

int next_pow2_nb(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }

// LDS of one workgroup; `mf`: matrix-core products (f16 planes of h, four
// partial sums per output).
size_t lds_bytes(int NR, int H, int esize, int NB, bool mf) {
  const int H4 = (H + 31) & ~31;
  const size_t r = (size_t(NR) * (H4 + 8) * esize + 15) & ~size_t(15);
  if (mf) return r + size_t(4) * NB * (H4 + 8) + size_t(4) * NR * NB * 4;
  return r + size_t(NB) * H4 * 4 + size_t(2) * NR * NB * 4;
}

// All activation slots are the cell's ONNX defaults.
bool default_acts(const Problem& p) {
  const int c = p.desc.cell;
  for (int d = 0; d < p.D; ++d)
    for (int k = 0; k < p.slots; ++k) {
      const int kind = p.desc.activations[d * p.slots + k].kind;
      const int want = (c == RNN_CELL_RNN) ? RNN_ACT_TANH : (k == 0 ? RNN_ACT_SIGMOID : RNN_ACT_TANH);
      if (kind != want) return false;
    }
  return true;
}

constexpr size_t kLdsLimit = 160 * 1024;

}  // namespace

bool persistent_supported(const Problem& p, int* blocks, int* units, int* wg_per_dir) {
  if (p.B < 1 || p.B > kMaxNB || p.S < 1 || p.steps < 1) return false;
  if (p.H > 8192) return false;
  const int Gp = p.G - ((p.desc.cell == RNN_CELL_LSTM && p.desc.input_forget) ? 1 : 0);
  const int NB = next_pow2_nb(int(p.B));
  const int maxw = 256 / p.D;  // one workgroup per compute unit
  // R rows per workgroup: about 16.  The vector-ALU products: more
  // workgroups share each step's products (C2 3.54 us per step at 16 rows
  // against 3.73 at 32 and 3.76 at 64).  The matrix-core products work in
  // blocks of 16 rows, and a second block costs more than the extra
  // workgroups: biGRU seq 128, batch 8, hidden 512, f16 with
  // linear_before_reset = 1 took 494 us of steps at 12 or 15 rows (4 or 5
  // units) against 524 us at 18 or 24; with linear_before_reset = 0 (two
  // phases of 2U and U rows) 854 us either way.
  // RNN_PERSISTENT_UNITS overrides the choice for tuning.
  const bool mf_rows = p.esize == 2 && NB >= 4 && default_acts(p);   // the matrix-core products
  int U = std::max(1, 16 / Gp);
  if (const char* env = std::getenv("RNN_PERSISTENT_UNITS")) U = std::max(1, std::atoi(env));
  U = std::min(U, 64 / NB);
  int wpd = int((p.H + U - 1) / U);
  if (wpd > maxw) {
    wpd = maxw;
    U = int((p.H + wpd - 1) / wpd);
    wpd = int((p.H + U - 1) / U);
  }
  if (U * NB > 64) return false;  // one gate thread per (unit, batch row), all in wave 0
  if (lds_bytes(Gp * U, int(p.H), p.esize, NB, mf_rows) > kLdsLimit) return false;
  *blocks = wpd * p.D;
  *units = U;
  *wg_per_dir = wpd;
  return true;
}

template <typename T, int NB, bool DEF>
static hipError_t launch_nb(const PersArgs& pa, int blocks, size_t lds, hipStream_t s) {
  auto kern = persistent_kernel<T, NB, DEF>;
  auto fk = persistent_fallback_kernel<T, NB, DEF>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(fk), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(lds))) != hipSuccess)
    return e;
  PersArgs arg = pa;
  // A plain launch after checking on the host that every workgroup fits on
  // the device at once; the kernel itself settles whether they all run
  // together (residency.h).  RNN_COOPERATIVE_LAUNCH=1 takes the cooperative
  // launch instead (about 18 us more per launch here).
  const char* coop_env = std::getenv("RNN_COOPERATIVE_LAUNCH");
  if (!(coop_env && coop_env[0] == '1')) {
    int per_cu = 0, dev = 0, cus = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kPThreads,
                                                           lds)) != hipSuccess)
      return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if (per_cu * cus < blocks) return hipErrorCooperativeLaunchTooLarge;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kPThreads), lds, s, arg);
    e = hipGetLastError();
  } else {
    void* args[] = {&arg};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(blocks), dim3(kPThreads), args,
                                   unsigned(lds), s);
  }
  if (e != hipSuccess) return e;
  // the fallback (it exits at once unless the decision was ABORT)
  hipLaunchKernelGGL(fk, dim3(pa.a.D), dim3(kPThreads), lds, s, arg);
  return hipGetLastError();
}

hipError_t launch_step_persistent(const StepArgs& a, const Problem& p, const PersistentIO& io, hipStream_t s) {
  PersArgs pa{};
  pa.a = a;
  pa.U = p.pers_units;
  pa.WPD = p.pers_wg_per_dir;
  const bool skip_f = p.desc.cell == RNN_CELL_LSTM && p.desc.input_forget;
  pa.Gp = p.G - (skip_f ? 1 : 0);
  int gi = 0;
  for (int g = 0; g < p.G; ++g) {
    if (skip_f && g == 2) continue;
    pa.gate_of[gi++] = g;
  }
  pa.NR = pa.Gp * pa.U;
  pa.cand = (p.desc.cell == RNN_CELL_GRU && !p.desc.linear_before_reset) ? 2 : -1;
  pa.layout = p.desc.layout;
  pa.init_h = io.init_h;
  pa.init_c = io.init_c;
  pa.Y = io.Y;
  pa.Y_h = io.Y_h;
  pa.Y_c = io.Y_c;
  pa.status = io.status;
  if (const char* e = std::getenv("RNN_PERSISTENT_FALLBACK")) pa.fallback = std::max(0, std::atoi(e));
  const int NB = next_pow2_nb(a.B);
  const int blocks = p.pers_blocks;
  const bool def = default_acts(p);
  const size_t lds = lds_bytes(pa.NR, a.H, p.esize, NB, p.esize == 2 && NB >= 4 && def);
#define RNN_PERS_CASE(T, NB)                                                      \
  return def ? launch_nb<T, NB, true>(pa, blocks, lds, s) : launch_nb<T, NB, false>(pa, blocks, lds, s)
  if (a.dtype == RNN_DTYPE_F32) {
    switch (NB) {
      case 1: RNN_PERS_CASE(float, 1);
      case 2: RNN_PERS_CASE(float, 2);
      case 4: RNN_PERS_CASE(float, 4);
      default: RNN_PERS_CASE(float, 8);
    }
  }
  switch (NB) {
    case 1: RNN_PERS_CASE(half_t, 1);
    case 2: RNN_PERS_CASE(half_t, 2);
    case 4: RNN_PERS_CASE(half_t, 4);
    default: RNN_PERS_CASE(half_t, 8);
  }
#undef RNN_PERS_CASE
}

}  // namespace rnnhip

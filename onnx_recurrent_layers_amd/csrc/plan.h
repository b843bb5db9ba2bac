// plan.h -- the validated problem and the launch interface between the host
// library (api.cpp) and the kernel files.  Internal; not part of the C ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "rnn.h"

namespace rnnhip {

constexpr int kMaxActs = 6;

struct Act {
  int32_t kind;
  float alpha;
  float beta;
};

// Byte offsets of the regions inside the caller's state scratch (SIZE_MAX:
// the layout has no such region; the small-batch persistent engine keeps h in
// its exchange words and has no h slots nor r*h buffer).
struct StateLayout {
  size_t hbuf;     // f32 h, two slots of [D][B][H]: slot s & 1 holds h of step s (slot 0 = initial h)
  size_t cell;     // f32 c: [D][B][H] (LSTM), updated in place, final after the last step
  size_t zbuf;     // f32 GRU z for the two-phase step: [D][B][H]
  size_t rhbuf;    // f32 GRU r*h for the two-phase step: [D][B][H]
  size_t rsplit;   // bf16 R as two planes (hi, lo) of [D][G*H][H] (f32 layers on the bf16 matrix cores)
  size_t hsplit;   // h as 16-bit halves (f16 or bf16): two slots of two planes (hi, lo) of [D][B][H]
  size_t rhsplit;  // GRU r*h likewise: two planes of [D][B][H]
  size_t xch;      // u64 tagged exchange words of the persistent engine: [2][D][B][H]
  size_t xch2;     // u64 tagged r*h words (GRU, linear_before_reset = 0): [2][D][B][H]
  size_t status;   // int[3]: persistent engine status (1: a wait hit its safety bound), arrival tickets, residency decision
  size_t flags;    // int per workgroup of the persistent matrix-core step: phases finished
  size_t total;
};

struct Problem {
  rnn_problem_desc desc;
  int G = 1;        // gates
  int D = 1;        // directions
  int slots = 1;    // activation slots per direction
  int64_t S = 0, B = 0, I = 0, H = 0;
  int64_t steps = 0;  // steps run: max_length or S
  int esize = 4;      // element size of float tensors
  size_t xw_bytes = 0;
  // the projection scratch: xw_slots (1 or 2) slots of xw_tc steps each; two
  // slots form a ring through which the projection runs chunk by chunk,
  // ahead of the steps
  int64_t xw_tc = 0;
  int xw_slots = 1;
  StateLayout st{};
  int engine = RNN_ENGINE_LAUNCH;
  bool def_acts = false;  // every activation slot holds the cell's ONNX default
  // persistent engine geometry
  int pers_blocks = 0;       // workgroups of the persistent launch
  int pers_units = 0;        // units per workgroup
  int pers_wg_per_dir = 0;
  // the persistent engine in its matrix-core form (batches above eight)
  bool pers_mfma = false;
  // tile of the matrix-core step (batch rows, units), fixed when the problem
  // is created (batches above eight)
  int mfma_bm = 16, mfma_uj = 16;
  // f32 tensors: the projection on the bf16 matrix cores (three split
  // products) instead of the f32 matrix cores
  bool f32_split_proj = false;
  // f32 tensors: the per-step matrix-core product on the bf16 matrix cores
  bool f32_split_step = false;
  // the step that produces h also writes it as two 16-bit planes for the
  // matrix-core step's operand: 1 f16 halves (f16 layers with the default
  // activations), 2 bf16 halves (f32 layers on the bf16 matrix cores), 0 none
  int h_split = 0;
};

// Arguments shared by the step kernels.
struct StepArgs {
  int cell, G, D, H, B, S;
  int steps;
  int dir_reverse[2];      // 1 when direction d runs backwards in time
  int dtype;               // RNN_DTYPE_*
  const void* R;           // [D][G*H][H]
  const void* bias;        // [D][2*G*H] or null
  const void* P;           // [D][3*H] or null
  const int32_t* lens;     // [B] or null
  // the projection, step-major: slab (d, s) [B][G*H] holds, in row b, the
  // projection of the X row that step s of batch row b of direction d reads
  // (time s, or len_b - 1 - s for a reverse direction).  Chunked: a ring of
  // two slots of xw_tc steps each, [slot][D][xw_tc][B][G*H], step s in slot
  // (s / xw_tc) & 1; unchunked: xw_tc = S, one slot.
  const float* xw;
  int xw_tc;
  float* hbuf;             // [2][D][B][H]: slot s & 1 holds h of step s
  void* Y;                 // [S][D][B][H] (layout 0) or [B][S][D][H] (layout 1), or null
  void* Y_h;               // [D][B][H] (layout 0) or [B][D][H] (layout 1), or null
  void* Y_c;               // the same (LSTM), or null
  int layout;
  float* cell_state;       // [D][B][H]
  float* zbuf;             // [D][B][H]
  float* rhbuf;            // [D][B][H]
  // 16-bit halves of R, h and r*h for the matrix-core step's operands (null
  // when not used): bit patterns, hi and lo planes of each tensor.  R only for
  // f32 layers on the bf16 matrix cores.
  unsigned short* rsplit;  // [2][D][G*H][H], bf16
  unsigned short* hsplit;  // [2 slots][2][D][B][H]: slot s & 1 holds h of step s
  unsigned short* rhsplit; // [2][D][B][H]
  int split_kind;          // of hsplit and rhsplit: 1 f16 halves, 2 bf16 halves
  unsigned long long* xch; // [2][D][B][H]
  unsigned long long* xch2;// [2][D][B][H]
  float clip;              // > 0: clamp
  int input_forget;
  int lbr;
  int slots;
  Act act[kMaxActs];
};

struct ProjArgs {
  const void* X;      // layout-mapped rows
  const void* W;      // [D][N][K]
  float* xw;          // output row m of direction d at xw + d * out_dstride + m * N
  int64_t out_dstride;
  // output row m = (s - s0) * B + b is the projection of the X row that step
  // s of batch row b reads: time s forward, len_b - 1 - s in a reverse
  // direction (rev[d]); rows of a step past the row's length take time s
  const int32_t* lens;
  int rev[2];
  int64_t s0, steps;
  int64_t M, N, K;
  int64_t S, B;
  int layout;
  int D;
  int skip_block;     // gate block of H columns not needed (input_forget: f), or -1
  int64_t H;
  int f32_split;      // f32 tensors: products on the bf16 matrix cores as three split products
  // X rows in two pieces (the Y [S,2,B,K/2] of a bidirectional layout-0 layer
  // read as X): elements k >= xkh of a row lie xjump elements further on.
  // Otherwise xkh = K and xjump = 0.
  int64_t xkh, xjump;
};

struct SetupArgs {
  int D, B, H;
  int layout;
  int dtype;
  const void* init_h;  // or null
  const void* init_c;  // or null
  float* hbuf;         // slot 0 of the per-step engines' h, or null
  unsigned short* hsplit;  // slot 0 of h as 16-bit hi and lo planes, or null
  int split_kind;          // 1 f16 halves, 2 bf16 halves
  float* cell_state;   // or null
  unsigned long long* xch;   // tagged h words [2][D][B][H], or null (per-step engine)
  unsigned long long* xch2;  // tagged r*h words [2][D][B][H], or null
  int* status;               // persistent engine status word and the two residency words after it, or null
  int* flags;                // workgroup flags of the persistent matrix-core step, zeroed here, or null
  int nflags;
  // outputs no step writes: Y past each row's length, the final states of
  // rows of length 0, and every final state when Seq = 0
  void* Y;
  void* Y_h;
  void* Y_c;
  const int32_t* lens;
  int S, steps;
};

// What the persistent engine reads and writes besides StepArgs.
struct PersistentIO {
  const void* init_h;
  const void* init_c;
  void* Y;
  void* Y_h;
  void* Y_c;
  int* status;
};

// rnn_encode with the scratch pointers already chosen (api.cpp), and the
// thread's error message set from another file.
int encode_layer(const rnn_problem* problem, const rnn_operands* ops, void* xw_scratch, void* state_scratch,
                 void* stream);
int set_error(int code, int cell, const char* msg);

hipError_t launch_projection(const ProjArgs& a, const SetupArgs& sa, int dtype, hipStream_t s);  // also runs the state setup
hipError_t launch_setup(const SetupArgs& a, hipStream_t s);
hipError_t launch_split_r(const void* R, unsigned short* rsplit, int64_t n, hipStream_t s);
hipError_t launch_step_generic(const StepArgs& a, int step, hipStream_t s);
int step_generic_launches_per_step(const StepArgs& a);
hipError_t launch_step_mfma(const StepArgs& a, const Problem& p, int step, hipStream_t s);
bool mfma_step_supported(const Problem& p);
// Tile of the matrix-core step for a problem (RNN_MFMA_TILE may force one).
void mfma_tile(int B, int H, int D, int Gp, int* bm, int* uj);
// Persistent form of the matrix-core step: one launch for every
// step, at most kPersistentMfmaTiles workgroups (one per compute unit).
constexpr int kPersistentMfmaTiles = 256;
bool mfma_persistent_supported(const Problem& p, int* tiles);
hipError_t launch_step_mfma_persistent(const StepArgs& a, const Problem& p, int* flags, int* status, hipStream_t s);
// Whether the direct-to-LDS matrix-core step takes this shape in a mode (0:
// f32 on the f32 matrix cores, 1: f16 with split h, 2: f32 on the bf16 matrix
// cores).
bool step_dma_supported(const StepArgs& a, int mode);
hipError_t launch_step_persistent(const StepArgs& a, const Problem& p, const PersistentIO& io, hipStream_t s);
bool persistent_supported(const Problem& p, int* blocks, int* units, int* wg_per_dir);

}  // namespace rnnhip

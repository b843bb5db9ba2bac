/*
 * rnn.h -- C ABI of the MI355X (gfx950) library for ONNX recurrent layers:
 * RNN, GRU and LSTM; forward, reverse and bidirectional; layouts 0 and 1;
 * sequence_lens; initial states; peepholes; clip; input_forget;
 * linear_before_reset; the eleven ONNX activations.
 *
 * The operations are those of the "Recurrent layers" page of the OneGpu docs
 * (recursiveai.org/onegpu/docs/recurrent): the problem description and its
 * checks (introduction and "Scratch"), the four stages of a layer ("How a
 * layer runs"), the arithmetic order ("Arithmetic and determinism") and the
 * edge rules ("Semantics"), with tensor shapes from the ONNX operator
 * definitions the page defers to.
 *
 * Conventions
 *   - Every float tensor of one layer has the same element type, f32 or f16
 *     (IEEE binary16).  Arithmetic and the recurrent state are f32; f16
 *     outputs are rounded to nearest even once.
 *   - Tensors are device pointers plus an element offset (rnn_tensor).  The
 *     address ptr + elem_offset * element_size must be aligned to the element
 *     size; no other alignment is required.  Outputs whose pointer is NULL are
 *     not written; nothing outside an output's extent is ever written.
 *   - W, R, B and P are read exactly as ONNX stores them (gate blocks i,o,f,c
 *     for an LSTM, z,r,h for a GRU); nothing is repacked.
 *   - All memory is owned by the caller.  rnn_encode allocates nothing and
 *     synchronises nothing: it enqueues kernels on the caller's HIP stream and
 *     returns.  Each call uses its scratch buffers exclusively until the
 *     stream has finished the call's work.
 *   - Errors: a non-zero rnn_status; rnn_last_error() then returns a message
 *     naming the cell (LSTM, GRU or RNN) and the offending argument.  When any
 *     check fails, nothing has been enqueued.
 *   - Environment switches, for tests and tuning (unset is the default;
 *     each is read when a layer is planned or enqueued, and each keeps the
 *     results within the layer's tolerance):
 *       RNN_COOPERATIVE_LAUNCH=1    persistent kernels through the cooperative
 *                                   launch API (bit-identical results)
 *       RNN_PERSISTENT_UNITS=u      hidden units per workgroup of the
 *                                   persistent engine
 *       RNN_PERSISTENT_FALLBACK=k   force the persistent kernels' fallback: k
 *                                   workgroups take the place of the whole
 *                                   grid in turn (bit-identical results)
 *       RNN_MFMA_RRES=0             stream R every step in the persistent
 *                                   matrix-core step (bit-identical results)
 *       RNN_MFMA_TILE=BMxUJ         force a matrix-core step tile
 *       RNN_F32_SPLIT=0|1           f32 products on the f32 matrix cores (0)
 *                                   or as three bf16 products (1, any size)
 *       RNN_SMALL_PROJECTION=0|1    small-layer projection off or on
 *       RNN_PROJ_LDS_MIN_TILES=n    tile count from which the 256x256
 *                                   projection is taken
 *       RNN_CHUNK_OVERLAP=1         a chunked projection runs on a second
 *                                   stream (default priority), each chunk
 *                                   overlapping the steps of the chunk before
 *                                   (off by default: measured no faster)
 */
#ifndef ONNX_RNN_MI355X_H
#define ONNX_RNN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status of every call.  The page's exceptions map onto them: a shape
 * exception naming the cell and the argument ("Scratch": checked in safe
 * arithmetic before anything is recorded) is RNN_ERR_SHAPE or RNN_ERR_ARG,
 * an option on the wrong cell ("Semantics": anything else throws) is
 * RNN_ERR_ARG, and the unsupported-layer exception ("Scratch": larger layers
 * throw) is RNN_ERR_UNSUPPORTED. */
typedef enum {
  RNN_OK = 0,
  RNN_ERR_ARG = 1,         /* a NULL or malformed argument, an option on the wrong cell */
  RNN_ERR_SHAPE = 2,       /* a negative or overflowing size, a bad max_length */
  RNN_ERR_UNSUPPORTED = 3, /* a valid layer this build cannot run (limits below) */
  RNN_ERR_HIP = 4          /* the HIP runtime refused a launch */
} rnn_status;

typedef enum { RNN_CELL_RNN = 0, RNN_CELL_GRU = 1, RNN_CELL_LSTM = 2 } rnn_cell;
typedef enum { RNN_DTYPE_F32 = 0, RNN_DTYPE_F16 = 1 } rnn_dtype;
typedef enum { RNN_DIR_FORWARD = 0, RNN_DIR_REVERSE = 1, RNN_DIR_BIDIRECTIONAL = 2 } rnn_direction;

/* The eleven ONNX activations (operator definitions):
 *   Relu max(0,x); Tanh; Sigmoid 1/(1+e^-x); Affine a*x+b; LeakyRelu x>=0 ? x : a*x;
 *   ThresholdedRelu x>a ? x : 0; ScaledTanh a*tanh(b*x); HardSigmoid min(max(a*x+b,0),1);
 *   Elu x>=0 ? x : a*(e^x-1); Softsign x/(1+|x|); Softplus log(1+e^x). */
typedef enum {
  RNN_ACT_RELU = 0, RNN_ACT_TANH = 1, RNN_ACT_SIGMOID = 2, RNN_ACT_AFFINE = 3,
  RNN_ACT_LEAKY_RELU = 4, RNN_ACT_THRESHOLDED_RELU = 5, RNN_ACT_SCALED_TANH = 6,
  RNN_ACT_HARD_SIGMOID = 7, RNN_ACT_ELU = 8, RNN_ACT_SOFTSIGN = 9, RNN_ACT_SOFTPLUS = 10
} rnn_activation_kind;

/* One activation with its alpha and beta already resolved by the caller (the
 * page's GpuRecurrentActivation): defaults of ONNX are not applied here. */
typedef struct {
  int32_t kind;  /* rnn_activation_kind */
  float alpha;
  float beta;
} rnn_activation;

/* Step-engine choice.  AUTO picks per problem from measured speed. */
typedef enum {
  RNN_ENGINE_AUTO = 0,
  RNN_ENGINE_LAUNCH = 1,      /* one kernel launch per step (two for GRU linear_before_reset=0) */
  RNN_ENGINE_PERSISTENT = 2   /* one launch for all steps (batches up to eight; the matrix-core step above eight) */
} rnn_engine;

/* Layer description (the page's RecurrentProblem plus ONNX attributes). */
typedef struct {
  int32_t cell;                /* rnn_cell */
  int32_t dtype;               /* rnn_dtype: the type of every float tensor */
  int32_t direction;           /* rnn_direction */
  int32_t layout;              /* 0: X [S,B,I], states [D,B,H], Y [S,D,B,H]; 1: X [B,S,I], states [B,D,H], Y [B,S,D,H] */
  int64_t seq;                 /* S >= 0 */
  int64_t batch;               /* B >= 0 */
  int64_t input;               /* I >= 0 */
  int64_t hidden;              /* H >= 1 */
  float clip;                  /* clamp every gate pre-activation to [-clip, clip] when clip > 0; NaN passes */
  int32_t input_forget;        /* LSTM only: 0 or 1 (forget gate f = 1 - i) */
  int32_t linear_before_reset; /* GRU only: 0 or 1 */
  int32_t num_activations;     /* slots x directions: LSTM 3 (f,g,h), GRU 2 (f,g), RNN 1 (f) per direction */
  rnn_activation activations[6]; /* forward slots, then reverse slots */
  int64_t max_length;          /* 0: S.  Otherwise a host-side bound on the sequence lengths (<= S):
                                  only that many steps run, and longer rows are cut to it */
  int32_t engine;              /* rnn_engine hint */
  int32_t x_bidirectional_y;   /* 0, or 1: X is the Y output of a bidirectional layer of the same layout and
                                  sequence length, read in place as this layer's input (stacked layers; the
                                  recognizer of the onegpu docs' CRNN stacks two bidirectional LSTMs).  input
                                  must then be even, I = 2 H'.  Layout 0: Y [S, 2, B, H'] is read as X
                                  [S, B, 2H'], element (t, b, k) = Y[t, k / H', b, k % H'] (two pieces of
                                  H' per row, B*H' elements apart, gathered by the projection; no transpose).
                                  Layout 1: Y [B, S, 2, H'] already is X [B, S, 2H'] in memory, so 1 changes
                                  nothing. */
  int64_t xw_chunk_steps;      /* the input projection in chunks of this many steps, through a ring of two
                                  chunks in the projection scratch (the page's "Scratch": XwLength grows with
                                  the layer), each chunk's projection enqueued right before its steps (or
                                  ahead of them on a second stream, RNN_CHUNK_OVERLAP): 0 lets the library choose (one
                                  chunk, unless the whole projection exceeds 512 MiB); n > 0 asks for chunks
                                  of n steps.  Only the per-step engine (RNN_ENGINE_LAUNCH) runs in chunks;
                                  the persistent engines read every step's projection in their one launch
                                  and always take one chunk.  rnn_scratch_size and rnn_problem_plan report
                                  the outcome.  >= 0. */
} rnn_problem_desc;

/* Opaque, immutable after creation; safe to share between threads. */
typedef struct rnn_problem rnn_problem;

/* A device buffer plus an element offset (the page's GpuTensorRef). */
typedef struct {
  void* ptr;            /* device pointer, or NULL for an absent tensor */
  int64_t elem_offset;  /* >= 0, in elements of the tensor's type */
} rnn_tensor;

/* Operands in ONNX shapes (D = 2 for bidirectional, else 1; G = 4 LSTM, 3 GRU, 1 RNN):
 *   X [S,B,I] (layout 1: [B,S,I])      required
 *   W [D, G*H, I]                      required
 *   R [D, G*H, H]                      required
 *   B [D, 2*G*H] = Wb then Rb          optional (zeros)
 *   sequence_lens [B] int32            optional (all S); values above S act as S, below 0 as 0
 *   initial_h [D,B,H] (layout 1: [B,D,H])  optional (zeros)
 *   initial_c  same shape, LSTM only   optional (zeros)
 *   P [D, 3*H] (i, o, f), LSTM only    optional (no peepholes)
 *   Y [S,D,B,H] (layout 1: [B,S,D,H])  optional output
 *   Y_h [D,B,H] (layout 1: [B,D,H])    optional output
 *   Y_c  same shape, LSTM only         optional output */
typedef struct {
  rnn_tensor X, W, R, B, sequence_lens, initial_h, initial_c, P, Y, Y_h, Y_c;
} rnn_operands;

/* Validate a description (64-bit checked arithmetic) and build the immutable
 * problem.  On success *out owns the problem; free it with
 * rnn_problem_destroy.  On error *out is set to NULL.
 *
 * Limits (RNN_ERR_UNSUPPORTED): hidden above 2^24; batch or seq above 2^30;
 * engine = RNN_ENGINE_PERSISTENT on a shape that neither persistent form
 * takes (the vector form needs a batch of at most 8 whose units fit the
 * workgroups' LDS; the matrix-core form a batch above 8, rows of whole
 * 16-byte segments and tiles that fit the chip at once).  RNN_ENGINE_AUTO never
 * fails for that reason; rnn_problem_plan shows the engine it chose.  A
 * tensor, Y or the projection scratch above 2^52 bytes is RNN_ERR_SHAPE. */
int rnn_problem_create(const rnn_problem_desc* desc, rnn_problem** out);

/* Free a problem (NULL is ignored). */
void rnn_problem_destroy(rnn_problem* problem);

/* Scratch the caller must supply to rnn_encode (the page's "Scratch"):
 *   *xw_bytes    = 4 * slots * D * C * B * G * H: the f32 input projection
 *                  in `slots` slots of C steps each (one slot of C = the steps
 *                  run, max_length or S, unless the projection runs in chunks:
 *                  then two slots of C = the chunk's steps), laid out
 *                  step-major [slot][D][C][B][G*H]: row b of step s of
 *                  direction d holds X[t,b,:] . W[d]^T for the time t that
 *                  step reads (s forward, len_b - 1 - s backward);
 *   *state_bytes = the f32 hidden state (two slots of [D][B][H]), the f32
 *                  cell state, the GRU two-pass buffers, and for the
 *                  persistent engine its exchange words and status words.
 * Either may be 0 (then the matching pointer may be NULL).  Both buffers must
 * be 256-byte aligned; they may be two regions of one arena. */
int rnn_scratch_size(const rnn_problem* problem, size_t* xw_bytes, size_t* state_bytes);

/* Enqueue one layer on `stream` (a hipStream_t; NULL is the default stream):
 * the four stages of "How a layer runs" on the "Recurrent layers" page (the
 * page's Encode into a caller's command encoder), with the edge rules of its
 * "Semantics" list and the arithmetic order of "Arithmetic and determinism".
 * Stages: the input projection (carrying the state setup), then the
 * recurrent steps, which write whichever of Y, Y_h, Y_c is requested as they
 * go (the setup writes the outputs no step reaches).  Batch = 0 enqueues
 * nothing; Seq = 0 writes only Y_h / Y_c (initial states or zeros).  All
 * checks run before the first launch ("Scratch": sizes, offsets and shapes
 * are checked before anything is recorded); when one fails nothing is
 * enqueued.  Arguments: `operands` as described above (device pointers with
 * element offsets, owned by the caller); `xw_scratch` and `state_scratch` the
 * caller's device buffers of at least the sizes rnn_scratch_size reports,
 * 256-byte aligned (the page's xwScratch and stateScratch).
 * RNN_ERR_HIP (the runtime refused a launch) may come after earlier stages
 * were enqueued: the outputs are then undefined, and the scratch is in use
 * until the stream has finished that work.  sequence_lens is read on the
 * device and not validated there (rnn_validate_lengths checks it on the
 * host). */
int rnn_encode(const rnn_problem* problem, const rnn_operands* operands,
               void* xw_scratch, void* state_scratch, void* stream);

/* rnn_encode with timing marks: the same launches, plus hipEventRecord of
 * events[i] (a hipEvent_t, or NULL to skip that mark) on `stream` at the
 * stage boundaries: [0] before the projection, [1] before the state setup
 * (its own launch only when Seq = 0), [2] before the recurrent steps, [3]
 * after them, [4] at the end (the outputs have no pass of their own).
 * Lets a caller time each stage with events on the stream the kernels run on. */
int rnn_encode_timed(const rnn_problem* problem, const rnn_operands* operands,
                     void* xw_scratch, void* state_scratch, void* stream, void* const events[5]);

/* rnn_encode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * projection and state scratch come from a fixed device array of
 * RNN_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * (allocated when the library's code is loaded on that device, released when
 * the process ends); the caller still passes inputs and outputs.  The layer
 * runs on the device current on the calling thread, which must be the
 * stream's device.  Nothing is allocated and nothing needs clearing: each call
 * writes every scratch value its results depend on.  All calls on one device share that
 * device's array, so calls that overlap in time on one device race: order
 * them on one stream (or with an event).  Errors as rnn_encode, plus
 * RNN_ERR_UNSUPPORTED when the layer's scratch (rnn_scratch_size: the two
 * sizes, each rounded up to 256 bytes) exceeds RNN_NOALLOC_SCRATCH_BYTES; as
 * with rnn_encode, nothing is enqueued when a check fails. */
#define RNN_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int rnn_encode_noalloc(const rnn_problem* problem, const rnn_operands* operands, void* stream);

/* Host-side check of sequence lengths (the page asks callers to validate them
 * on the host): every value in [0, seq].  On success *max_len_out (if not
 * NULL) receives the largest length, usable as max_length. */
int rnn_validate_lengths(const int32_t* host_lens, int64_t batch, int64_t seq, int64_t* max_len_out);

/* What rnn_encode will launch for this problem, and which arithmetic units
 * carry its products (for measurement against the right peak). */
typedef enum {
  RNN_PRODUCTS_F32_VALU = 0,   /* f32 fused multiply-adds on the vector ALUs */
  RNN_PRODUCTS_F32_MFMA = 1,   /* f32 matrix cores */
  RNN_PRODUCTS_F16_MFMA = 2,   /* f16 matrix cores, f32 accumulation; in the steps h as two f16 halves
                                  (two products per product of the method) */
  RNN_PRODUCTS_BF16X3_MFMA = 3 /* bf16 matrix cores, each f32 product as three bf16 products */
} rnn_products;
typedef struct {
  int32_t engine;          /* rnn_engine actually used */
  int32_t steps;           /* number of recurrent steps run (max_length or S) */
  int32_t launches;        /* kernel launches per rnn_encode (with the persistent engine, one of them is
                              the fallback kernel that follows the step kernel and exits at once
                              unless the step kernel's grid was not all resident) */
  int32_t step_blocks;     /* workgroups of the persistent step kernel (0 for the per-step engine) */
  int32_t step_launches;   /* launches of the recurrent-step kernel per rnn_encode */
  int32_t proj_products;   /* rnn_products of the input projection */
  int32_t step_products;   /* rnn_products of the recurrent products (R * h) */
  int32_t xw_chunk_steps;  /* steps per chunk of the projection (the steps run when it is one chunk) */
  int32_t xw_slots;        /* 1, or 2 (a ring of chunks) */
} rnn_plan_info;
int rnn_problem_plan(const rnn_problem* problem, rnn_plan_info* info);

/* What the recurrent-step stage of the last rnn_encode on this state scratch
 * did, read back from the status words a persistent step kernel leaves in the
 * state scratch ("Recurrent layers" page, "How a layer runs", item 3: the
 * steps; here they may run in one launch whose workgroups wait on one
 * another).  Enqueues a copy of those words on `stream` (a hipStream_t; NULL
 * is the default stream) and waits for the stream, so it returns after every
 * call enqueued there before it has finished.
 *   persistent          1 when a persistent step kernel ran, else 0 (and the
 *                       fields below are 0)
 *   fallback_workgroups 0: every workgroup of the grid ran at once (the fast
 *                       path); k > 0: the device did not hold the whole grid
 *                       at once (say, it was partly busy with other work) and
 *                       k workgroups took the place of the others in turn.
 *                       The outputs are bit-identical either way; the
 *                       fallback is slower.
 *   timed_out           1: a wait between workgroups passed its safety bound
 *                       (several seconds) and the kernel ended early: the
 *                       outputs are incomplete
 * Errors: RNN_ERR_ARG for a NULL argument (state_scratch may be NULL only
 * when rnn_scratch_size reports 0 state bytes), RNN_ERR_HIP when the copy
 * fails.  The state scratch is owned by the caller and only read. */
typedef struct {
  int32_t persistent;
  int32_t fallback_workgroups;
  int32_t timed_out;
} rnn_run_status;
int rnn_read_run_status(const rnn_problem* problem, const void* state_scratch, void* stream, rnn_run_status* out);

/* Message of the last failed call on this thread ("" if none): the cell
 * (LSTM, GRU or RNN) and the argument at fault, as the page's shape
 * exception names them ("Scratch").  The string is owned by the library and
 * valid until the thread's next call. */
const char* rnn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ONNX_RNN_MI355X_H */

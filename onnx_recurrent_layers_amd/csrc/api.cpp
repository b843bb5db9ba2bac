// api.cpp -- the C ABI: validation, planning, scratch sizing and the launch
// sequence of one layer ("Recurrent layers" page, "How a layer runs": input
// projection, state setup, the recurrent steps, the outputs written by the
// steps themselves).
//
// Every check runs in 64-bit checked arithmetic before anything is enqueued
// (the page's "Scratch" paragraph); messages name the cell and the argument.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "plan.h"

using namespace rnnhip;

namespace {

thread_local std::string g_error;

const char* cell_name(int cell) {
  switch (cell) {
    case RNN_CELL_LSTM: return "LSTM";
    case RNN_CELL_GRU: return "GRU";
    case RNN_CELL_RNN: return "RNN";
    default: return "RNN layer";
  }
}

int fail(int code, int cell, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = std::string(cell_name(cell)) + ": " + buf;
  return code;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  int64_t t;
  return mul_ok(a, b, &t) && mul_ok(t, c, out);
}

bool mul4(int64_t a, int64_t b, int64_t c, int64_t d, int64_t* out) {
  int64_t t;
  return mul3(a, b, c, &t) && mul_ok(t, d, out);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The stream on which the per-step engine runs the later chunks of a chunked
// projection, beside the caller's stream: one per device, created on first
// use (default priority), kept until the process ends.
hipError_t side_stream(hipStream_t* out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev] && (e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking)) != hipSuccess) return e;
  *out = streams[dev];
  return hipSuccess;
}

// Events ordering the two streams of one chunked rnn_encode (created and
// destroyed per call: calls on different threads never share them).
struct ChunkEvents {
  hipEvent_t ev[5] = {};   // fork, projection done [2], steps done [2]
  ~ChunkEvents() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  hipError_t create() {
    for (hipEvent_t& e : ev) {
      hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
};

// Largest tensor byte count accepted: keeps every offset computation far from
// 64-bit overflow.
constexpr int64_t kMaxBytes = int64_t(1) << 52;

}  // namespace

extern "C" const char* rnn_last_error(void) { return g_error.c_str(); }

extern "C" int rnn_problem_create(const rnn_problem_desc* desc, rnn_problem** out) {
  g_error.clear();
  if (out) *out = nullptr;
  if (!desc) return fail(RNN_ERR_ARG, -1, "desc: NULL");
  const int cell = desc->cell;
  if (!out) return fail(RNN_ERR_ARG, cell, "out: NULL");
  if (cell != RNN_CELL_RNN && cell != RNN_CELL_GRU && cell != RNN_CELL_LSTM)
    return fail(RNN_ERR_ARG, cell, "cell: unknown value %d", cell);
  if (desc->dtype != RNN_DTYPE_F32 && desc->dtype != RNN_DTYPE_F16)
    return fail(RNN_ERR_ARG, cell, "dtype: unknown value %d", desc->dtype);
  if (desc->direction < RNN_DIR_FORWARD || desc->direction > RNN_DIR_BIDIRECTIONAL)
    return fail(RNN_ERR_ARG, cell, "direction: unknown value %d", desc->direction);
  if (desc->layout != 0 && desc->layout != 1)
    return fail(RNN_ERR_ARG, cell, "layout: must be 0 or 1, got %d", desc->layout);
  if (desc->seq < 0) return fail(RNN_ERR_SHAPE, cell, "seq: negative (%lld)", (long long)desc->seq);
  if (desc->batch < 0) return fail(RNN_ERR_SHAPE, cell, "batch: negative (%lld)", (long long)desc->batch);
  if (desc->input < 0) return fail(RNN_ERR_SHAPE, cell, "input: negative (%lld)", (long long)desc->input);
  if (desc->hidden < 1) return fail(RNN_ERR_SHAPE, cell, "hidden: must be at least 1 (%lld)", (long long)desc->hidden);
  if (std::isnan(desc->clip)) return fail(RNN_ERR_ARG, cell, "clip: NaN");
  if (desc->input_forget != 0 && desc->input_forget != 1)
    return fail(RNN_ERR_ARG, cell, "input_forget: must be 0 or 1");
  if (desc->input_forget && cell != RNN_CELL_LSTM)
    return fail(RNN_ERR_ARG, cell, "input_forget: only an LSTM takes input_forget");
  if (desc->linear_before_reset != 0 && desc->linear_before_reset != 1)
    return fail(RNN_ERR_ARG, cell, "linear_before_reset: must be 0 or 1");
  if (desc->linear_before_reset && cell != RNN_CELL_GRU)
    return fail(RNN_ERR_ARG, cell, "linear_before_reset: only a GRU takes linear_before_reset");
  if (desc->engine < RNN_ENGINE_AUTO || desc->engine > RNN_ENGINE_PERSISTENT)
    return fail(RNN_ERR_ARG, cell, "engine: unknown value %d", desc->engine);
  if (desc->xw_chunk_steps < 0)
    return fail(RNN_ERR_SHAPE, cell, "xw_chunk_steps: negative (%lld)", (long long)desc->xw_chunk_steps);
  if (desc->x_bidirectional_y != 0 && desc->x_bidirectional_y != 1)
    return fail(RNN_ERR_ARG, cell, "x_bidirectional_y: must be 0 or 1");
  if (desc->x_bidirectional_y && desc->input % 2 != 0)
    return fail(RNN_ERR_SHAPE, cell, "x_bidirectional_y: input must be even (two directions of H'), got %lld",
                (long long)desc->input);

  Problem* p = new (std::nothrow) Problem();
  if (!p) return fail(RNN_ERR_ARG, cell, "out of host memory");
  p->desc = *desc;
  p->G = cell == RNN_CELL_LSTM ? 4 : (cell == RNN_CELL_GRU ? 3 : 1);
  p->slots = cell == RNN_CELL_LSTM ? 3 : (cell == RNN_CELL_GRU ? 2 : 1);
  p->D = desc->direction == RNN_DIR_BIDIRECTIONAL ? 2 : 1;
  p->S = desc->seq;
  p->B = desc->batch;
  p->I = desc->input;
  p->H = desc->hidden;
  p->esize = desc->dtype == RNN_DTYPE_F32 ? 4 : 2;

  auto bad = [&](int code, const char* fmt, auto... args) {
    delete p;
    return fail(code, cell, fmt, args...);
  };
  if (desc->num_activations != p->slots * p->D)
    return bad(RNN_ERR_ARG, "activations: expected %d (slots x directions), got %d", p->slots * p->D,
               desc->num_activations);
  for (int i = 0; i < desc->num_activations; ++i)
    if (desc->activations[i].kind < RNN_ACT_RELU || desc->activations[i].kind > RNN_ACT_SOFTPLUS)
      return bad(RNN_ERR_ARG, "activations[%d]: unknown kind %d", i, desc->activations[i].kind);
  if (desc->max_length < 0 || desc->max_length > desc->seq)
    return bad(RNN_ERR_SHAPE, "max_length: must be in [0, seq], got %lld", (long long)desc->max_length);
  p->steps = desc->max_length > 0 ? desc->max_length : desc->seq;
  p->def_acts = true;
  for (int d = 0; d < p->D; ++d)
    for (int k = 0; k < p->slots; ++k) {
      const int kind = desc->activations[d * p->slots + k].kind;
      const int want = cell == RNN_CELL_RNN ? RNN_ACT_TANH : (k == 0 ? RNN_ACT_SIGMOID : RNN_ACT_TANH);
      if (kind != want) p->def_acts = false;
    }
  if (p->H > (int64_t(1) << 24)) return bad(RNN_ERR_UNSUPPORTED, "hidden: above 16777216");
  if (p->B > (int64_t(1) << 30)) return bad(RNN_ERR_UNSUPPORTED, "batch: above 2^30");
  if (p->S > (int64_t(1) << 30)) return bad(RNN_ERR_UNSUPPORTED, "seq: above 2^30");

  // Tensor sizes in checked 64-bit arithmetic.
  int64_t n;
  const int64_t GH = p->G * p->H;
  if (!mul3(p->S, p->B, p->I, &n) || !mul_ok(n, p->esize, &n) || n > kMaxBytes)
    return bad(RNN_ERR_SHAPE, "X: size overflows");
  if (!mul3(p->D, GH, p->I, &n) || !mul_ok(n, p->esize, &n) || n > kMaxBytes)
    return bad(RNN_ERR_SHAPE, "W: size overflows");
  if (!mul3(p->D, GH, p->H, &n) || !mul_ok(n, p->esize, &n) || n > kMaxBytes)
    return bad(RNN_ERR_SHAPE, "R: size overflows");
  if (!mul4(p->S, p->D, p->B, p->H, &n) || !mul_ok(n, p->esize, &n) || n > kMaxBytes)
    return bad(RNN_ERR_SHAPE, "Y: size overflows");
  int64_t xw;
  if (!mul4(p->D, p->S, p->B, GH, &xw) || !mul_ok(xw, 4, &xw) || xw > kMaxBytes)
    return bad(RNN_ERR_SHAPE, "xw scratch: size overflows");
  int64_t dbh;
  if (!mul3(p->D, p->B, p->H, &dbh) || dbh > kMaxBytes / 8) return bad(RNN_ERR_SHAPE, "state: size overflows");
  // The matrix-core step's tile, once: every launch of this problem uses it
  // (RNN_MFMA_TILE is read here only).
  if (mfma_step_supported(*p))
    mfma_tile(int(p->B), int(p->H), p->D, p->G - ((cell == RNN_CELL_LSTM && desc->input_forget) ? 1 : 0),
              &p->mfma_bm, &p->mfma_uj);
  // Engine choice.
  int blocks = 0, units = 0, wpd = 0;
  const bool pers_ok = persistent_supported(*p, &blocks, &units, &wpd);
  int engine = desc->engine;
  if (p->S == 0 || p->steps == 0 || p->B == 0) engine = RNN_ENGINE_LAUNCH;  // nothing to step
  // f32 layers whose per-step matrix-core product is 2^28 flops or more run it
  // on the bf16 matrix cores (h and R as bf16 hi/lo planes; R is split once
  // per layer); RNN_F32_SPLIT=0 or 1 overrides the choice, as for the
  // projection below.
  if (desc->dtype == RNN_DTYPE_F32 && !pers_ok && mfma_step_supported(*p)) {
    StepArgs t{};
    t.G = p->G;
    t.D = p->D;
    t.H = int(p->H);
    t.B = int(p->B);
    const double flops = 2.0 * double(p->D) * double(p->B) * double(GH) * double(p->H);
    bool want = flops >= 268435456.0;
    if (const char* e = std::getenv("RNN_F32_SPLIT")) want = std::atoi(e) != 0;
    p->f32_split_step = want && step_dma_supported(t, 2);
  }
  // Batches above eight: the matrix-core step, in one persistent launch when
  // its tiles fit the chip (else one launch per step).  The automatic choice
  // takes the persistent launch for f16 layers with the default activations
  // (split h), where it measured faster than one launch per step (LSTM
  // 256/64/1024/1024: 2.41 against 2.53 ms of steps), and for layers whose
  // per-step product is below 2^28 flops, whose steps are too short to cover
  // a launch each; large f32 layers measured slower persistent (RNN
  // 1024/256/1024/2048 in bf16 split mode: 35 against 33 ms).
  int mfma_tiles = 0;
  const bool pers_mfma_ok =
      !pers_ok && p->S > 0 && p->steps > 0 && p->B > 0 && mfma_persistent_supported(*p, &mfma_tiles);
  const double step_flops = 2.0 * double(p->D) * double(p->B) * double(GH) * double(p->H);
  const bool pers_mfma_auto =
      pers_mfma_ok && ((desc->dtype == RNN_DTYPE_F16 && p->def_acts) || step_flops < 268435456.0);
  if (engine == RNN_ENGINE_AUTO)
    engine = (pers_ok || pers_mfma_auto) ? RNN_ENGINE_PERSISTENT : RNN_ENGINE_LAUNCH;
  if (engine == RNN_ENGINE_PERSISTENT && !pers_ok && !pers_mfma_ok)
    return bad(RNN_ERR_UNSUPPORTED, "engine: the persistent engine does not take this shape");
  p->engine = engine;
  p->pers_mfma = engine == RNN_ENGINE_PERSISTENT && !pers_ok;
  // h as 16-bit halves for the matrix-core step: bf16 with the bf16 mode;
  // f16 for f16 layers with the default activations whose rows are whole
  // 16-byte segments (the direct-to-LDS kernel's f16 mode; whether it runs is
  // settled at encode time by R's alignment, and the planes are written in
  // any case)
  if (p->f32_split_step) {
    p->h_split = 2;
  } else if (!pers_ok && mfma_step_supported(*p) && desc->dtype == RNN_DTYPE_F16 && p->def_acts) {
    StepArgs t{};
    t.G = p->G;
    t.D = p->D;
    t.H = int(p->H);
    t.B = int(p->B);
    if (step_dma_supported(t, 1)) p->h_split = 1;
  }
  if (p->pers_mfma) p->pers_blocks = mfma_tiles;
  // f32 projections of 2^32 flops and more run as three bf16 products (the
  // f32 matrix cores have a sixteenth of the bf16 rate); RNN_F32_SPLIT=0 or 1
  // overrides the choice, so that tests reach both forms on any shape.
  if (desc->dtype == RNN_DTYPE_F32) {
    const double flops = 2.0 * double(p->D) * double(p->S) * double(p->B) * double(GH) * double(p->I);
    p->f32_split_proj = flops >= 4294967296.0;
    if (const char* e = std::getenv("RNN_F32_SPLIT")) p->f32_split_proj = std::atoi(e) != 0;
  }

  // The projection scratch, step-major.  The per-step engine may run the
  // projection in chunks through a ring of two slots: at the caller's
  // request, or when the whole projection would exceed 512 MiB (then slots
  // of 256 MiB, which keeps each chunk's projection in whole 256x256 tiles
  // for the large layers that reach this size).  The persistent engines read
  // every step's projection in their one launch: one slot of every step.
  {
    const int64_t per_step = int64_t(p->D) * p->B * GH * 4;   // bytes of one step of every direction
    int64_t tc = p->steps;
    if (engine == RNN_ENGINE_LAUNCH && p->steps > 0 && per_step > 0) {
      if (desc->xw_chunk_steps > 0) {
        tc = std::min<int64_t>(desc->xw_chunk_steps, p->steps);
      } else if (p->steps * per_step > (int64_t(512) << 20)) {
        tc = std::max<int64_t>(1, (int64_t(256) << 20) / per_step);
      }
    }
    p->xw_tc = std::max<int64_t>(tc, 1);
    p->xw_slots = tc < p->steps ? 2 : 1;
    p->xw_bytes = (p->S > 0 && p->B > 0 && p->steps > 0) ? size_t(p->xw_slots) * size_t(p->xw_tc) * size_t(per_step) : 0;
  }

  StateLayout& st = p->st;
  st = StateLayout{};
  size_t off = 0;
  if (engine == RNN_ENGINE_PERSISTENT && !p->pers_mfma) {
    p->pers_blocks = blocks;
    p->pers_units = units;
    p->pers_wg_per_dir = wpd;
    st.xch = off;   off = align256(off + 2 * size_t(dbh) * 8);
    st.xch2 = off;  off = align256(off + (cell == RNN_CELL_GRU && !desc->linear_before_reset ? 2 * size_t(dbh) * 8 : 0));
    st.status = off; off = align256(off + 3 * 4);   // status, arrival tickets, residency decision
    // what the fallback (taken when the grid does not run all at once) keeps
    // in memory where the fast path keeps registers: the cell state and a
    // GRU's z between its two phases.  No h slots: h travels in the words.
    st.cell = off;  off = align256(off + size_t(dbh) * 4);
    st.zbuf = off;  off = align256(off + (cell == RNN_CELL_GRU ? size_t(dbh) * 4 : 0));
    st.hbuf = st.rhbuf = SIZE_MAX;
  } else {
    st.hbuf = off;  off = align256(off + 2 * size_t(dbh) * 4);
    st.cell = off;  off = align256(off + size_t(dbh) * 4);
    st.zbuf = off;  off = align256(off + (cell == RNN_CELL_GRU ? size_t(dbh) * 4 : 0));
    st.rhbuf = off; off = align256(off + (cell == RNN_CELL_GRU ? size_t(dbh) * 4 : 0));
    if (p->f32_split_step) {
      st.rsplit = off;  off = align256(off + 2 * size_t(p->D) * size_t(GH) * size_t(p->H) * 2);
    }
    if (p->h_split) {
      st.hsplit = off;  off = align256(off + 4 * size_t(dbh) * 2);
      st.rhsplit = off; off = align256(off + (cell == RNN_CELL_GRU && !desc->linear_before_reset ? 2 * size_t(dbh) * 2 : 0));
    }
    if (p->pers_mfma) {
      st.flags = off;   off = align256(off + size_t(kPersistentMfmaTiles) * 4);
      st.status = off;  off = align256(off + 3 * 4);   // status, arrival tickets, residency decision
    }
  }
  st.total = p->B > 0 ? off : 0;

  *out = reinterpret_cast<rnn_problem*>(p);
  return RNN_OK;
}

extern "C" void rnn_problem_destroy(rnn_problem* problem) { delete reinterpret_cast<Problem*>(problem); }

extern "C" int rnn_scratch_size(const rnn_problem* problem, size_t* xw_bytes, size_t* state_bytes) {
  g_error.clear();
  if (!problem) return fail(RNN_ERR_ARG, -1, "problem: NULL");
  const Problem* p = reinterpret_cast<const Problem*>(problem);
  if (xw_bytes) *xw_bytes = p->xw_bytes;
  if (state_bytes) *state_bytes = p->st.total;
  return RNN_OK;
}

extern "C" int rnn_validate_lengths(const int32_t* host_lens, int64_t batch, int64_t seq, int64_t* max_len_out) {
  g_error.clear();
  if (batch < 0) return fail(RNN_ERR_SHAPE, -1, "sequence_lens: negative batch");
  if (batch > 0 && !host_lens) return fail(RNN_ERR_ARG, -1, "sequence_lens: NULL");
  int64_t mx = 0;
  for (int64_t b = 0; b < batch; ++b) {
    if (host_lens[b] < 0 || host_lens[b] > seq)
      return fail(RNN_ERR_SHAPE, -1, "sequence_lens[%lld]: %d outside [0, %lld]", (long long)b, host_lens[b],
                  (long long)seq);
    if (host_lens[b] > mx) mx = host_lens[b];
  }
  if (max_len_out) *max_len_out = mx;
  return RNN_OK;
}

namespace {

int step_launch_count(const Problem& p) {
  if (p.engine == RNN_ENGINE_PERSISTENT) return p.steps > 0 ? 1 : 0;
  const int per = (p.desc.cell == RNN_CELL_GRU && !p.desc.linear_before_reset) ? 2 : 1;
  return int(p.steps) * per;
}

}  // namespace

extern "C" int rnn_problem_plan(const rnn_problem* problem, rnn_plan_info* info) {
  g_error.clear();
  if (!problem || !info) return fail(RNN_ERR_ARG, -1, "problem/info: NULL");
  const Problem* p = reinterpret_cast<const Problem*>(problem);
  info->engine = p->engine;
  info->steps = int32_t(p->steps);
  info->step_blocks = p->engine == RNN_ENGINE_PERSISTENT ? p->pers_blocks : 0;
  int n = 0;
  if (p->B > 0) {
    n += 1;                        // projection with the state setup (or the setup alone when Seq = 0); the
                                   // steps and the setup write the outputs
    if (p->S > 0) n += step_launch_count(*p);
    if (p->S > 0 && p->steps > 0) n += int((p->steps + p->xw_tc - 1) / p->xw_tc) - 1;   // the later chunks' projections
    if (p->S > 0 && p->steps > 0 && p->engine == RNN_ENGINE_PERSISTENT) n += 1;   // the fallback kernel
    if (p->S > 0 && p->f32_split_step) n += 1;   // R split into bf16 planes
  }
  info->launches = n;
  info->step_launches = (p->B > 0 && p->S > 0) ? step_launch_count(*p) : 0;
  // projection: f16 tensors on the f16 matrix cores; f32 tensors on the f32
  // matrix cores or as three bf16 products
  info->proj_products = p->desc.dtype == RNN_DTYPE_F16 ? RNN_PRODUCTS_F16_MFMA
                        : p->f32_split_proj ? RNN_PRODUCTS_BF16X3_MFMA : RNN_PRODUCTS_F32_MFMA;
  // steps: the small-batch persistent engine uses the f16 matrix cores for f16
  // layers with the default activations and 3 to 8 rows (padded to 4 or 8),
  // else vector-ALU products; the matrix-core step (16 rows and more) runs in
  // its mode; the per-step engine for other batches uses the vector ALUs
  if (p->engine == RNN_ENGINE_PERSISTENT && !p->pers_mfma)
    info->step_products = (p->esize == 2 && p->def_acts && p->B >= 3) ? RNN_PRODUCTS_F16_MFMA : RNN_PRODUCTS_F32_VALU;
  else if (mfma_step_supported(*p))
    info->step_products = p->f32_split_step ? RNN_PRODUCTS_BF16X3_MFMA
                          : (p->esize == 2 && p->def_acts) ? RNN_PRODUCTS_F16_MFMA : RNN_PRODUCTS_F32_MFMA;
  else
    info->step_products = RNN_PRODUCTS_F32_VALU;
  info->xw_chunk_steps = int32_t(p->xw_tc);
  info->xw_slots = p->xw_slots;
  return RNN_OK;
}

extern "C" int rnn_read_run_status(const rnn_problem* problem, const void* state_scratch, void* stream,
                                   rnn_run_status* out) {
  g_error.clear();
  if (!problem || !out) return fail(RNN_ERR_ARG, -1, "problem/out: NULL");
  const Problem& p = *reinterpret_cast<const Problem*>(problem);
  *out = rnn_run_status{0, 0, 0};
  if (p.engine != RNN_ENGINE_PERSISTENT || p.st.total == 0) return RNN_OK;
  if (!state_scratch) return fail(RNN_ERR_ARG, p.desc.cell, "state_scratch: NULL");
  // status (1: a wait passed its bound), arrival tickets, residency decision
  // (0: no kernel ran, 1: every workgroup at once, 2 | k << 8: k workgroups
  // ran the fallback)
  int words[3] = {0, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(words, static_cast<const char*>(state_scratch) + p.st.status, sizeof words,
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(RNN_ERR_HIP, p.desc.cell, "status read: %s", hipGetErrorString(e));
  if (words[2] == 0) return RNN_OK;
  out->persistent = 1;
  out->fallback_workgroups = words[2] == 1 ? 0 : (words[2] >> 8);
  out->timed_out = words[0] != 0;
  return RNN_OK;
}

namespace {

// Resolve one tensor to a byte pointer, checking alignment and offset.
int resolve(const rnn_tensor& t, int esize, int cell, const char* name, bool required, const char** out) {
  *out = nullptr;
  if (!t.ptr) {
    if (required) return fail(RNN_ERR_ARG, cell, "%s: NULL", name);
    return RNN_OK;
  }
  if (t.elem_offset < 0) return fail(RNN_ERR_ARG, cell, "%s: negative element offset", name);
  if (t.elem_offset > kMaxBytes / esize) return fail(RNN_ERR_SHAPE, cell, "%s: element offset overflows", name);
  const char* base = static_cast<const char*>(t.ptr) + t.elem_offset * esize;
  if (reinterpret_cast<uintptr_t>(base) % uintptr_t(esize) != 0)
    return fail(RNN_ERR_ARG, cell, "%s: address not aligned to its %d-byte element", name, esize);
  *out = base;
  return RNN_OK;
}

}  // namespace

namespace {

int encode_impl(const rnn_problem* problem, const rnn_operands* ops, void* xw_scratch, void* state_scratch,
                void* stream, void* const* events, bool may_fork);

}  // namespace

namespace rnnhip {

int encode_layer(const rnn_problem* problem, const rnn_operands* ops, void* xw_scratch, void* state_scratch,
                 void* stream) {
  // (no second stream: this path serves callers that cannot create objects)
  return encode_impl(problem, ops, xw_scratch, state_scratch, stream, nullptr, false);
}

int set_error(int code, int cell, const char* msg) { return fail(code, cell, "%s", msg); }

}  // namespace rnnhip

extern "C" int rnn_encode(const rnn_problem* problem, const rnn_operands* ops, void* xw_scratch,
                          void* state_scratch, void* stream) {
  return encode_impl(problem, ops, xw_scratch, state_scratch, stream, nullptr, true);
}

extern "C" int rnn_encode_timed(const rnn_problem* problem, const rnn_operands* ops, void* xw_scratch,
                                void* state_scratch, void* stream, void* const events[5]) {
  return encode_impl(problem, ops, xw_scratch, state_scratch, stream, events, true);
}

namespace {

int encode_impl(const rnn_problem* problem, const rnn_operands* ops, void* xw_scratch, void* state_scratch,
                void* stream, void* const* events, bool may_fork) {
  g_error.clear();
  // a chunked projection may run on a second stream, overlapping the steps
  // of the chunk before (RNN_CHUNK_OVERLAP=1).  Off by default: measured on
  // the RNN 1024/256/1024/2048 layer it gains nothing (40.2 ms against 40.0
  // ms on the caller's stream), since every step kernel holds the LDS of
  // every compute unit and the projection's tiles only run between steps.
  bool chunk_overlap = false;
  if (const char* env = std::getenv("RNN_CHUNK_OVERLAP")) chunk_overlap = may_fork && std::atoi(env) != 0;
  if (!problem) return fail(RNN_ERR_ARG, -1, "problem: NULL");
  const Problem& p = *reinterpret_cast<const Problem*>(problem);
  const int cell = p.desc.cell;
  if (!ops) return fail(RNN_ERR_ARG, cell, "operands: NULL");
  const bool lstm = cell == RNN_CELL_LSTM;
  if (!lstm && ops->initial_c.ptr) return fail(RNN_ERR_ARG, cell, "initial_c: only an LSTM takes initial_c");
  if (!lstm && ops->P.ptr) return fail(RNN_ERR_ARG, cell, "P: only an LSTM takes peepholes");
  if (!lstm && ops->Y_c.ptr) return fail(RNN_ERR_ARG, cell, "Y_c: only an LSTM has Y_c");

  const int es = p.esize;
  const char *X, *W, *R, *Bp, *lens, *ih, *ic, *P, *Y, *Yh, *Yc;
  int rc;
  if ((rc = resolve(ops->X, es, cell, "X", true, &X))) return rc;
  if ((rc = resolve(ops->W, es, cell, "W", true, &W))) return rc;
  if ((rc = resolve(ops->R, es, cell, "R", true, &R))) return rc;
  if ((rc = resolve(ops->B, es, cell, "B", false, &Bp))) return rc;
  if ((rc = resolve(ops->sequence_lens, 4, cell, "sequence_lens", false, &lens))) return rc;
  if ((rc = resolve(ops->initial_h, es, cell, "initial_h", false, &ih))) return rc;
  if ((rc = resolve(ops->initial_c, es, cell, "initial_c", false, &ic))) return rc;
  if ((rc = resolve(ops->P, es, cell, "P", false, &P))) return rc;
  if ((rc = resolve(ops->Y, es, cell, "Y", false, &Y))) return rc;
  if ((rc = resolve(ops->Y_h, es, cell, "Y_h", false, &Yh))) return rc;
  if ((rc = resolve(ops->Y_c, es, cell, "Y_c", false, &Yc))) return rc;

  if (p.B == 0) return RNN_OK;  // nothing is recorded
  if (p.xw_bytes > 0) {
    if (!xw_scratch) return fail(RNN_ERR_ARG, cell, "xw_scratch: NULL (needs %zu bytes)", p.xw_bytes);
    if (reinterpret_cast<uintptr_t>(xw_scratch) % 256) return fail(RNN_ERR_ARG, cell, "xw_scratch: not 256-byte aligned");
  }
  if (!state_scratch) return fail(RNN_ERR_ARG, cell, "state_scratch: NULL (needs %zu bytes)", p.st.total);
  if (reinterpret_cast<uintptr_t>(state_scratch) % 256)
    return fail(RNN_ERR_ARG, cell, "state_scratch: not 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* st = static_cast<char*>(state_scratch);
  const bool pers = p.engine == RNN_ENGINE_PERSISTENT && !p.pers_mfma;   // the small-batch persistent engine
  float* hbuf = p.st.hbuf == SIZE_MAX ? nullptr : reinterpret_cast<float*>(st + p.st.hbuf);
  float* cstate = reinterpret_cast<float*>(st + p.st.cell);
  int* status = (pers || p.pers_mfma) ? reinterpret_cast<int*>(st + p.st.status) : nullptr;
  int* flags = p.pers_mfma ? reinterpret_cast<int*>(st + p.st.flags) : nullptr;

  // -- state setup (slot 0 of the state, the cell state, the exchange words)
  SetupArgs sa{};
  sa.D = p.D;
  sa.B = int(p.B);
  sa.H = int(p.H);
  sa.layout = p.desc.layout;
  sa.dtype = p.desc.dtype;
  sa.init_h = ih;
  sa.init_c = ic;
  sa.hbuf = hbuf;
  unsigned short* rsplit = p.f32_split_step ? reinterpret_cast<unsigned short*>(st + p.st.rsplit) : nullptr;
  unsigned short* hsplit = p.h_split ? reinterpret_cast<unsigned short*>(st + p.st.hsplit) : nullptr;
  sa.hsplit = hsplit;
  sa.split_kind = p.h_split;
  sa.cell_state = cstate;
  sa.xch = pers ? reinterpret_cast<unsigned long long*>(st + p.st.xch) : nullptr;
  sa.xch2 = (pers && cell == RNN_CELL_GRU && !p.desc.linear_before_reset)
                ? reinterpret_cast<unsigned long long*>(st + p.st.xch2) : nullptr;
  sa.status = status;
  sa.flags = flags;
  sa.nflags = flags ? kPersistentMfmaTiles : 0;
  sa.Y = const_cast<char*>(Y);
  sa.Y_h = const_cast<char*>(Yh);
  sa.Y_c = const_cast<char*>(Yc);
  sa.lens = reinterpret_cast<const int32_t*>(lens);
  sa.S = int(p.S);
  sa.steps = int(p.steps);

  StepArgs a{};
  a.cell = cell;
  a.G = p.G;
  a.D = p.D;
  a.H = int(p.H);
  a.B = int(p.B);
  a.S = int(p.S);
  a.steps = int(p.steps);
  a.dir_reverse[0] = p.desc.direction == RNN_DIR_REVERSE;
  a.dir_reverse[1] = 1;
  a.dtype = p.desc.dtype;
  a.R = R;
  a.bias = Bp;
  a.P = P;
  a.lens = reinterpret_cast<const int32_t*>(lens);
  a.xw = static_cast<const float*>(xw_scratch);
  a.xw_tc = int(p.xw_tc);
  a.hbuf = hbuf;
  a.rsplit = rsplit;
  a.hsplit = hsplit;
  a.rhsplit = (p.h_split && cell == RNN_CELL_GRU && !p.desc.linear_before_reset)
                  ? reinterpret_cast<unsigned short*>(st + p.st.rhsplit) : nullptr;
  a.split_kind = p.h_split;
  a.Y = const_cast<char*>(Y);
  a.Y_h = const_cast<char*>(Yh);
  a.Y_c = const_cast<char*>(Yc);
  a.layout = p.desc.layout;
  a.cell_state = cstate;
  a.zbuf = reinterpret_cast<float*>(st + p.st.zbuf);
  a.rhbuf = p.st.rhbuf == SIZE_MAX ? nullptr : reinterpret_cast<float*>(st + p.st.rhbuf);
  a.xch = reinterpret_cast<unsigned long long*>(st + p.st.xch);
  a.xch2 = reinterpret_cast<unsigned long long*>(st + p.st.xch2);
  a.clip = p.desc.clip > 0.f ? p.desc.clip : 0.f;
  a.input_forget = p.desc.input_forget;
  a.lbr = p.desc.linear_before_reset;
  a.slots = p.slots;
  for (int i = 0; i < p.slots * p.D; ++i)
    a.act[i] = Act{p.desc.activations[i].kind, p.desc.activations[i].alpha, p.desc.activations[i].beta};

  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    if (events && events[i]) return hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
    return hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return fail(RNN_ERR_HIP, cell, "event record: %s", hipGetErrorString(e));
  // 1. input projection: chunk c covers steps [c*tc, (c+1)*tc) and fills
  // slot c & 1 of the projection scratch (one chunk unless the per-step
  // engine runs it in chunks, interleaved with the steps below)
  const int64_t tc = p.xw_tc;
  const int64_t nchunks = p.steps > 0 ? (p.steps + tc - 1) / tc : 0;
  ProjArgs pa{};
  pa.X = X;
  pa.W = W;
  pa.N = p.G * p.H;
  pa.K = p.I;
  pa.S = p.S;
  pa.B = p.B;
  pa.layout = p.desc.layout;
  pa.D = p.D;
  pa.skip_block = (lstm && p.desc.input_forget) ? 2 : -1;
  pa.H = p.H;
  pa.f32_split = p.f32_split_proj;
  pa.lens = reinterpret_cast<const int32_t*>(lens);
  pa.rev[0] = a.dir_reverse[0];
  pa.rev[1] = a.dir_reverse[1];
  pa.steps = p.steps;
  pa.out_dstride = tc * p.B * pa.N;
  // X as the Y [S,2,B,I/2] of a bidirectional layout-0 layer: rows in two
  // pieces, the second (B-1)*I/2 elements after the end of the first
  const bool split_x = p.desc.x_bidirectional_y && p.desc.layout == 0 && p.B > 1;
  pa.xkh = split_x ? p.I / 2 : p.I;
  pa.xjump = split_x ? (p.B - 1) * (p.I / 2) : 0;
  auto project = [&](int64_t c) -> hipError_t {
    ProjArgs q = pa;
    q.s0 = c * tc;
    q.M = std::min<int64_t>(tc, p.steps - q.s0) * p.B;
    q.xw = static_cast<float*>(xw_scratch) + (c & 1) * int64_t(p.D) * pa.out_dstride;
    // the state setup rides in the first chunk's launch (extra workgroups)
    SetupArgs none{};
    return launch_projection(q, c == 0 ? sa : none, p.desc.dtype, s);
  };
  if (nchunks > 0 && (e = project(0)) != hipSuccess)
    return fail(RNN_ERR_HIP, cell, "projection launch: %s", hipGetErrorString(e));
  if ((e = mark(1)) != hipSuccess) return fail(RNN_ERR_HIP, cell, "event record: %s", hipGetErrorString(e));
  // 2. state setup (its own launch only when there is no projection)
  if (nchunks == 0 && (e = launch_setup(sa, s)) != hipSuccess)
    return fail(RNN_ERR_HIP, cell, "setup launch: %s", hipGetErrorString(e));
  if ((e = mark(2)) != hipSuccess) return fail(RNN_ERR_HIP, cell, "event record: %s", hipGetErrorString(e));
  // 3. recurrent steps
  if (nchunks > 0) {
    if (pers) {
      PersistentIO io{ih, ic, const_cast<char*>(Y), const_cast<char*>(Yh), const_cast<char*>(Yc), status};
      if ((e = launch_step_persistent(a, p, io, s)) != hipSuccess)
        return fail(RNN_ERR_HIP, cell, "persistent step launch: %s", hipGetErrorString(e));
    } else {
      // batches above eight: the product of each step on the matrix cores
      const bool mfma = mfma_step_supported(p);
      if (p.f32_split_step && (e = launch_split_r(R, rsplit, int64_t(p.D) * p.G * p.H * p.H, s)) != hipSuccess)
        return fail(RNN_ERR_HIP, cell, "R split launch: %s", hipGetErrorString(e));
      bool done = false;
      if (p.pers_mfma) {
        e = launch_step_mfma_persistent(a, p, flags, status, s);
        // not supported (R's alignment, epilogue planes) or not every tile
        // resident at once on this device: one launch per step instead
        if (e == hipErrorCooperativeLaunchTooLarge) (void)hipGetLastError();
        if (e != hipSuccess && e != hipErrorNotSupported && e != hipErrorCooperativeLaunchTooLarge)
          return fail(RNN_ERR_HIP, cell, "persistent matrix-core step launch: %s", hipGetErrorString(e));
        done = e == hipSuccess;
      }
      // Chunks after the first: with overlap, each projection runs on the
      // side stream one chunk ahead of the steps (chunk c+1's projection
      // while chunk c steps), each chunk's steps wait for their projection,
      // and a projection waits for the steps of the chunk that last used its
      // slot; without, each projection is enqueued on the caller's stream
      // right before its chunk's first step.
      ChunkEvents ev;
      hipStream_t side = nullptr;
      const bool overlap = !done && nchunks > 1 && chunk_overlap;
      if (overlap) {
        if ((e = ev.create()) != hipSuccess || (e = side_stream(&side)) != hipSuccess)
          return fail(RNN_ERR_HIP, cell, "chunk streams: %s", hipGetErrorString(e));
        // the side stream starts after everything enqueued so far on the
        // caller's stream (an earlier call may still read the ring)
        if ((e = hipEventRecord(ev.ev[0], s)) != hipSuccess || (e = hipStreamWaitEvent(side, ev.ev[0], 0)) != hipSuccess)
          return fail(RNN_ERR_HIP, cell, "chunk fork: %s", hipGetErrorString(e));
      }
      auto project_on = [&](int64_t c, hipStream_t st) -> hipError_t {
        ProjArgs q = pa;
        q.s0 = c * tc;
        q.M = std::min<int64_t>(tc, p.steps - q.s0) * p.B;
        q.xw = static_cast<float*>(xw_scratch) + (c & 1) * int64_t(p.D) * pa.out_dstride;
        SetupArgs none{};
        return launch_projection(q, none, p.desc.dtype, st);
      };
      if (overlap) {
        if ((e = project_on(1, side)) != hipSuccess || (e = hipEventRecord(ev.ev[1 + 1], side)) != hipSuccess)
          return fail(RNN_ERR_HIP, cell, "projection launch (chunk 1): %s", hipGetErrorString(e));
      }
      for (int64_t c = 0; !done && c < nchunks; ++c) {
        if (c > 0) {
          if (overlap) e = hipStreamWaitEvent(s, ev.ev[1 + (c & 1)], 0);
          else e = project_on(c, s);
          if (e != hipSuccess)
            return fail(RNN_ERR_HIP, cell, "projection (chunk %lld): %s", (long long)c, hipGetErrorString(e));
        }
        const int64_t last = std::min<int64_t>((c + 1) * tc, p.steps);
        for (int64_t step = c * tc; step < last; ++step)
          if ((e = mfma ? launch_step_mfma(a, p, int(step), s) : launch_step_generic(a, int(step), s)) != hipSuccess)
            return fail(RNN_ERR_HIP, cell, "step %lld launch: %s", (long long)step, hipGetErrorString(e));
        if (overlap && c + 2 < nchunks) {
          // chunk c+2 reuses chunk c's slot: after chunk c's steps
          if ((e = hipEventRecord(ev.ev[3 + (c & 1)], s)) != hipSuccess ||
              (e = hipStreamWaitEvent(side, ev.ev[3 + (c & 1)], 0)) != hipSuccess ||
              (e = project_on(c + 2, side)) != hipSuccess || (e = hipEventRecord(ev.ev[1 + (c & 1)], side)) != hipSuccess)
            return fail(RNN_ERR_HIP, cell, "projection launch (chunk %lld): %s", (long long)(c + 2),
                        hipGetErrorString(e));
        }
      }
    }
  }
  if ((e = mark(3)) != hipSuccess) return fail(RNN_ERR_HIP, cell, "event record: %s", hipGetErrorString(e));
  // 4. outputs: written by the steps and the state setup (no pass of their own)
  if ((e = mark(4)) != hipSuccess) return fail(RNN_ERR_HIP, cell, "event record: %s", hipGetErrorString(e));
  return RNN_OK;
}

}  // namespace

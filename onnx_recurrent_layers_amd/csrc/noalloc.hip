// noalloc.hip -- rnn_encode_noalloc: one layer with the library's own scratch,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The projection scratch and the state scratch of rnn_encode come from one
// fixed device array, `scratch`, of RNN_NOALLOC_SCRATCH_BYTES.  Every device
// the library runs on holds its own copy from module load until the process
// ends.  In host code the array's name is a host-side stand-in, not a device
// address: the entry point asks the runtime for the device address once per
// device (hipGetSymbolAddress, with that device current) and passes only that
// address on.  Nothing is allocated and nothing is cleared here: every
// scratch value a result of the layer depends on is written earlier in the
// same call (the projection fills the projection scratch, the state setup
// initialises the state, its exchange words, flags and status words), so the
// contents a previous call left behind never matter.  Calls that overlap on
// one device share the array and race: a caller serialises them (one stream,
// or an event between them).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "plan.h"

namespace rnnhip {

static __device__ __align__(256) unsigned char scratch[RNN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

}  // namespace rnnhip

using namespace rnnhip;

extern "C" int rnn_encode_noalloc(const rnn_problem* problem, const rnn_operands* operands, void* stream) {
  if (!problem) return set_error(RNN_ERR_ARG, -1, "problem: NULL");
  const int cell = reinterpret_cast<const Problem*>(problem)->desc.cell;
  size_t xw = 0, st = 0;
  if (rnn_scratch_size(problem, &xw, &st) != RNN_OK) return RNN_ERR_ARG;
  const size_t need = align256(xw) + align256(st);
  if (need > size_t(RNN_NOALLOC_SCRATCH_BYTES)) {
    char msg[160];
    snprintf(msg, sizeof msg, "rnn_encode_noalloc: the layer needs %zu bytes of scratch, above the %zu of the library's "
             "fixed scratch (use rnn_encode with caller scratch)", need, size_t(RNN_NOALLOC_SCRATCH_BYTES));
    return set_error(RNN_ERR_UNSUPPORTED, cell, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(RNN_ERR_HIP, cell, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(RNN_ERR_UNSUPPORTED, cell, "rnn_encode_noalloc: device index");
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        char msg[160];
        snprintf(msg, sizeof msg, "rnn_encode_noalloc: device address of the fixed scratch: %s",
                 hipGetErrorString(e));
        return set_error(RNN_ERR_HIP, cell, msg);
      }
      g_ptr[dev] = p;
    }
    base = g_ptr[dev];
  }
  char* b = static_cast<char*>(base);
  return encode_layer(problem, operands, xw ? b : nullptr, b + align256(xw), stream);
}

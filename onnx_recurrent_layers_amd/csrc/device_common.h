// device_common.h -- device helpers shared by the kernels: element loads,
// f16 rounding, the ONNX activations and clip.  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "plan.h"

// Address-space casts for the loads that write LDS directly.
#define RNN_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define RNN_GLOBAL_PTR(p) ((__attribute__((address_space(1))) void*)(const_cast<float*>(p)))

namespace rnnhip {

typedef _Float16 half_t;

// Widen one stored element (f32, or f16 which widens exactly) to f32.
template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return static_cast<float>(p[i]);
}

// Round an f32 value to the tensor type: f16 rounds to nearest even (the
// hardware conversion under the default round-to-nearest-even mode).
template <typename T>
__device__ __forceinline__ T to_elem(float v) {
  return static_cast<T>(v);
}

// clip: clamp to [-c, c] when c > 0.  Compare-and-select so that NaN passes
// (fminf/fmaxf would turn it into a bound).
__device__ __forceinline__ float clipf(float x, float c) {
  if (c > 0.f) {
    x = x < -c ? -c : x;
    x = x > c ? c : x;
  }
  return x;
}

// Logistic sigmoid 1/(1+e^-x) from the hardware exponential (v_exp_f32) and
// reciprocal; relative error a few ulp, saturating to 0 and 1, NaN passes.
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// tanh(x) = 1 - 2/(e^(2x)+1): absolute error a few 1e-8, exact limits +-1, NaN passes.
__device__ __forceinline__ float tanh_f(float x) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(__expf(2.f * x) + 1.f);
}

// The eleven ONNX activations in f32 (alpha, beta resolved by the caller),
// one function per kind, and the same chosen at run time.
template <int K>
__device__ __forceinline__ float activate_k(float a, float b, float x) {
  if constexpr (K == RNN_ACT_RELU) return x < 0.f ? 0.f : x;
  else if constexpr (K == RNN_ACT_TANH) return tanh_f(x);
  else if constexpr (K == RNN_ACT_SIGMOID) return sigmoid_f(x);
  else if constexpr (K == RNN_ACT_AFFINE) return a * x + b;
  else if constexpr (K == RNN_ACT_LEAKY_RELU) return x >= 0.f ? x : a * x;
  else if constexpr (K == RNN_ACT_THRESHOLDED_RELU) return x > a ? x : 0.f;
  else if constexpr (K == RNN_ACT_SCALED_TANH) return a * tanh_f(b * x);
  else if constexpr (K == RNN_ACT_HARD_SIGMOID) {
    float v = a * x + b;
    v = v < 0.f ? 0.f : v;
    return v > 1.f ? 1.f : v;
  } else if constexpr (K == RNN_ACT_ELU) return x >= 0.f ? x : a * expm1f(x);
  else if constexpr (K == RNN_ACT_SOFTSIGN) return x / (1.f + fabsf(x));
  else if constexpr (K == RNN_ACT_SOFTPLUS) return (x > 0.f ? x : 0.f) + log1pf(expf(-fabsf(x)));  // log(1+e^x), overflow-free
  else return __builtin_nanf("");
}

__device__ __forceinline__ float activate(int kind, float a, float b, float x) {
  switch (kind) {
    case RNN_ACT_RELU: return activate_k<RNN_ACT_RELU>(a, b, x);
    case RNN_ACT_TANH: return activate_k<RNN_ACT_TANH>(a, b, x);
    case RNN_ACT_SIGMOID: return activate_k<RNN_ACT_SIGMOID>(a, b, x);
    case RNN_ACT_AFFINE: return activate_k<RNN_ACT_AFFINE>(a, b, x);
    case RNN_ACT_LEAKY_RELU: return activate_k<RNN_ACT_LEAKY_RELU>(a, b, x);
    case RNN_ACT_THRESHOLDED_RELU: return activate_k<RNN_ACT_THRESHOLDED_RELU>(a, b, x);
    case RNN_ACT_SCALED_TANH: return activate_k<RNN_ACT_SCALED_TANH>(a, b, x);
    case RNN_ACT_HARD_SIGMOID: return activate_k<RNN_ACT_HARD_SIGMOID>(a, b, x);
    case RNN_ACT_ELU: return activate_k<RNN_ACT_ELU>(a, b, x);
    case RNN_ACT_SOFTSIGN: return activate_k<RNN_ACT_SOFTSIGN>(a, b, x);
    case RNN_ACT_SOFTPLUS: return activate_k<RNN_ACT_SOFTPLUS>(a, b, x);
    default: return __builtin_nanf("");
  }
}

__device__ __forceinline__ float activate(const Act& a, float x) { return activate(a.kind, a.alpha, a.beta, x); }

// Step-to-time map of one (direction, batch row): the row runs its first L
// steps; a reverse direction starts at L-1.
__device__ __forceinline__ int row_length(const int32_t* lens, int b, int S, int steps) {
  int L = lens ? lens[b] : S;
  L = L < 0 ? 0 : L;
  L = L > S ? S : L;
  return L < steps ? L : steps;
}

// f32 -> two bf16 values hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in
// f32), as bit patterns; rounding to nearest even.
__device__ __forceinline__ void split_bf16_bits(float x, unsigned short& hi, unsigned short& lo) {
  const __bf16 h = __bf16(x);
  hi = __builtin_bit_cast(unsigned short, h);
  lo = __builtin_bit_cast(unsigned short, __bf16(x - float(h)));
}

// The same split into f16 halves: hi = f16(x), lo = f16(x - hi).
__device__ __forceinline__ void split_f16_bits(float x, unsigned short& hi, unsigned short& lo) {
  const _Float16 h = _Float16(x);
  hi = __builtin_bit_cast(unsigned short, h);
  lo = __builtin_bit_cast(unsigned short, _Float16(x - float(h)));
}

// kind 1: f16 halves; kind 2: bf16 halves.
__device__ __forceinline__ void split_bits(int kind, float x, unsigned short& hi, unsigned short& lo) {
  if (kind == 1) split_f16_bits(x, hi, lo);
  else split_bf16_bits(x, hi, lo);
}

// Index of output Y at time t, direction d, batch row b, unit j:
// layout 0 [S][D][B][H], layout 1 [B][S][D][H].
__device__ __forceinline__ int64_t y_index(int layout, int S, int D, int B, int H, int t, int d, int b, int j) {
  return layout == 0 ? ((int64_t(t) * D + d) * B + b) * H + j : ((int64_t(b) * S + t) * D + d) * H + j;
}

// Element offset in X of row m = t*B + b of the projection's A operand:
// layout 0 m*K, layout 1 (b*S + t)*K.  A row in two pieces (X is the Y
// [S,2,B,H'] of a bidirectional layout-0 layer, K = 2H'): it starts at
// Y[t,0,b,0] = (2tB + b)*H' and its second half at Y[t,1,b,0], B*H'
// elements after the first; x_col maps element k of the row to its offset
// from the row start.
__device__ __forceinline__ int64_t x_row_off(const ProjArgs& a, int64_t m) {
  const int64_t t = m / a.B, b = m - t * a.B;
  if (a.layout == 1) return (b * a.S + t) * a.K;
  if (a.xjump != 0) return (2 * t * a.B + b) * a.xkh;
  return m * a.K;
}
__device__ __forceinline__ int64_t x_col(const ProjArgs& a, int64_t k) { return k + (k >= a.xkh ? a.xjump : 0); }

// Element offset in X of the row that output row m (step s0 + m / B, batch
// row m % B) of direction d of a projection launch reads: time s forward,
// len_b - 1 - s backward while the row runs, time s after it has ended (never
// read).
__device__ __forceinline__ int64_t x_row_step(const ProjArgs& a, int d, int64_t m) {
  const int64_t sl = m / a.B, b = m - sl * a.B;
  const int64_t s = a.s0 + sl;
  int64_t t = s;
  if (a.rev[d]) {
    int64_t L = a.lens ? a.lens[b] : a.S;
    L = L < 0 ? 0 : (L > a.S ? a.S : L);
    L = L < a.steps ? L : a.steps;
    if (s < L) t = L - 1 - s;
  }
  return x_row_off(a, t * a.B + b);
}

// The [B][G*H] slab of the projection that step s of direction d reads.
__device__ __forceinline__ const float* xw_slab(const StepArgs& a, int d, int s) {
  const int q = s / a.xw_tc;
  return a.xw + ((int64_t(q & 1) * a.D + d) * a.xw_tc + (s - q * a.xw_tc)) * int64_t(a.B) * (a.G * a.H);
}

// Direction d's first slab when the projection scratch is one slot of every
// step (the persistent engines): step s's slab follows it at s * B * G * H,
// an address with no division in it.
__device__ __forceinline__ const float* xw_dir(const StepArgs& a, int d) {
  return a.xw + int64_t(d) * a.xw_tc * int64_t(a.B) * (a.G * a.H);
}

// Index of a state tensor (initial_h, initial_c, Y_h, Y_c) for direction d,
// batch row b, unit j: layout 0 [D][B][H], layout 1 [B][D][H].
__device__ __forceinline__ int64_t state_index(int layout, int D, int B, int H, int d, int b, int j) {
  return layout == 0 ? (int64_t(d) * B + b) * H + j : (int64_t(b) * D + d) * H + j;
}

// Stage 2 ("Recurrent layers" page, "How a layer runs", item 2): the first
// hidden and cell state from initial_h / initial_c or zeros, for one share of
// the (d, b, j) elements (`part` of `parts` workgroups): slot 0 of the
// per-step state, the cell state, and for the persistent engine the tagged
// exchange words of step 0 with the other slots marked empty.  For the
// per-step engine it also writes the outputs that no step writes ("Semantics"
// rules): Y is zero past each row's length, a row of length 0 has zero final
// states, and Seq = 0 gives the initial states as final states.
template <typename T>
__device__ __forceinline__ void setup_state(const SetupArgs& a, int part, int parts) {
  const int64_t DBH = int64_t(a.D) * a.B * a.H;
  for (int64_t i = part * int64_t(blockDim.x) + threadIdx.x; i < DBH; i += int64_t(parts) * blockDim.x) {
    const int64_t j = i % a.H;
    const int64_t b = (i / a.H) % a.B;
    const int64_t d = i / (int64_t(a.H) * a.B);
    // ONNX state layout: 0 -> [D,B,H]; 1 -> [B,D,H]
    const int64_t src = a.layout == 0 ? i : (b * a.D + d) * a.H + j;
    const float h0 = a.init_h ? ld(static_cast<const T*>(a.init_h), src) : 0.f;
    const float c0 = a.init_c ? ld(static_cast<const T*>(a.init_c), src) : 0.f;
    if (a.hbuf) a.hbuf[i] = h0;
    if (a.hsplit) split_bits(a.split_kind, h0, a.hsplit[i], a.hsplit[DBH + i]);
    if (a.cell_state) a.cell_state[i] = c0;
    if (a.xch) {
      // word = (tag << 32) | value bits; slot 0 carries step 0, slot 1 no step yet.
      a.xch[i] = (0ull << 32) | __float_as_uint(h0);
      a.xch[DBH + i] = 0xffffffffull << 32;
    }
    if (a.xch2) {
      a.xch2[i] = 0xffffffffull << 32;
      a.xch2[DBH + i] = 0xffffffffull << 32;
    }
    if (a.Y || a.Y_h || a.Y_c) {
      const int L = a.S > 0 ? row_length(a.lens, int(b), a.S, a.steps) : 0;
      if (a.Y)
        for (int t = L; t < a.S; ++t)
          static_cast<T*>(a.Y)[y_index(a.layout, a.S, a.D, a.B, a.H, t, int(d), int(b), int(j))] = to_elem<T>(0.f);
      if (L == 0) {
        if (a.Y_h) static_cast<T*>(a.Y_h)[src] = to_elem<T>(a.S == 0 ? h0 : 0.f);
        if (a.Y_c) static_cast<T*>(a.Y_c)[src] = to_elem<T>(a.S == 0 ? c0 : 0.f);
      }
    }
  }
  // status word, arrival tickets and residency decision of a persistent launch
  if (a.status && part == 0 && threadIdx.x < 3) a.status[threadIdx.x] = 0;
  for (int i = part * int(blockDim.x) + int(threadIdx.x); i < a.nflags; i += parts * int(blockDim.x)) a.flags[i] = 0;
}

}  // namespace rnnhip

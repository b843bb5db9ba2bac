// cells.h -- the gate arithmetic of one hidden unit for one batch row, in the
// order the "Recurrent layers" page fixes ("Arithmetic and determinism"):
// pre = ((xw + rec) + Wb) + Rb, then the peephole terms (i and f with the
// previous cell state, o with the new one), then clip, then the activation,
// then c = f*c + i*c~, h = o*h_act(c); GRU h = (1 - z)*h~ + z*h.  input_forget
// and linear_before_reset follow the page's "Semantics" list.
//
// DEF = true compiles the ONNX default activations (LSTM Sigmoid/Tanh/Tanh,
// GRU Sigmoid/Tanh, RNN Tanh) without the eleven-way switch: the page found
// that carrying every activation inline costs step time through code size
// alone ("What a step costs"), so the common case gets its own kernel.
// Internal.
#pragma once

#include "device_common.h"

namespace rnnhip {

// Outputs of one (direction d, batch row b, unit j) after a step at time t:
// Y, and after the row's last step (`last`) the final states Y_h and Y_c,
// rounded to the tensor type.  Null outputs are skipped.
template <typename T>
__device__ __forceinline__ void store_outputs(const StepArgs& a, int d, int b, int j, int t, bool last, float h,
                                              float c) {
  if (a.Y) static_cast<T*>(a.Y)[y_index(a.layout, a.S, a.D, a.B, a.H, t, d, b, j)] = to_elem<T>(h);
  if (last) {
    const int64_t si = state_index(a.layout, a.D, a.B, a.H, d, b, j);
    if (a.Y_h) static_cast<T*>(a.Y_h)[si] = to_elem<T>(h);
    if (a.Y_c) static_cast<T*>(a.Y_c)[si] = to_elem<T>(c);
  }
}

template <bool DEF>
__device__ __forceinline__ float act_sig(const Act& a, float x) {
  if constexpr (DEF) return sigmoid_f(x);
  else return activate(a, x);
}

template <bool DEF>
__device__ __forceinline__ float act_tanh(const Act& a, float x) {
  if constexpr (DEF) return tanh_f(x);
  else return activate(a, x);
}

// pre-activation sum in the page's order; absent biases add nothing.
__device__ __forceinline__ float pre_sum(float xw, float rec, float wb, float rb) {
  return ((xw + rec) + wb) + rb;
}

// LSTM.  pre[g] for g = i, o, f, c (already summed); peep = P_i, P_o, P_f or
// null; acts = f, g, h slots of this direction.
template <bool DEF = false>
__device__ __forceinline__ void lstm_unit(const float pre[4], const float* peep, float c_prev, float clip,
                                          int input_forget, const Act* acts, float* h_out, float* c_out) {
  float pi = pre[0], pf = pre[2], pc = pre[3];
  if (peep) {
    pi = pi + peep[0] * c_prev;
    pf = pf + peep[2] * c_prev;
  }
  pi = clipf(pi, clip);
  pf = clipf(pf, clip);
  pc = clipf(pc, clip);
  const float ig = act_sig<DEF>(acts[0], pi);
  const float fg = input_forget ? 1.f - ig : act_sig<DEF>(acts[0], pf);
  const float ct = act_tanh<DEF>(acts[1], pc);
  const float c = fg * c_prev + ig * ct;
  float po = pre[1];
  if (peep) po = po + peep[1] * c;
  po = clipf(po, clip);
  const float og = act_sig<DEF>(acts[0], po);
  *c_out = c;
  *h_out = og * act_tanh<DEF>(acts[2], c);
}

// GRU update-gate and reset-gate activations.
template <bool DEF = false>
__device__ __forceinline__ float gru_gate(float pre, float clip, const Act* acts) {
  return act_sig<DEF>(acts[0], clipf(pre, clip));
}

// GRU candidate and new state.  `ph` is the candidate pre-activation already
// formed in the right order for linear_before_reset (see the step kernels).
template <bool DEF = false>
__device__ __forceinline__ float gru_unit(float z, float ph, float h_prev, float clip, const Act* acts) {
  const float hh = act_tanh<DEF>(acts[1], clipf(ph, clip));
  return (1.f - z) * hh + z * h_prev;
}

// Plain RNN.
template <bool DEF = false>
__device__ __forceinline__ float rnn_unit(float pre, float clip, const Act* acts) {
  return act_tanh<DEF>(acts[0], clipf(pre, clip));
}

}  // namespace rnnhip

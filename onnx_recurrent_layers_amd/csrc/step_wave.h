// step_wave.h -- one wave's share of a recurrent step: the recurrent product
// rec = R[d] . h_prev of one hidden unit for up to kRows batch rows, fused with
// the gate arithmetic of cells.h ("Recurrent layers" page, "How a layer runs",
// item 3).  Used by the per-step kernel (one wave per unit and row block).
// Internal.
#pragma once

#include "cells.h"

namespace rnnhip {

constexpr int kRows = 8;  // batch rows per wave

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Unit j, batch rows b0 .. b0+kRows-1, direction d, step s; GRU with
// linear_before_reset = 0 in two phases (0: z and r*h, 1: the candidate).
// Needs all 64 lanes of the wave.
template <typename T>
__device__ __forceinline__ void step_wave(const StepArgs& a, int s, int phase, int j, int b0, int d, int lane) {
  const int H = a.H, B = a.B, G = a.G;

  int L[kRows];
  bool on[kRows];
  bool any = false;
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    const int b = b0 + u;
    L[u] = b < B ? row_length(a.lens, b, a.S, a.steps) : 0;
    on[u] = s < L[u];
    any |= on[u];
  }
  if (!any) return;

  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  const float* hprev = a.hbuf + int64_t(s & 1) * DBH + dBH;
  float* hnext = a.hbuf + int64_t((s + 1) & 1) * DBH + dBH;
  const T* Rd = static_cast<const T*>(a.R) + int64_t(d) * G * H * H;
  const bool gru_two_phase = a.cell == RNN_CELL_GRU && !a.lbr;

  // gate rows of this launch
  int g_lo = 0, g_hi = G;
  if (gru_two_phase) {
    g_lo = phase == 0 ? 0 : 2;
    g_hi = phase == 0 ? 2 : 3;
  }
  const float* src = (gru_two_phase && phase == 1) ? a.rhbuf + dBH : hprev;

  float acc[4][kRows];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int u = 0; u < kRows; ++u) acc[g][u] = 0.f;

#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g < g_lo || g >= g_hi) continue;
    if (a.cell == RNN_CELL_LSTM && a.input_forget && g == 2) continue;  // f rows unused
    const T* row = Rd + int64_t(g * H + j) * H;
    for (int k = lane; k < H; k += 64) {
      const float r = ld(row, k);
#pragma unroll
      for (int u = 0; u < kRows; ++u)
        if (on[u]) acc[g][u] += r * src[int64_t(b0 + u) * H + k];
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) acc[g][u] = wave_sum(acc[g][u]);
  }

  // lane u < 8 finishes batch row b0 + u
  if (lane >= kRows) return;
  float rec[4];
  int Lr = 0;
  bool active = false;
#pragma unroll
  for (int g = 0; g < 4; ++g) rec[g] = acc[g][0];
  Lr = L[0];
  active = on[0];
#pragma unroll
  for (int u = 1; u < kRows; ++u)
    if (lane == u) {
#pragma unroll
      for (int g = 0; g < 4; ++g) rec[g] = acc[g][u];
      Lr = L[u];
      active = on[u];
    }
  if (!active) return;
  const int b = b0 + lane;
  const int t = a.dir_reverse[d] ? (Lr - 1 - s) : s;
  const int GH = G * H;
  const float* xw = xw_slab(a, d, s) + int64_t(b) * GH;
  const T* bias = a.bias ? static_cast<const T*>(a.bias) + int64_t(d) * 2 * GH : nullptr;
  const Act* acts = a.act + d * a.slots;
  const int64_t sidx = int64_t(b) * H + j;  // within direction d

  auto pre = [&](int g) {
    const int n = g * H + j;
    const float wb = bias ? ld(bias, n) : 0.f;
    const float rb = bias ? ld(bias, GH + n) : 0.f;
    return pre_sum(xw[n], rec[g], wb, rb);
  };

  if (a.cell == RNN_CELL_LSTM) {
    float p4[4];
    p4[0] = pre(0);
    p4[1] = pre(1);
    p4[2] = a.input_forget ? 0.f : pre(2);
    p4[3] = pre(3);
    // (two calls, each with a fixed peephole pointer, so that the array stays
    // in registers instead of scratch memory)
    float peep[3] = {0.f, 0.f, 0.f};
    if (a.P) {
      const T* P = static_cast<const T*>(a.P) + int64_t(d) * 3 * H;
      peep[0] = ld(P, j);
      peep[1] = ld(P, H + j);
      peep[2] = ld(P, 2 * H + j);
    }
    float* cst = a.cell_state + dBH + sidx;
    float h, c;
    if (a.P)
      lstm_unit(p4, peep, *cst, a.clip, a.input_forget, acts, &h, &c);
    else
      lstm_unit(p4, nullptr, *cst, a.clip, a.input_forget, acts, &h, &c);
    *cst = c;
    hnext[sidx] = h;
    store_outputs<T>(a, d, b, j, t, s == Lr - 1, h, c);
  } else if (a.cell == RNN_CELL_GRU) {
    if (!gru_two_phase) {
      // linear_before_reset = 1: h~ = g(xw_h + r * (rec_h + Rb_h) + Wb_h)
      const float z = gru_gate(pre(0), a.clip, acts);
      const float r = gru_gate(pre(1), a.clip, acts);
      const int n = 2 * H + j;
      const float wb = bias ? ld(bias, n) : 0.f;
      const float rb = bias ? ld(bias, GH + n) : 0.f;
      const float ph = (xw[n] + r * (rec[2] + rb)) + wb;
      const float h = gru_unit(z, ph, hprev[sidx], a.clip, acts);
      hnext[sidx] = h;
      store_outputs<T>(a, d, b, j, t, s == Lr - 1, h, 0.f);
    } else if (phase == 0) {
      const float z = gru_gate(pre(0), a.clip, acts);
      const float r = gru_gate(pre(1), a.clip, acts);
      a.zbuf[dBH + sidx] = z;
      a.rhbuf[dBH + sidx] = r * hprev[sidx];
    } else {
      // linear_before_reset = 0: h~ = g(((xw_h + R_h.(r*h)) + Wb_h) + Rb_h)
      const float z = a.zbuf[dBH + sidx];
      const float h = gru_unit(z, pre(2), hprev[sidx], a.clip, acts);
      hnext[sidx] = h;
      store_outputs<T>(a, d, b, j, t, s == Lr - 1, h, 0.f);
    }
  } else {
    const float h = rnn_unit(pre(0), a.clip, acts);
    hnext[sidx] = h;
    store_outputs<T>(a, d, b, j, t, s == Lr - 1, h, 0.f);
  }
}

}  // namespace rnnhip

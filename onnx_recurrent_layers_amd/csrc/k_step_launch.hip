// k_step_launch.hip -- stage 3 of a layer as one kernel launch per step
// ("Recurrent layers" page, "How a layer runs", item 3): the recurrent product
// rec = R[d] . h_prev of every active (direction, batch row), fused with the
// gate arithmetic of cells.h.  A GRU with linear_before_reset = 0 takes two
// launches per step, because its candidate product needs r*h of every unit.
//
// One wave64 per (direction, hidden unit, block of 8 batch rows) covers all
// gate rows of that unit, so the gate arithmetic stays in the wave.  Lanes walk
// k = lane, lane+64, ... in increasing order and the 64 partial sums are
// combined by a fixed xor butterfly: the summation order depends only on the
// shapes, never on scheduling (no atomics), so runs are bit-identical.
// Rows whose sequence has ended are skipped: their h stays in the state slot
// of their last step, and nothing reads it again.  Each step writes Y (and,
// after a row's last step, Y_h / Y_c) itself.
#include "cells.h"

namespace rnnhip {

constexpr int kRows = 8;  // batch rows per wave

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <typename T>
__global__ __launch_bounds__(64) void step_launch_kernel(StepArgs a, int s, int phase) {
  const int j = blockIdx.x;
  const int b0 = blockIdx.y * kRows;
  const int d = blockIdx.z;
  const int lane = threadIdx.x;
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
  const float* xw = a.xw + ((int64_t(d) * a.S + t) * B + b) * GH;
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
    float peep[3];
    const float* pp = nullptr;
    if (a.P) {
      const T* P = static_cast<const T*>(a.P) + int64_t(d) * 3 * H;
      peep[0] = ld(P, j);
      peep[1] = ld(P, H + j);
      peep[2] = ld(P, 2 * H + j);
      pp = peep;
    }
    float* cst = a.cell_state + dBH + sidx;
    float h, c;
    lstm_unit(p4, pp, *cst, a.clip, a.input_forget, acts, &h, &c);
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

int step_generic_launches_per_step(const StepArgs& a) { return (a.cell == RNN_CELL_GRU && !a.lbr) ? 2 : 1; }

hipError_t launch_step_generic(const StepArgs& a, int step, hipStream_t s) {
  const dim3 grid(unsigned(a.H), unsigned((a.B + kRows - 1) / kRows), unsigned(a.D));
  if (grid.y > 65535) return hipErrorInvalidValue;
  const int phases = step_generic_launches_per_step(a);
  for (int ph = 0; ph < phases; ++ph) {
    if (a.dtype == RNN_DTYPE_F32)
      hipLaunchKernelGGL(step_launch_kernel<float>, grid, dim3(64), 0, s, a, step, ph);
    else
      hipLaunchKernelGGL(step_launch_kernel<half_t>, grid, dim3(64), 0, s, a, step, ph);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rnnhip

// step_mfma.h -- what the two matrix-core step kernels share: the launch
// arguments of one step and the fused gate arithmetic that finishes a product
// tile (stage 3 of a layer, "Recurrent layers" page, "How a layer runs",
// item 3).  Internal.
#pragma once

#include "cells.h"

namespace rnnhip {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMThreads = 256;
constexpr int kMaxNC = 128;      // gate rows per tile (Gp * UJ)

struct MfmaStepArgs {
  StepArgs a;
  int UJ;           // units per tile (multiple of 16)
  int Gp;           // gate blocks computed in this phase
  int gate_of[4];   // gate block index of each computed block
  int phase;        // GRU linear_before_reset = 0: 0 = z and r, 1 = candidate; else 0
  int step;
};

// Gate block of computed block gi, as selects over the argument words held in
// scalar registers (an indexed read of the argument array would be a memory
// load per lane, waited for on the spot).
__device__ __forceinline__ int gate_block(const MfmaStepArgs& m, int gi) {
  const int g0 = __builtin_amdgcn_readfirstlane(m.gate_of[0]), g1 = __builtin_amdgcn_readfirstlane(m.gate_of[1]);
  const int g2 = __builtin_amdgcn_readfirstlane(m.gate_of[2]), g3 = __builtin_amdgcn_readfirstlane(m.gate_of[3]);
  return gi == 0 ? g0 : gi == 1 ? g1 : gi == 2 ? g2 : g3;
}

// Gate arithmetic of a finished product tile rec[BM][Gp*UJ] (row stride
// kMaxNC + 1): one thread per (batch row, unit), in the order of cells.h.
template <typename T, int BM>
__device__ __forceinline__ void mfma_epilogue(const MfmaStepArgs& m, const float* rec, const int* len_s, int b0,
                                              int j0, int d) {
  const StepArgs& a = m.a;
  const int H = a.H, B = a.B, G = a.G;
  const int s = m.step;
  const int tid = threadIdx.x;
  const int UJ = m.UJ;
  const int64_t DBH = int64_t(a.D) * B * H;
  const int64_t dBH = int64_t(d) * B * H;
  constexpr int LDR = kMaxNC + 1;
  const int GH = G * H;
  const T* bias = a.bias ? static_cast<const T*>(a.bias) + int64_t(d) * 2 * GH : nullptr;
  const Act* acts = a.act + d * a.slots;
  const float* hprev = a.hbuf + int64_t(s & 1) * DBH + dBH;
  float* hnext = a.hbuf + int64_t((s + 1) & 1) * DBH + dBH;
  for (int e = tid; e < BM * UJ; e += kMThreads) {
    const int r = e / UJ, u = e - r * UJ;
    const int b = b0 + r, j = j0 + u;
    if (b >= B || j >= H) continue;
    const int L = len_s[r];
    if (s >= L) continue;
    const int t = a.dir_reverse[d] ? (L - 1 - s) : s;
    const float* xw = xw_slab(a, d, m.step) + int64_t(b) * GH;
    const int64_t sidx = int64_t(b) * H + j;
    const float* rrow = rec + r * LDR;
    auto pre = [&](int gi, int g) {
      const int n = g * H + j;
      const float wb = bias ? ld(bias, n) : 0.f;
      const float rbv = bias ? ld(bias, GH + n) : 0.f;
      return pre_sum(xw[n], rrow[gi * UJ + u], wb, rbv);
    };
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
      store_outputs<T>(a, d, b, j, t, s == L - 1, h, c);
    } else if (a.cell == RNN_CELL_GRU) {
      if (a.lbr) {
        // linear_before_reset = 1: h~ = g(xw_h + r * (rec_h + Rb_h) + Wb_h)
        const float z = gru_gate(pre(0, 0), a.clip, acts);
        const float rg = gru_gate(pre(1, 1), a.clip, acts);
        const int n = 2 * H + j;
        const float wb = bias ? ld(bias, n) : 0.f;
        const float rbv = bias ? ld(bias, GH + n) : 0.f;
        const float ph = (xw[n] + rg * (rrow[2 * UJ + u] + rbv)) + wb;
        const float h = gru_unit(z, ph, hprev[sidx], a.clip, acts);
        hnext[sidx] = h;
        store_outputs<T>(a, d, b, j, t, s == L - 1, h, 0.f);
      } else if (m.phase == 0) {
        const float z = gru_gate(pre(0, 0), a.clip, acts);
        const float rg = gru_gate(pre(1, 1), a.clip, acts);
        a.zbuf[dBH + sidx] = z;
        a.rhbuf[dBH + sidx] = rg * hprev[sidx];
      } else {
        // linear_before_reset = 0: h~ = g(((xw_h + R_h.(r*h)) + Wb_h) + Rb_h)
        const int n = 2 * H + j;
        const float wb = bias ? ld(bias, n) : 0.f;
        const float rbv = bias ? ld(bias, GH + n) : 0.f;
        const float ph = pre_sum(xw[n], rrow[u], wb, rbv);
        const float h = gru_unit(a.zbuf[dBH + sidx], ph, hprev[sidx], a.clip, acts);
        hnext[sidx] = h;
        store_outputs<T>(a, d, b, j, t, s == L - 1, h, 0.f);
      }
    } else {
      const float h = rnn_unit(pre(0, 0), a.clip, acts);
      hnext[sidx] = h;
      store_outputs<T>(a, d, b, j, t, s == L - 1, h, 0.f);
    }
  }
}

// The matrix-core step whose operands go straight from global memory into
// LDS (k_step_mfma_dma.hip): usable when R rows and h rows are whole 16-byte
// segments and every byte offset fits 32 bits.  mode 0: f32 tensors on the
// f32 matrix cores; 1: f16 tensors with the default activations (split h);
// 2: f32 tensors on the bf16 matrix cores (h and R as bf16 hi/lo planes).
hipError_t launch_step_dma(const MfmaStepArgs& m, int bm, int mode, hipStream_t s);
// Every step in one launch of the same kernel body (`ph`: the
// arguments of each of the P phases of a step; `flags`: one int per
// workgroup, zeroed beforehand).  hipErrorNotSupported: the tile's epilogue
// planes do not fit; the caller then launches per step.
hipError_t launch_step_dma_persistent(const MfmaStepArgs* ph, int P, int bm, int mode, int* flags, int* status,
                                      hipStream_t s);

}  // namespace rnnhip

"""An independent brute-force evaluation of ONNX RNN / GRU / LSTM layers in
50-digit arithmetic (mpmath), for tiny layers only.

Test infrastructure: it pins the C oracle (``oracle/rnn_oracle.c``) on tiny
shapes, where 50 digits make its own rounding invisible, so the oracle's
float64 result must agree to about 1e-12 whatever order it sums in.  It is
written separately from the oracle, from the same definitions:

* "Recurrent layers" page, "Arithmetic and determinism": a gate's
  pre-activation is the input term plus the recurrent term plus Wb plus Rb,
  then the peephole terms (i and f with the previous cell state, o with the
  new one), then clip, then the activation; c = f*c + i*c~, h = o*h_act(c);
  GRU h = (1 - z)*h~ + z*h_prev;
* the same page, "Semantics": sequence lengths (a reverse row starts at its
  own last step, Y zero past the length, final states after the last step,
  zero final states for length 0, lengths above Seq act as Seq), Seq = 0,
  clip, input_forget f = 1 - i, the two GRU candidate forms;
* the ONNX operator definitions the page defers to: tensor shapes per
  layout, gate block orders (LSTM i,o,f,c; GRU z,r,h), P order (i,o,f),
  activation slots and formulas.

Every sequence (direction, batch row) is evaluated on its own, one unit at a
time, with each sum written out over its terms.
"""
from __future__ import annotations

import numpy as np
from mpmath import mp, mpf

mp.dps = 50


def act(name, alpha, beta, x):
    """The ONNX activation `name` at x, in 50-digit arithmetic."""
    a, b = mpf(alpha), mpf(beta)
    if name == "Relu":
        return x if x > 0 else mpf(0)
    if name == "Tanh":
        return mp.tanh(x)
    if name == "Sigmoid":
        return 1 / (1 + mp.exp(-x))
    if name == "Affine":
        return a * x + b
    if name == "LeakyRelu":
        return x if x >= 0 else a * x
    if name == "ThresholdedRelu":
        return x if x > a else mpf(0)
    if name == "ScaledTanh":
        return a * mp.tanh(b * x)
    if name == "HardSigmoid":
        return min(max(a * x + b, mpf(0)), mpf(1))
    if name == "Elu":
        return x if x >= 0 else a * (mp.exp(x) - 1)
    if name == "Softsign":
        return x / (1 + abs(x))
    if name == "Softplus":
        return mp.log(1 + mp.exp(x))
    raise ValueError(name)


def _m(v):
    return mpf(float(v))


def _clamp(x, clip):
    if clip is not None and clip > 0:
        c = mpf(clip)
        if x > c:
            return c
        if x < -c:
            return -c
    return x


def layer(spec, t):
    """Y, Y_h, Y_c (numpy float64, rounded from 50 digits) of one layer."""
    S, B, I, H = spec.seq, spec.batch, spec.input, spec.hidden
    D = spec.num_directions
    G = spec.gates
    lay = spec.layout
    acts = spec.activations
    nslot = {"RNN": 1, "GRU": 2, "LSTM": 3}[spec.cell]
    X, W, R = t["X"], t["W"], t["R"]
    Bias, P = t.get("B"), t.get("P")
    h0, c0, lens = t.get("initial_h"), t.get("initial_c"), t.get("sequence_lens")

    Y = np.zeros((S, D, B, H) if lay == 0 else (B, S, D, H))
    Yh = np.zeros((D, B, H) if lay == 0 else (B, D, H))
    Yc = np.zeros_like(Yh)

    def x_at(tt, b, k):
        return _m(X[tt, b, k] if lay == 0 else X[b, tt, k])

    def st(arr, d, b, j):
        if arr is None:
            return mpf(0)
        return _m(arr[d, b, j] if lay == 0 else arr[b, d, j])

    for d in range(D):
        rev = spec.direction == "reverse" or (spec.direction == "bidirectional" and d == 1)
        f_a, g_a, h_a = (acts[d * nslot + k] if k < nslot else None for k in range(3))

        def wrow(n, tt, b):    # input term of gate row n at time tt
            return mp.fsum(_m(W[d, n, k]) * x_at(tt, b, k) for k in range(I))

        def rrow(n, v):        # recurrent term of gate row n against vector v
            return mp.fsum(_m(R[d, n, k]) * v[k] for k in range(H))

        def wb(n):
            return _m(Bias[d, n]) if Bias is not None else mpf(0)

        def rb(n):
            return _m(Bias[d, G * H + n]) if Bias is not None else mpf(0)

        for b in range(B):
            h = [st(h0, d, b, j) for j in range(H)]
            c = [st(c0, d, b, j) for j in range(H)]
            if S == 0:
                for j in range(H):
                    idx = (d, b, j) if lay == 0 else (b, d, j)
                    Yh[idx] = float(h[j])
                    Yc[idx] = float(c[j])
                continue
            L = S if lens is None else max(0, min(int(lens[b]), S))
            if spec.max_length:
                L = min(L, spec.max_length)
            for s in range(L):
                tt = L - 1 - s if rev else s
                if spec.cell == "RNN":
                    nh = [act(*f_a, _clamp(wrow(j, tt, b) + rrow(j, h) + wb(j) + rb(j), spec.clip))
                          for j in range(H)]
                    nc = c
                elif spec.cell == "GRU":
                    z = [act(*f_a, _clamp(wrow(j, tt, b) + rrow(j, h) + wb(j) + rb(j), spec.clip))
                         for j in range(H)]
                    r = [act(*f_a, _clamp(wrow(H + j, tt, b) + rrow(H + j, h) + wb(H + j) + rb(H + j), spec.clip))
                         for j in range(H)]
                    nh = []
                    for j in range(H):
                        n = 2 * H + j
                        if spec.linear_before_reset:
                            pre = wrow(n, tt, b) + r[j] * (rrow(n, h) + rb(n)) + wb(n)
                        else:
                            pre = wrow(n, tt, b) + rrow(n, [r[k] * h[k] for k in range(H)]) + wb(n) + rb(n)
                        cand = act(*g_a, _clamp(pre, spec.clip))
                        nh.append((1 - z[j]) * cand + z[j] * h[j])
                    nc = c
                else:
                    nh, nc = [], []
                    for j in range(H):
                        pre = [wrow(g * H + j, tt, b) + rrow(g * H + j, h) + wb(g * H + j) + rb(g * H + j)
                               for g in range(4)]   # i, o, f, c
                        pi, po, pf = (_m(P[d, k * H + j]) if P is not None else mpf(0) for k in range(3))
                        ig = act(*f_a, _clamp(pre[0] + pi * c[j], spec.clip))
                        if spec.input_forget:
                            fg = 1 - ig
                        else:
                            fg = act(*f_a, _clamp(pre[2] + pf * c[j], spec.clip))
                        ct = act(*g_a, _clamp(pre[3], spec.clip))
                        cn = fg * c[j] + ig * ct
                        og = act(*f_a, _clamp(pre[1] + po * cn, spec.clip))
                        nc.append(cn)
                        nh.append(og * act(*h_a, cn))
                h, c = nh, nc
                for j in range(H):
                    Y[(tt, d, b, j) if lay == 0 else (b, tt, d, j)] = float(h[j])
            for j in range(H):
                idx = (d, b, j) if lay == 0 else (b, d, j)
                Yh[idx] = float(h[j]) if L > 0 else 0.0
                Yc[idx] = float(c[j]) if L > 0 else 0.0
    return {"Y": Y, "Y_h": Yh, "Y_c": Yc if spec.cell == "LSTM" else None}

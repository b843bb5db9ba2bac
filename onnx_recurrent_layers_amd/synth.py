"""Seeded synthetic layer descriptions and inputs.

This module holds no arithmetic of the recurrent layers: it only describes a
layer (cell, sizes, options, resolved activation list) and draws its input
tensors from a seeded numpy generator.  Both the HIP library's tests and the
CPU oracle receive the same arrays from here.

Draw order (float64, then cast to the tensor type with round-to-nearest-even):
X, W, R, B, P, initial_h, initial_c, sequence_lens.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import numpy as np

GATES = {"RNN": 1, "GRU": 3, "LSTM": 4}
SLOTS = {"RNN": 1, "GRU": 2, "LSTM": 3}
# ONNX default activations per cell: LSTM f,g,h; GRU f,g; RNN f.
DEFAULT_ACTS = {
    "LSTM": (("Sigmoid", 0.0, 0.0), ("Tanh", 0.0, 0.0), ("Tanh", 0.0, 0.0)),
    "GRU": (("Sigmoid", 0.0, 0.0), ("Tanh", 0.0, 0.0)),
    "RNN": (("Tanh", 0.0, 0.0),),
}
ACTIVATIONS = ("Relu", "Tanh", "Sigmoid", "Affine", "LeakyRelu", "ThresholdedRelu",
               "ScaledTanh", "HardSigmoid", "Elu", "Softsign", "Softplus")


@dataclass
class LayerSpec:
    cell: str                      # "RNN" | "GRU" | "LSTM"
    seq: int
    batch: int
    input: int
    hidden: int
    direction: str = "forward"     # "forward" | "reverse" | "bidirectional"
    layout: int = 0
    dtype: str = "f32"             # "f32" | "f16"
    clip: Optional[float] = None
    input_forget: int = 0
    linear_before_reset: int = 0
    acts: Optional[Sequence[Tuple[str, float, float]]] = None  # None: ONNX defaults
    max_length: int = 0
    # which optional inputs exist
    bias: bool = True
    peephole: bool = False
    init_h: bool = False
    init_c: bool = False
    lens: bool = False
    outputs: Tuple[str, ...] = ("Y", "Y_h", "Y_c")
    # X is the Y of a bidirectional layer of the same layout, read in place
    # (layout 0: [S, 2, B, input/2] read as [S, B, input])
    x_bidirectional_y: int = 0
    # the projection in chunks of this many steps (0: the library chooses)
    xw_chunk_steps: int = 0

    @property
    def num_directions(self) -> int:
        return 2 if self.direction == "bidirectional" else 1

    @property
    def gates(self) -> int:
        return GATES[self.cell]

    @property
    def activations(self):
        """Resolved (name, alpha, beta) list: forward slots, then reverse slots."""
        if self.acts is not None:
            acts = tuple(tuple(a) for a in self.acts)
            n = SLOTS[self.cell]
            if len(acts) == n and self.num_directions == 2:
                acts = acts + acts
            return acts
        return DEFAULT_ACTS[self.cell] * self.num_directions

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


@dataclass
class Dists:
    """Distributions: ("U", lo, hi) continuous uniform, ("N", mean, std) normal,
    ("I", lo, hi) inclusive integer uniform."""
    X: tuple = ("N", 0.0, 1.0)
    W: tuple = ("U", -0.25, 0.25)
    R: tuple = ("U", -0.25, 0.25)
    B: tuple = ("U", -0.25, 0.25)
    P: tuple = ("U", -0.1, 0.1)
    initial_h: tuple = ("N", 0.0, 0.5)
    initial_c: tuple = ("N", 0.0, 0.5)
    sequence_lens: tuple = None     # None: ("I", 0, seq)


def _draw(rng, dist, shape):
    kind = dist[0]
    if kind == "U":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "N":
        return rng.normal(dist[1], dist[2], size=shape)
    if kind == "I":
        return rng.integers(dist[1], dist[2], size=shape, endpoint=True)
    raise ValueError(dist)


def shapes(spec: LayerSpec) -> dict:
    S, B, I, H = spec.seq, spec.batch, spec.input, spec.hidden
    D, G = spec.num_directions, spec.gates
    st = (D, B, H) if spec.layout == 0 else (B, D, H)
    return {
        "X": (S, B, I) if spec.layout == 0 else (B, S, I),
        "W": (D, G * H, I), "R": (D, G * H, H), "B": (D, 2 * G * H),
        "P": (D, 3 * H), "initial_h": st, "initial_c": st, "sequence_lens": (B,),
        "Y": (S, D, B, H) if spec.layout == 0 else (B, S, D, H), "Y_h": st, "Y_c": st,
    }


def make_inputs(spec: LayerSpec, seed: int, dists: Optional[Dists] = None) -> dict:
    """Draw the layer's inputs; float tensors come back in the tensor type."""
    dists = dists or Dists()
    rng = np.random.default_rng(seed)
    shp = shapes(spec)
    npt = np.float32 if spec.dtype == "f32" else np.float16
    out = {}
    out["X"] = _draw(rng, dists.X, shp["X"]).astype(npt)
    out["W"] = _draw(rng, dists.W, shp["W"]).astype(npt)
    out["R"] = _draw(rng, dists.R, shp["R"]).astype(npt)
    if spec.bias:
        out["B"] = _draw(rng, dists.B, shp["B"]).astype(npt)
    if spec.peephole:
        out["P"] = _draw(rng, dists.P, shp["P"]).astype(npt)
    if spec.init_h:
        out["initial_h"] = _draw(rng, dists.initial_h, shp["initial_h"]).astype(npt)
    if spec.init_c:
        out["initial_c"] = _draw(rng, dists.initial_c, shp["initial_c"]).astype(npt)
    if spec.lens:
        d = dists.sequence_lens or ("I", 0, spec.seq)
        out["sequence_lens"] = _draw(rng, d, shp["sequence_lens"]).astype(np.int32)
    return out


# The five seeded synthetic workloads.
CONFIGS = {
    "C1": dict(
        spec=LayerSpec("LSTM", seq=8, batch=1, input=16, hidden=32, dtype="f32",
                       outputs=("Y", "Y_h", "Y_c")),
        dists=Dists(W=("U", -0.25, 0.25), R=("U", -0.25, 0.25), B=("U", -0.25, 0.25)),
        seed=0,
        name="LSTM fwd S8 B1 I16 H32 f32 L0"),
    "C2": dict(
        spec=LayerSpec("LSTM", seq=80, batch=1, input=256, hidden=256, direction="bidirectional",
                       dtype="f32", init_h=True, init_c=True, outputs=("Y", "Y_h")),
        dists=Dists(W=("U", -1 / 16, 1 / 16), R=("U", -1 / 16, 1 / 16), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 0.5), initial_c=("N", 0.0, 0.5)),
        seed=2,
        name="biLSTM S80 B1 I256 H256 f32 L0"),
    "C3": dict(
        spec=LayerSpec("GRU", seq=128, batch=8, input=512, hidden=512, direction="bidirectional",
                       dtype="f16", init_h=True, lens=True, outputs=("Y", "Y_h")),
        dists=Dists(W=("U", -0.044, 0.044), R=("U", -0.044, 0.044), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 1.0), sequence_lens=("I", 1, 128)),
        seed=3,
        name="biGRU S128 B8 I512 H512 f16 L0 lens"),
    # the same GRU layer with the reset gate applied after the recurrent
    # product (linear_before_reset = 1): same shapes, distributions and seed
    "C3L1": dict(
        spec=LayerSpec("GRU", seq=128, batch=8, input=512, hidden=512, direction="bidirectional",
                       dtype="f16", init_h=True, lens=True, linear_before_reset=1, outputs=("Y", "Y_h")),
        dists=Dists(W=("U", -0.044, 0.044), R=("U", -0.044, 0.044), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 1.0), sequence_lens=("I", 1, 128)),
        seed=3,
        name="biGRU S128 B8 I512 H512 f16 L0 lens linear_before_reset"),
    "C4": dict(
        spec=LayerSpec("LSTM", seq=256, batch=64, input=1024, hidden=1024, layout=1, dtype="f16",
                       clip=3.0, input_forget=1, bias=False, peephole=True, lens=True,
                       outputs=("Y", "Y_h", "Y_c")),
        dists=Dists(W=("U", -0.03, 0.03), R=("U", -0.03, 0.03), P=("U", -0.1, 0.1),
                    sequence_lens=("I", 128, 256)),
        seed=4,
        name="LSTM fwd S256 B64 I1024 H1024 f16 L1 peephole clip3 input_forget lens"),
    "C5": dict(
        spec=LayerSpec("RNN", seq=1024, batch=256, input=1024, hidden=2048, direction="bidirectional",
                       dtype="f32", acts=(("Relu", 0.0, 0.0), ("ScaledTanh", 1.5, 0.5)),
                       outputs=("Y", "Y_h")),
        dists=Dists(W=("U", -0.02, 0.02), R=("U", -0.02, 0.02), B=("U", -0.05, 0.05)),
        seed=5,
        name="biRNN S1024 B256 I1024 H2048 f32 L0 Relu/ScaledTanh"),
    # The C2 layer at batch 8 (the small-batch engine's largest) and batch 12
    # (the matrix-core step with one 16-row block): the cost of a batch
    # above eight.
    "C2B8": dict(
        spec=LayerSpec("LSTM", seq=80, batch=8, input=256, hidden=256, direction="bidirectional",
                       dtype="f32", init_h=True, init_c=True, outputs=("Y", "Y_h")),
        dists=Dists(W=("U", -1 / 16, 1 / 16), R=("U", -1 / 16, 1 / 16), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 0.5), initial_c=("N", 0.0, 0.5)),
        seed=2,
        name="biLSTM S80 B8 I256 H256 f32 L0"),
    "C2B12": dict(
        spec=LayerSpec("LSTM", seq=80, batch=12, input=256, hidden=256, direction="bidirectional",
                       dtype="f32", init_h=True, init_c=True, outputs=("Y", "Y_h")),
        dists=Dists(W=("U", -1 / 16, 1 / 16), R=("U", -1 / 16, 1 / 16), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 0.5), initial_c=("N", 0.0, 0.5)),
        seed=2,
        name="biLSTM S80 B12 I256 H256 f32 L0"),
    # The text-line recognizer shapes the "Recurrent layers" page tests
    # ("Tolerance and evidence"): bidirectional LSTMs of sequence 80 and 48,
    # batch 1 and 8, input 256 and 192, hidden 256 and 96.  The page gives
    # no distributions; these follow C2 (uniform weights of scale
    # about 1/sqrt(hidden), N(0,1) inputs, N(0, 0.5) initial states).
    "REC80": dict(
        spec=LayerSpec("LSTM", seq=80, batch=1, input=256, hidden=256, direction="bidirectional",
                       dtype="f32", init_h=True, init_c=True, outputs=("Y", "Y_h", "Y_c")),
        dists=Dists(W=("U", -1 / 16, 1 / 16), R=("U", -1 / 16, 1 / 16), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 0.5), initial_c=("N", 0.0, 0.5)),
        seed=6,
        name="biLSTM S80 B1 I256 H256 f32 L0 (recognizer)"),
    "REC48": dict(
        spec=LayerSpec("LSTM", seq=48, batch=8, input=192, hidden=96, direction="bidirectional",
                       dtype="f32", init_h=True, init_c=True, outputs=("Y", "Y_h", "Y_c")),
        dists=Dists(W=("U", -0.1, 0.1), R=("U", -0.1, 0.1), B=("U", -0.1, 0.1),
                    initial_h=("N", 0.0, 0.5), initial_c=("N", 0.0, 0.5)),
        seed=7,
        name="biLSTM S48 B8 I192 H96 f32 L0 (recognizer)"),
}


def config(name: str, **overrides):
    """(spec, inputs) of a named workload; ``overrides`` replace spec fields."""
    c = CONFIGS[name]
    spec = c["spec"].replace(**overrides) if overrides else c["spec"]
    return spec, make_inputs(spec, c["seed"], c["dists"])

"""ONNX recurrent layers (RNN, GRU, LSTM) on MI355X (gfx950).

A thin ctypes binding over the C ABI of ``include/rnn.h`` (library
``librnn_mi355x.so``, built in-tree by ``onnx_recurrent_layers_amd.build``).
The functions carry the C names and only marshal arguments: every stage of a
layer runs in the library's HIP kernels.  PyTorch supplies device memory and
the stream.  There is no fallback: when the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librnn_mi355x.so")

RNN_OK, RNN_ERR_ARG, RNN_ERR_SHAPE, RNN_ERR_UNSUPPORTED, RNN_ERR_HIP = range(5)
CELLS = {"RNN": 0, "GRU": 1, "LSTM": 2}
DTYPES = {"f32": 0, "f16": 1}
DIRECTIONS = {"forward": 0, "reverse": 1, "bidirectional": 2}
ACTIVATIONS = {
    "Relu": 0, "Tanh": 1, "Sigmoid": 2, "Affine": 3, "LeakyRelu": 4, "ThresholdedRelu": 5,
    "ScaledTanh": 6, "HardSigmoid": 7, "Elu": 8, "Softsign": 9, "Softplus": 10,
}
ENGINES = {"auto": 0, "launch": 1, "persistent": 2}


class RnnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


class rnn_activation(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("alpha", ctypes.c_float), ("beta", ctypes.c_float)]


class rnn_problem_desc(ctypes.Structure):
    _fields_ = [
        ("cell", ctypes.c_int32), ("dtype", ctypes.c_int32), ("direction", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("seq", ctypes.c_int64), ("batch", ctypes.c_int64),
        ("input", ctypes.c_int64), ("hidden", ctypes.c_int64), ("clip", ctypes.c_float),
        ("input_forget", ctypes.c_int32), ("linear_before_reset", ctypes.c_int32),
        ("num_activations", ctypes.c_int32), ("activations", rnn_activation * 6),
        ("max_length", ctypes.c_int64), ("engine", ctypes.c_int32), ("x_bidirectional_y", ctypes.c_int32),
        ("xw_chunk_steps", ctypes.c_int64),
    ]


class rnn_tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("elem_offset", ctypes.c_int64)]


OPERAND_NAMES = ("X", "W", "R", "B", "sequence_lens", "initial_h", "initial_c", "P", "Y", "Y_h", "Y_c")


class rnn_operands(ctypes.Structure):
    _fields_ = [(n, rnn_tensor) for n in OPERAND_NAMES]


class rnn_run_status(ctypes.Structure):
    _fields_ = [("persistent", ctypes.c_int32), ("fallback_workgroups", ctypes.c_int32),
                ("timed_out", ctypes.c_int32)]


class rnn_plan_info(ctypes.Structure):
    _fields_ = [("engine", ctypes.c_int32), ("steps", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("step_blocks", ctypes.c_int32), ("step_launches", ctypes.c_int32),
                ("proj_products", ctypes.c_int32), ("step_products", ctypes.c_int32),
                ("xw_chunk_steps", ctypes.c_int32), ("xw_slots", ctypes.c_int32)]


# rnn_products: which arithmetic units carry a stage's products
PRODUCTS = {0: "f32 vector ALU", 1: "f32 matrix cores", 2: "f16 matrix cores", 3: "bf16x3 matrix cores"}


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m onnx_recurrent_layers_amd.build`")
    # One HIP runtime per process: when PyTorch supplies device memory and
    # streams, load it first so that this library binds to the same runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.rnn_problem_create.argtypes = [P(rnn_problem_desc), P(ctypes.c_void_p)]
    lib.rnn_problem_create.restype = ctypes.c_int
    lib.rnn_problem_destroy.argtypes = [ctypes.c_void_p]
    lib.rnn_problem_destroy.restype = None
    lib.rnn_scratch_size.argtypes = [ctypes.c_void_p, P(ctypes.c_size_t), P(ctypes.c_size_t)]
    lib.rnn_scratch_size.restype = ctypes.c_int
    lib.rnn_encode.argtypes = [ctypes.c_void_p, P(rnn_operands), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.rnn_encode.restype = ctypes.c_int
    lib.rnn_encode_timed.argtypes = [ctypes.c_void_p, P(rnn_operands), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, P(ctypes.c_void_p)]
    lib.rnn_encode_timed.restype = ctypes.c_int
    lib.rnn_validate_lengths.argtypes = [P(ctypes.c_int32), ctypes.c_int64, ctypes.c_int64, P(ctypes.c_int64)]
    lib.rnn_validate_lengths.restype = ctypes.c_int
    lib.rnn_problem_plan.argtypes = [ctypes.c_void_p, P(rnn_plan_info)]
    lib.rnn_problem_plan.restype = ctypes.c_int
    lib.rnn_encode_noalloc.argtypes = [ctypes.c_void_p, P(rnn_operands), ctypes.c_void_p]
    lib.rnn_encode_noalloc.restype = ctypes.c_int
    lib.rnn_read_run_status.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, P(rnn_run_status)]
    lib.rnn_read_run_status.restype = ctypes.c_int
    lib.rnn_last_error.argtypes = []
    lib.rnn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def hip_runtime():
    """The HIP runtime library this process uses (the one the library is bound to)."""
    load_library()
    for line in open("/proc/self/maps"):
        path = line.split()[-1]
        if os.path.basename(path).startswith("libamdhip64.so"):
            return ctypes.CDLL(path)
    return ctypes.CDLL("libamdhip64.so")


def rnn_last_error() -> str:
    return load_library().rnn_last_error().decode()


def _check(rc: int):
    if rc != RNN_OK:
        raise RnnError(rc, rnn_last_error())


def make_desc(spec, engine: str = "auto") -> rnn_problem_desc:
    """rnn_problem_desc from a layer description (``synth.LayerSpec`` fields)."""
    d = rnn_problem_desc()
    d.cell = CELLS[spec.cell]
    d.dtype = DTYPES[spec.dtype]
    d.direction = DIRECTIONS[spec.direction]
    d.layout = int(spec.layout)
    d.seq, d.batch, d.input, d.hidden = int(spec.seq), int(spec.batch), int(spec.input), int(spec.hidden)
    d.clip = float(spec.clip) if spec.clip is not None else 0.0
    d.input_forget = int(spec.input_forget)
    d.linear_before_reset = int(spec.linear_before_reset)
    acts = list(spec.activations)
    d.num_activations = len(acts)
    for i, (name, a, b) in enumerate(acts):
        d.activations[i].kind = ACTIVATIONS[name]
        d.activations[i].alpha = float(a)
        d.activations[i].beta = float(b)
    d.max_length = int(spec.max_length or 0)
    d.engine = ENGINES[engine]
    d.x_bidirectional_y = int(getattr(spec, "x_bidirectional_y", 0))
    d.xw_chunk_steps = int(getattr(spec, "xw_chunk_steps", 0))
    return d


def rnn_problem_create(desc: rnn_problem_desc) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().rnn_problem_create(ctypes.byref(desc), ctypes.byref(h)))
    return h


def rnn_problem_destroy(handle) -> None:
    load_library().rnn_problem_destroy(handle)


def rnn_scratch_size(handle):
    xw, st = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().rnn_scratch_size(handle, ctypes.byref(xw), ctypes.byref(st)))
    return xw.value, st.value


def rnn_problem_plan(handle) -> rnn_plan_info:
    info = rnn_plan_info()
    _check(load_library().rnn_problem_plan(handle, ctypes.byref(info)))
    return info


def rnn_read_run_status(handle, state_scratch_ptr: int, stream_ptr: int = 0) -> rnn_run_status:
    out = rnn_run_status()
    _check(load_library().rnn_read_run_status(handle, ctypes.c_void_p(state_scratch_ptr or None),
                                              ctypes.c_void_p(stream_ptr or None), ctypes.byref(out)))
    return out


def rnn_validate_lengths(lens, seq: int) -> int:
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    mx = ctypes.c_int64()
    _check(load_library().rnn_validate_lengths(arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                               arr.size, int(seq), ctypes.byref(mx)))
    return mx.value


def make_operands(tensors: dict, offsets: Optional[dict] = None) -> rnn_operands:
    """rnn_operands from device tensors (torch) keyed by ONNX names; ``offsets``
    gives element offsets into each tensor's storage (default 0)."""
    ops = rnn_operands()
    offsets = offsets or {}
    for name in OPERAND_NAMES:
        t = tensors.get(name)
        if t is None:
            continue
        tr = getattr(ops, name)
        tr.ptr = t.data_ptr()
        tr.elem_offset = int(offsets.get(name, 0))
    return ops


def rnn_encode(handle, operands: rnn_operands, xw_scratch_ptr: int, state_scratch_ptr: int,
               stream_ptr: int = 0) -> None:
    _check(load_library().rnn_encode(handle, ctypes.byref(operands), ctypes.c_void_p(xw_scratch_ptr or None),
                                     ctypes.c_void_p(state_scratch_ptr or None), ctypes.c_void_p(stream_ptr or None)))


def rnn_encode_noalloc(handle, operands: rnn_operands, stream_ptr: int = 0) -> None:
    """rnn_encode with the library's fixed scratch (no caller scratch)."""
    _check(load_library().rnn_encode_noalloc(handle, ctypes.byref(operands), ctypes.c_void_p(stream_ptr or None)))


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def rnn_encode_timed(handle, operands: rnn_operands, xw_scratch_ptr: int, state_scratch_ptr: int,
                     stream_ptr: int, events) -> None:
    """rnn_encode plus hipEventRecord of five stage-boundary events (hipEvent_t
    handles as ints, or None) on the same stream."""
    ev = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e) if e else None for e in events])
    _check(load_library().rnn_encode_timed(handle, ctypes.byref(operands), ctypes.c_void_p(xw_scratch_ptr or None),
                                           ctypes.c_void_p(state_scratch_ptr or None),
                                           ctypes.c_void_p(stream_ptr or None), ev))


class Layer:
    """One created problem plus its scratch, for repeated encodes."""

    def __init__(self, spec, engine: str = "auto", device: str = "cuda"):
        import torch
        self.spec = spec
        self.handle = rnn_problem_create(make_desc(spec, engine))
        self.xw_bytes, self.state_bytes = rnn_scratch_size(self.handle)
        self.plan = rnn_problem_plan(self.handle)
        self.device = torch.device(device)
        self.xw = torch.empty(max(self.xw_bytes, 256), dtype=torch.uint8, device=self.device)
        self.state = torch.empty(max(self.state_bytes, 256), dtype=torch.uint8, device=self.device)

    def encode(self, tensors: dict, offsets: Optional[dict] = None, stream=None, events=None) -> None:
        import torch
        ops = make_operands(tensors, offsets)
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        xw = self.xw.data_ptr() if self.xw_bytes else 0
        if events is None:
            rnn_encode(self.handle, ops, xw, self.state.data_ptr(), st.cuda_stream)
        else:
            rnn_encode_timed(self.handle, ops, xw, self.state.data_ptr(), st.cuda_stream, events)

    def run_status(self, stream=None) -> rnn_run_status:
        """rnn_read_run_status of this layer's state scratch (waits for the stream)."""
        import torch
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        return rnn_read_run_status(self.handle, self.state.data_ptr() if self.state_bytes else 0, st.cuda_stream)

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                rnn_problem_destroy(self.handle)
                self.handle = None
        except Exception:
            pass


def output_shapes(spec) -> dict:
    S, B, H = spec.seq, spec.batch, spec.hidden
    D = 2 if spec.direction == "bidirectional" else 1
    st = (D, B, H) if spec.layout == 0 else (B, D, H)
    return {"Y": (S, D, B, H) if spec.layout == 0 else (B, S, D, H), "Y_h": st, "Y_c": st}


def to_device(inputs: dict, device: str = "cuda") -> dict:
    """numpy inputs -> torch device tensors (same dtypes)."""
    import numpy as np
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in inputs.items()}


def run(spec, inputs: dict, engine: str = "auto", outputs=None, device: str = "cuda"):
    """Run one layer on device tensors (or numpy arrays, copied to the device);
    returns the requested outputs as torch tensors on the device."""
    import numpy as np
    import torch
    tens = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(device) if isinstance(v, np.ndarray) else v)
            for k, v in inputs.items()}
    dt = torch.float32 if spec.dtype == "f32" else torch.float16
    shapes = output_shapes(spec)
    want = outputs if outputs is not None else spec.outputs
    outs = {}
    for n in want:
        if n == "Y_c" and spec.cell != "LSTM":
            continue
        outs[n] = torch.empty(shapes[n], dtype=dt, device=device)
    layer = Layer(spec, engine=engine, device=device)
    layer.encode({**tens, **outs})
    return outs

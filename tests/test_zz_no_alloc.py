"""rnn_encode_noalloc (the entry point for callers that cannot allocate)
against rnn_encode: the same kernels, so the outputs must be bit-identical.
Two calls in a row share the library's fixed scratch; the second takes a
smaller layer, so whatever the first left behind must not matter."""
import numpy as np
import pytest

import onnx_recurrent_layers_amd as rl
from onnx_recurrent_layers_amd import synth
from onnx_recurrent_layers_amd.synth import LayerSpec, Dists, make_inputs
from tests.gpu_harness import gpu_layer, note


def _noalloc(spec, inputs):
    """The layer through rnn_encode_noalloc, outputs surrounded by sentinels."""
    import torch
    dev = torch.device("cuda", 0)
    dt = torch.float32 if spec.dtype == "f32" else torch.float16
    tens = rl.to_device(inputs, "cuda:0")
    shapes = rl.output_shapes(spec)
    outs = {}
    for n in spec.outputs:
        if n == "Y_c" and spec.cell != "LSTM":
            continue
        numel = int(np.prod(shapes[n]))
        outs[n] = torch.full((numel + 8,), -777.0, dtype=dt, device=dev)
    h = rl.rnn_problem_create(rl.make_desc(spec, "auto"))
    try:
        ops = rl.make_operands({**tens, **outs})
        rl.rnn_encode_noalloc(h, ops, torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()
    finally:
        rl.rnn_problem_destroy(h)
    res = {}
    for n, buf in outs.items():
        host = buf.cpu()
        numel = int(np.prod(shapes[n]))
        assert bool((host[numel:] == -777.0).all()), f"{n}: written past its end"
        res[n] = host[:numel].view(shapes[n]).numpy()
    return res


# (large layer, smaller layer) pairs: the small-batch persistent engine, the
# matrix-core step in its persistent form, one launch per step
PAIRS = [
    ("C2", dict(), dict(seq=40, hidden=128, input=64)),
    ("C3", dict(), dict(seq=50, batch=5, hidden=200)),
    (None, LayerSpec("LSTM", seq=12, batch=24, input=40, hidden=64, dtype="f16", direction="bidirectional",
                     init_h=True, init_c=True, lens=True, peephole=True),
     dict(seq=7, batch=17, hidden=48)),
    (None, LayerSpec("GRU", seq=9, batch=11, input=30, hidden=70, direction="bidirectional", lens=True,
                     init_h=True), dict(seq=5, batch=10, hidden=33)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,first,second", PAIRS, ids=["C2", "C3", "matrix-core", "per-step"])
def test_noalloc_matches_rnn_encode(name, first, second):
    if name is not None:
        spec, inp = synth.config(name, **first)
    else:
        spec = first
        inp = make_inputs(spec, 5, Dists(sequence_lens=("I", 0, spec.seq)))
    small = spec.replace(**second)
    sinp = make_inputs(small, 6, Dists(sequence_lens=("I", 0, small.seq)))
    for sp, ip in ((spec, inp), (small, sinp)):
        note(f"case noalloc {sp}")
        want = gpu_layer(sp, ip)
        got = _noalloc(sp, ip)
        for n in want:
            assert np.array_equal(want[n].view(np.uint8), got[n].view(np.uint8)), f"{n}: rnn_encode_noalloc differs"


def test_noalloc_rejects_layers_above_its_scratch():
    """The size check runs before anything touches the device."""
    spec, _ = synth.config("C5")
    h = rl.rnn_problem_create(rl.make_desc(spec, "auto"))
    try:
        with pytest.raises(rl.RnnError) as err:
            rl.rnn_encode_noalloc(h, rl.rnn_operands(), 0)
        assert err.value.code == rl.RNN_ERR_UNSUPPORTED
        assert err.value.message.startswith("RNN:") and "fixed scratch" in err.value.message
    finally:
        rl.rnn_problem_destroy(h)

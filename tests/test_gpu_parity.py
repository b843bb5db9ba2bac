"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Bar: max abs error 1e-4 for f32 outputs and 5e-3 for f16 outputs; two runs
bit-identical; nothing outside an output's extent written (sentinels)."""
import itertools

import numpy as np
import pytest

from onnx_recurrent_layers_amd import synth
from onnx_recurrent_layers_amd.synth import LayerSpec, Dists, make_inputs
from oracle import oracle
from tests.gpu_harness import gpu_layer, compare, oracle_rows, select_rows, note

pytestmark = pytest.mark.gpu

ENGINES = ["launch", "persistent"]


def batch_for(engine, b_launch):
    """The persistent engine takes batches up to 8; the per-step one any batch."""
    return b_launch if engine == "launch" else min(b_launch, 7)


def check(spec, inputs, engine="auto", offsets=None, twice=True, what=""):
    note(f"case {what} engine={engine} spec={spec}")
    got = gpu_layer(spec, inputs, engine=engine, offsets=offsets)
    ref = oracle.run(spec, inputs, outputs=spec.outputs)
    rep = compare(spec, got, ref, what=what)
    if twice:
        again = gpu_layer(spec, inputs, engine=engine, offsets=offsets)
        for n in got:
            assert np.array_equal(got[n].view(np.uint8), again[n].view(np.uint8)), f"{what} {n}: runs differ"
    return rep


# ---------------------------------------------------------------------------
# projection (stage 1) against the oracle's plain product, read from scratch
# ---------------------------------------------------------------------------
def step_rows(X, layout, S, B, d):
    """A operand of direction d in the projection scratch's step order (full
    lengths): row s*B + b is X at time s (forward, d = 0) or S-1-s (the
    reverse direction, d = 1)."""
    Xs = X if layout == 0 else X.transpose(1, 0, 2)
    if d == 1:
        Xs = Xs[::-1]
    return np.ascontiguousarray(Xs).reshape(S * B, -1)


@pytest.mark.parametrize("dtype,layout", [("f32", 0), ("f16", 0), ("f32", 1), ("f16", 1)])
def test_projection_scratch(dtype, layout):
    import torch
    spec = LayerSpec("LSTM", seq=13, batch=11, input=70, hidden=37, layout=layout, dtype=dtype,
                     direction="bidirectional", outputs=("Y_h",))
    inp = make_inputs(spec, 5)
    note(f"case projection {dtype} L{layout}")
    _, layer = gpu_layer(spec, inp, engine="launch", return_layer=True)
    torch.cuda.synchronize()
    D, S, B, G, H, I = 2, spec.seq, spec.batch, 4, spec.hidden, spec.input
    xw = layer.xw[: layer.xw_bytes].view(torch.float32).view(D, S * B, G * H).cpu().numpy()
    for d in range(D):
        A = step_rows(inp["X"], layout, S, B, d)
        ref = oracle.projection(A, inp["W"][d])
        err = np.max(np.abs(xw[d].astype(np.float64) - ref))
        assert err <= 1e-4, (d, err)


# The latency-bound projection kernel for small layers (32x32 tiles, K split
# over the four waves, one round of loads per K block), forced on (and, for
# comparison, off) with RNN_SMALL_PROJECTION: whole K blocks and ragged ones,
# K not a whole number of 16-byte segments (element loads), several blocks
# per wave, tiles inside the skipped f block, M and N below one tile.
@pytest.mark.parametrize("dtype,layout,cell,input_forget,S,B,I,H", [
    ("f32", 0, "LSTM", 0, 13, 11, 70, 37),
    ("f32", 1, "GRU", 0, 9, 5, 256, 64),
    ("f16", 0, "RNN", 0, 7, 3, 520, 40),
    ("f32", 0, "LSTM", 1, 5, 2, 1000, 64),
    ("f16", 1, "LSTM", 1, 6, 4, 77, 50),
    ("f32", 0, "LSTM", 0, 8, 1, 16, 32),
])
@pytest.mark.parametrize("force", ["1", "0"])
def test_projection_small_kernel(dtype, layout, cell, input_forget, S, B, I, H, force, monkeypatch):
    import torch
    monkeypatch.setenv("RNN_SMALL_PROJECTION", force)
    spec = LayerSpec(cell, seq=S, batch=B, input=I, hidden=H, layout=layout, dtype=dtype, input_forget=input_forget,
                     direction="bidirectional", outputs=("Y_h",))
    inp = make_inputs(spec, 9)
    note(f"case projection small={force} {dtype} {cell} L{layout} S{S} B{B} I{I} H{H}")
    _, layer = gpu_layer(spec, inp, engine="launch", return_layer=True)
    torch.cuda.synchronize()
    D, G = 2, spec.gates
    xw = layer.xw[: layer.xw_bytes].view(torch.float32).view(D, S * B, G * H).cpu().numpy()
    for d in range(D):
        A = step_rows(inp["X"], layout, S, B, d)
        ref = oracle.projection(A, inp["W"][d])
        cols = np.ones(G * H, bool)
        if input_forget:
            cols[2 * H:3 * H] = False     # the f block is not computed
        # f16 products are exact in f32 and f32 products round once; the f32
        # sums of K terms (in any fixed order) stay within (K + 4) * 2^-23 of
        # sum |x_k * w_k|
        bound = (I + 4) * 2.0 ** -23 * (np.abs(A.astype(np.float64)) @ np.abs(inp["W"][d].astype(np.float64)).T)
        err = np.abs(xw[d][:, cols].astype(np.float64) - ref[:, cols])
        assert np.all(err <= bound[:, cols] + 1e-30), (d, float(np.max(err / (bound[:, cols] + 1e-30))))
    # and the whole layer through it
    check(spec, inp, engine="launch", twice=False, what=f"small projection {force}")


# f32 tensors with the projection on the bf16 matrix cores (three split
# products, forced with RNN_F32_SPLIT=1 on small shapes).  Each element of Xw
# must lie within 2^-15 * sum_k |x_k * w_k| of the exact product: the split
# leaves residuals of at most 2^-16 of each |x_k * w_k|, and f32 accumulation
# of K terms adds below K * 2^-24 of the same sum.
@pytest.mark.parametrize("layout,S,B,I,H", [(0, 13, 11, 70, 37), (1, 9, 21, 130, 72), (0, 3, 40, 1024, 64)])
def test_projection_scratch_bf16x3(layout, S, B, I, H, monkeypatch):
    import torch
    monkeypatch.setenv("RNN_F32_SPLIT", "1")
    spec = LayerSpec("GRU", seq=S, batch=B, input=I, hidden=H, layout=layout, dtype="f32",
                     direction="bidirectional", outputs=("Y_h",))
    inp = make_inputs(spec, 8)
    note(f"case projection bf16x3 L{layout} S{S} B{B} I{I} H{H}")
    _, layer = gpu_layer(spec, inp, engine="launch", return_layer=True)
    torch.cuda.synchronize()
    D, G = 2, 3
    xw = layer.xw[: layer.xw_bytes].view(torch.float32).view(D, S * B, G * H).cpu().numpy()
    for d in range(D):
        A = step_rows(inp["X"], layout, S, B, d)
        ref = oracle.projection(A, inp["W"][d])
        bound = 2.0 ** -15 * (np.abs(A.astype(np.float64)) @ np.abs(inp["W"][d].astype(np.float64)).T) + 1e-30
        err = np.abs(xw[d].astype(np.float64) - ref)
        assert np.all(err <= bound), (d, float(np.max(err / bound)))
        assert np.max(err) <= 1e-4


# The same split products in the 256x256 tiles loaded straight into LDS (f32
# operands split as they are read), forced onto small layers: ragged M, N and
# K tails, layout 1, the skipped f block.
@pytest.mark.parametrize("layout,cell,input_forget,S,B,I,H", [
    (0, "GRU", 0, 17, 19, 200, 90), (1, "LSTM", 1, 9, 70, 136, 256), (0, "RNN", 0, 3, 40, 1024, 300)])
def test_projection_lds_bf16x3(layout, cell, input_forget, S, B, I, H, monkeypatch):
    import torch
    monkeypatch.setenv("RNN_F32_SPLIT", "1")
    monkeypatch.setenv("RNN_PROJ_LDS_MIN_TILES", "1")
    spec = LayerSpec(cell, seq=S, batch=B, input=I, hidden=H, layout=layout, dtype="f32", input_forget=input_forget,
                     direction="bidirectional", outputs=("Y_h",))
    inp = make_inputs(spec, 12)
    note(f"case projection-lds bf16x3 {cell} L{layout} S{S} B{B} I{I} H{H}")
    _, layer = gpu_layer(spec, inp, engine="launch", return_layer=True)
    torch.cuda.synchronize()
    D, G = 2, spec.gates
    xw = layer.xw[: layer.xw_bytes].view(torch.float32).view(D, S * B, G * H).cpu().numpy()
    for d in range(D):
        A = step_rows(inp["X"], layout, S, B, d)
        ref = oracle.projection(A, inp["W"][d])
        bound = 2.0 ** -15 * (np.abs(A.astype(np.float64)) @ np.abs(inp["W"][d].astype(np.float64)).T) + 1e-30
        cols = np.ones(G * H, bool)
        if input_forget:
            cols[2 * H:3 * H] = False     # the f block is not computed
        err = np.abs(xw[d][:, cols].astype(np.float64) - ref[:, cols])
        assert np.all(err <= bound[:, cols]), (d, float(np.max(err / bound[:, cols])))
    check(spec, inp, engine="launch", twice=False, what=f"projection-lds bf16x3 {cell}")


@pytest.mark.parametrize("cell", ["LSTM", "GRU", "RNN"])
def test_layers_with_bf16x3_projection(cell, monkeypatch):
    """Whole f32 layers with the split projection, on both engines."""
    monkeypatch.setenv("RNN_F32_SPLIT", "1")
    for engine, B in (("launch", 37), ("persistent", 5), ("launch", 3)):
        spec = LayerSpec(cell, seq=9, batch=B, input=200, hidden=48, direction="bidirectional", dtype="f32",
                         layout=B % 2, init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM",
                         clip=2.5, linear_before_reset=1 if (B == 5 and cell == "GRU") else 0,
                         outputs=("Y", "Y_h", "Y_c"))
        inp = make_inputs(spec, 41, Dists(sequence_lens=("I", 0, 9)))
        check(spec, inp, engine=engine, what=f"bf16x3 projection {cell} {engine} B{B}")


@pytest.mark.parametrize("layout,cell,input_forget,S,B,I,H", [
    (0, "LSTM", 0, 13, 11, 72, 40),      # ragged M, N and K tails, several tiles
    (1, "LSTM", 1, 9, 70, 136, 256),     # skipped f block of whole tiles, layout 1
    (1, "GRU", 0, 33, 17, 264, 96),
    (0, "RNN", 0, 40, 20, 520, 300),
    (0, "GRU", 0, 11, 23, 64, 45),       # rows of Xw not in 16-byte groups (G*H odd): one value per store
])
def test_projection_lds_tiles(layout, cell, input_forget, S, B, I, H, monkeypatch):
    """The 256x256 f16 projection loaded straight into LDS, forced onto small
    layers, against the oracle's plain product."""
    import torch
    monkeypatch.setenv("RNN_PROJ_LDS_MIN_TILES", "1")
    spec = LayerSpec(cell, seq=S, batch=B, input=I, hidden=H, layout=layout, dtype="f16", input_forget=input_forget,
                     direction="bidirectional", outputs=("Y_h",))
    inp = make_inputs(spec, 7)
    note(f"case projection-lds {cell} L{layout} S{S} B{B} I{I} H{H}")
    _, layer = gpu_layer(spec, inp, engine="launch", return_layer=True)
    torch.cuda.synchronize()
    D, G = 2, spec.gates
    xw = layer.xw[: layer.xw_bytes].view(torch.float32).view(D, S * B, G * H).cpu().numpy()
    for d in range(D):
        A = step_rows(inp["X"], layout, S, B, d)
        ref = oracle.projection(A, inp["W"][d])
        cols = np.ones(G * H, bool)
        if input_forget:
            cols[2 * H:3 * H] = False     # the f block is not computed
        err = np.max(np.abs(xw[d][:, cols].astype(np.float64) - ref[:, cols]))
        assert err <= 1e-3, (d, err)


def test_projection_scratch_step_order_with_lengths():
    """The reverse direction with sequence lengths: row b of step s holds the
    projection of X at time len_b - 1 - s while the row runs."""
    import torch
    S, B, I, H = 9, 6, 24, 20
    spec = LayerSpec("RNN", seq=S, batch=B, input=I, hidden=H, direction="bidirectional", dtype="f32", lens=True,
                     outputs=("Y_h",))
    inp = make_inputs(spec, 15)
    inp["sequence_lens"] = np.array([9, 0, 4, 1, 7, 12], np.int32)
    _, layer = gpu_layer(spec, inp, engine="launch", return_layer=True)
    torch.cuda.synchronize()
    xw = layer.xw[: layer.xw_bytes].view(torch.float32).view(2, S, B, H).cpu().numpy()
    for d in range(2):
        ref = oracle.projection(inp["X"].reshape(S * B, I), inp["W"][d]).reshape(S, B, H)
        for b, Lb in enumerate(np.clip(inp["sequence_lens"], 0, S)):
            for st in range(Lb):
                t = st if d == 0 else Lb - 1 - st
                assert np.max(np.abs(xw[d, st, b] - ref[t, b])) <= 1e-4, (d, st, b)


# The projection in chunks through a ring of two slots (xw_chunk_steps), on
# the per-step engines: chunks of 3 over 10 steps (the ring wraps three times
# and the last chunk is short), the vector kernel and the matrix-core step,
# reverse rows with their own lengths, both layouts, a row split in two
# pieces (x_bidirectional_y); on the caller's stream and with each chunk's
# projection on a second stream ahead of the steps (RNN_CHUNK_OVERLAP); against
# the oracle, twice bit-identical.
CHUNKS = [("LSTM", 5, "f32", 0, 3), ("GRU", 18, "f16", 1, 3), ("RNN", 20, "f32", 0, 4), ("LSTM", 17, "f16", 0, 1),
          ("GRU", 3, "f32", 1, 7)]


@pytest.mark.parametrize("cell,B,dtype,layout,chunk", CHUNKS, ids=[f"{c}-B{b}-{d}-L{l}-c{k}" for c, b, d, l, k in CHUNKS])
@pytest.mark.parametrize("overlap", ["0", "1"])
def test_projection_in_chunks(cell, B, dtype, layout, chunk, overlap, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    monkeypatch.setenv("RNN_CHUNK_OVERLAP", overlap)
    spec = LayerSpec(cell, seq=10, batch=B, input=26, hidden=40, direction="bidirectional", layout=layout,
                     dtype=dtype, init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM",
                     clip=3.0, xw_chunk_steps=chunk, outputs=("Y", "Y_h", "Y_c"))
    layer = rl.Layer(spec, engine="launch", device="cuda:0")
    assert layer.plan.xw_slots == 2 and layer.plan.xw_chunk_steps == chunk
    inp = make_inputs(spec, 121, Dists(sequence_lens=("I", 0, 10), W=("U", -0.3, 0.3), R=("U", -0.3, 0.3)))
    check(spec, inp, engine="launch", what=f"chunks of {chunk} {cell} B{B} {dtype} L{layout}")


def test_projection_in_chunks_split_rows():
    """A stacked layout-0 layer (rows in two pieces) with its projection in
    chunks."""
    import onnx_recurrent_layers_amd as rl
    S, B, H1 = 10, 18, 16
    s1 = LayerSpec("GRU", seq=S, batch=B, input=12, hidden=H1, direction="bidirectional", layout=0, dtype="f32",
                   lens=True, outputs=("Y",))
    in1 = make_inputs(s1, 123, Dists(sequence_lens=("I", 1, S)))
    y1 = rl.run(s1, in1, outputs=("Y",))["Y"]
    s2 = LayerSpec("LSTM", seq=S, batch=B, input=2 * H1, hidden=24, direction="bidirectional", layout=0, dtype="f32",
                   lens=True, xw_chunk_steps=4, outputs=("Y", "Y_h"))
    in2 = make_inputs(s2, 124)
    in2["sequence_lens"] = in1["sequence_lens"]
    dev = rl.to_device({k: v for k, v in in2.items() if k != "X"})
    got = rl.run(s2.replace(x_bidirectional_y=1), {**dev, "X": y1}, engine="launch", outputs=s2.outputs)
    xt = y1.permute(0, 2, 1, 3).contiguous().view(S, B, 2 * H1).cpu().numpy()
    ref = oracle.run(s2, {**in2, "X": xt}, outputs=s2.outputs)
    compare(s2, {k: v.cpu().numpy() for k, v in got.items()}, ref, what="chunked split rows")


# ---------------------------------------------------------------------------
# the page's test matrix on small shapes that span several tiles and a ragged tail
# ---------------------------------------------------------------------------
MATRIX = []
for cell, direction, layout, dtype in itertools.product(("LSTM", "GRU", "RNN"),
                                                         ("forward", "reverse", "bidirectional"),
                                                         (0, 1), ("f32", "f16")):
    MATRIX.append((cell, direction, layout, dtype))


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("cell,direction,layout,dtype", MATRIX, ids=["-".join(map(str, m)) for m in MATRIX])
def test_matrix_options(cell, direction, layout, dtype, engine):
    lbrs = (0, 1) if cell == "GRU" else (0,)
    for lbr in lbrs:
        spec = LayerSpec(cell, seq=9, batch=batch_for(engine, 11), input=70, hidden=37, direction=direction, layout=layout,
                         dtype=dtype, linear_before_reset=lbr, init_h=True, init_c=cell == "LSTM",
                         lens=True, peephole=cell == "LSTM", clip=2.5,
                         outputs=("Y", "Y_h", "Y_c"))
        inp = make_inputs(spec, 17, Dists(sequence_lens=("I", 0, 9), W=("U", -0.3, 0.3), R=("U", -0.3, 0.3)))
        check(spec, inp, engine=engine, what=f"{cell}/{direction}/L{layout}/{dtype}/lbr{lbr}")
    if cell == "LSTM":
        spec = LayerSpec(cell, seq=6, batch=batch_for(engine, 9), input=33, hidden=70, direction=direction, layout=layout,
                         dtype=dtype, input_forget=1, peephole=True, bias=False, lens=False)
        check(spec, make_inputs(spec, 18), engine=engine, what=f"LSTM input_forget {direction} L{layout} {dtype}")


# f16 layers with the default activations and four to eight batch rows take
# the persistent engine's matrix-core products: one to four 16-row blocks per
# workgroup, k chunks that do not split evenly over the four waves (or leave
# waves without a chunk), partial last workgroups, both GRU forms.
PERS_MFMA_CASES = [
    # cell, direction, layout, option, B, H
    ("LSTM", "bidirectional", 0, "peep", 4, 100),     # 64 rows: four blocks
    ("LSTM", "forward", 1, "input_forget", 3, 300),   # 48 rows: three blocks
    ("LSTM", "reverse", 1, "peep", 8, 256),           # 32 rows: two blocks
    ("GRU", "bidirectional", 0, "lbr0", 8, 520),      # 16 + 8 rows, two products
    ("GRU", "forward", 1, "lbr1", 5, 33),             # 24 rows, k chunks on two waves only
    ("GRU", "reverse", 0, "lbr0", 4, 70),             # 32 + 16 rows
    ("RNN", "bidirectional", 0, "", 6, 1000),         # 8 rows, 32 k chunks
    ("RNN", "forward", 1, "", 4, 17),                 # 16 rows, one k chunk
]


@pytest.mark.parametrize("cell,direction,layout,opt,B,H", PERS_MFMA_CASES,
                         ids=[f"{c[0]}-{c[1]}-L{c[2]}-{c[3]}-B{c[4]}-H{c[5]}" for c in PERS_MFMA_CASES])
def test_persistent_matrix_products(cell, direction, layout, opt, B, H):
    spec = LayerSpec(cell, seq=11, batch=B, input=45, hidden=H, direction=direction, layout=layout, dtype="f16",
                     linear_before_reset=1 if opt == "lbr1" else 0, input_forget=1 if opt == "input_forget" else 0,
                     peephole=opt == "peep", clip=3.0 if cell == "LSTM" else None, init_h=True,
                     init_c=cell == "LSTM", lens=True, outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 31, Dists(sequence_lens=("I", 0, 11), W=("U", -0.2, 0.2), R=("U", -0.2, 0.2)))
    check(spec, inp, engine="persistent", what=f"persistent mfma {cell}/{direction}/L{layout}/{opt}/B{B}/H{H}")


def _residency_words(layer, spec):
    """status, arrival tickets and residency decision of the small-batch
    persistent engine, read back from the state scratch (they follow the two
    slots of exchange words, and the r*h words of a GRU with
    linear_before_reset = 0)."""
    import torch
    al = lambda n: (n + 255) // 256 * 256
    dbh = (2 if spec.direction == "bidirectional" else 1) * spec.batch * spec.hidden
    off = al(16 * dbh)
    if spec.cell == "GRU" and not spec.linear_before_reset:
        off += al(16 * dbh)
    torch.cuda.synchronize()
    return [int(v) for v in layer.state[off:off + 12].view(torch.int32).cpu()]


# The persistent engine is launched plainly and its workgroups agree first
# whether all of them run at once (GO), else the ones that arrived take the
# place of the whole grid in turn (the fallback), through the same products
# and gate code.  The fallback is forced here with RNN_PERSISTENT_FALLBACK = k
# (k workgroups take part): every cell and GRU form, lengths with 0, initial
# states, peepholes, clip, input_forget, both dtypes (the vector-ALU and the
# matrix-core instances), both layouts, one batch row (staggered polling).
# Its outputs must be bit-identical to the fast path's; the residency words
# and the library's run status show which path ran.
FALLBACK = [("LSTM", 0, "f32", 0, 5), ("LSTM", 1, "f16", 1, 6), ("GRU", 0, "f32", 1, 5), ("GRU", 1, "f16", 0, 6),
            ("RNN", 0, "f32", 0, 5), ("LSTM", 0, "f16", 0, 6), ("GRU", 0, "f16", 0, 4), ("LSTM", 0, "f32", 1, 1),
            ("GRU", 0, "f32", 0, 1)]


@pytest.mark.parametrize("cell,opt,dtype,layout,B", FALLBACK,
                         ids=[f"{c}-{o}-{d}-L{l}-B{b}" for c, o, d, l, b in FALLBACK])
@pytest.mark.parametrize("forced", ["1", "2"])
def test_persistent_fallback(cell, opt, dtype, layout, B, forced, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=10, batch=B, input=37, hidden=70, direction="bidirectional", layout=layout,
                     dtype=dtype, linear_before_reset=opt if cell == "GRU" else 0,
                     input_forget=opt if cell == "LSTM" else 0, peephole=cell == "LSTM", clip=2.5,
                     init_h=True, init_c=cell == "LSTM", lens=True, outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 61, Dists(sequence_lens=("I", 0, 10)))
    layer = rl.Layer(spec, engine="persistent", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_blocks > 2
    note(f"case persistent fallback {forced} {cell}/opt{opt}/{dtype}/L{layout}/B{B}")
    fast = gpu_layer(spec, inp, layer=layer)
    status, arrivals, decision = _residency_words(layer, spec)
    assert status == 0 and decision == 1 and arrivals == layer.plan.step_blocks, (status, arrivals, decision)
    compare(spec, fast, oracle.run(spec, inp, outputs=spec.outputs), what=f"persistent {cell}")
    monkeypatch.setenv("RNN_PERSISTENT_FALLBACK", forced)
    slow = gpu_layer(spec, inp, layer=layer)
    status, arrivals, decision = _residency_words(layer, spec)
    assert status == 0 and decision == (2 | (int(forced) << 8)), (status, arrivals, decision)
    run = layer.run_status()
    assert run.persistent == 1 and run.fallback_workgroups == int(forced) and run.timed_out == 0
    for n in fast:
        assert np.array_equal(fast[n].view(np.uint8), slow[n].view(np.uint8)), f"fallback {forced} {cell} {n}: bits differ"


# One batch row on the persistent engine: the staggered polling (hidden sizes
# up to 384) and the two lane groups per row of the vector-ALU products (16
# rows or fewer per workgroup, two k chunks or more), for every cell and GRU
# form, both directions, both dtypes, on both sides of each limit.
BATCH1 = [(c, o, H) for c, o in (("LSTM", 0), ("LSTM", 1), ("GRU", 0), ("GRU", 1), ("RNN", 0))
          for H in (32, 40, 64, 300, 400)]


@pytest.mark.parametrize("cell,opt,H", BATCH1, ids=[f"{c}-{o}-H{h}" for c, o, h in BATCH1])
def test_persistent_batch_one(cell, opt, H):
    import onnx_recurrent_layers_amd as rl
    for dtype, direction, layout in (("f32", "bidirectional", 0), ("f16", "reverse", 1)):
        spec = LayerSpec(cell, seq=7, batch=1, input=29, hidden=H, direction=direction, layout=layout, dtype=dtype,
                         linear_before_reset=opt if cell == "GRU" else 0, input_forget=opt if cell == "LSTM" else 0,
                         init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM", clip=2.5,
                         outputs=("Y", "Y_h", "Y_c"))
        layer = rl.Layer(spec, engine="persistent", device="cuda:0")
        assert layer.plan.engine == rl.ENGINES["persistent"]
        inp = make_inputs(spec, 101, Dists(sequence_lens=("I", 1, 7), W=("U", -0.15, 0.15), R=("U", -0.15, 0.15)))
        check(spec, inp, engine="persistent", what=f"batch one {cell}/opt{opt}/H{H}/{dtype}")


LARGE = [(c, d, dt) for c in ("LSTM", "GRU", "RNN") for d in ("forward", "bidirectional") for dt in ("f32", "f16")]


@pytest.mark.parametrize("cell,direction,dtype", LARGE, ids=["-".join(m) for m in LARGE])
def test_large_batch_matrix_engine(cell, direction, dtype):
    """Batches of 16 and more take the matrix-core step kernel: ragged batch
    and hidden sizes, every option, both GRU forms, both layouts."""
    for lbr, layout, B, H in ((0, 0, 37, 50), (1, 1, 70, 33), (0, 1, 16, 130), (1, 0, 20, 700)):
        if cell != "GRU" and lbr == 1:
            lbr = 0
        spec = LayerSpec(cell, seq=7, batch=B, input=29, hidden=H, direction=direction, layout=layout,
                         dtype=dtype, linear_before_reset=lbr if cell == "GRU" else 0, init_h=True,
                         init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM", clip=2.0,
                         input_forget=1 if (cell == "LSTM" and B == 70) else 0,
                         outputs=("Y", "Y_h", "Y_c"))
        inp = make_inputs(spec, 23, Dists(sequence_lens=("I", 0, 7), W=("U", -0.3, 0.3), R=("U", -0.3, 0.3)))
        check(spec, inp, engine="launch", what=f"large {cell}/{direction}/{dtype}/lbr{lbr}/L{layout}/B{B}/H{H}")


# Layers whose rows are whole 16-byte segments take the direct-to-LDS
# matrix-core step; RNN_MFMA_TILE forces each tile shape (and with it the
# one- or two-block column split) on small layers.  Hidden sizes leave a
# partial last k chunk and a partial last unit tile; batches leave empty rows.
DMA_CASES = [
    # cell, dtype, direction, layout, option, B, H, tile
    ("LSTM", "f32", "bidirectional", 0, 0, 37, 64, "16x16"),
    ("LSTM", "f32", "forward", 1, 0, 37, 72, "64x32"),
    ("LSTM", "f16", "bidirectional", 1, 1, 33, 264, "32x32"),
    ("LSTM", "f16", "reverse", 0, 0, 40, 136, "16x32"),
    ("GRU", "f16", "bidirectional", 0, 0, 70, 136, "64x32"),
    ("GRU", "f32", "reverse", 0, 1, 20, 256, "32x16"),
    ("GRU", "f32", "forward", 1, 0, 17, 96, "64x16"),
    ("RNN", "f32", "bidirectional", 0, 0, 20, 520, "64x64"),
    ("RNN", "f16", "forward", 1, 0, 64, 128, "64x64"),
    ("GRU", "f16", "forward", 0, 1, 16, 1024, None),
]


@pytest.mark.parametrize("cell,dtype,direction,layout,opt,B,H,tile", DMA_CASES,
                         ids=["-".join(map(str, c)) for c in DMA_CASES])
def test_matrix_step_direct_to_lds(cell, dtype, direction, layout, opt, B, H, tile, monkeypatch):
    if tile:
        monkeypatch.setenv("RNN_MFMA_TILE", tile)
    spec = LayerSpec(cell, seq=6, batch=B, input=24, hidden=H, direction=direction, layout=layout, dtype=dtype,
                     linear_before_reset=opt if cell == "GRU" else 0,
                     input_forget=opt if cell == "LSTM" else 0, init_h=True, init_c=cell == "LSTM",
                     lens=True, peephole=cell == "LSTM", clip=2.0, outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 31, Dists(sequence_lens=("I", 0, 6), W=("U", -0.2, 0.2), R=("U", -0.1, 0.1)))
    check(spec, inp, engine="launch", what=f"lds-direct {cell}/{dtype}/{direction}/L{layout}/opt{opt}/B{B}/H{H}/{tile}")


# f32 layers whose per-step product runs on the bf16 matrix cores (h and R as
# bf16 hi/lo planes, three split products), forced with RNN_F32_SPLIT=1 on
# small layers: every cell, both GRU forms, every tile shape, ragged batch
# and a partial last k chunk, non-default activations.
SPLIT_CASES = [
    # cell, direction, layout, option, B, H, tile, activations
    ("LSTM", "bidirectional", 0, 0, 37, 64, "16x16", None),
    ("LSTM", "forward", 1, 1, 40, 136, "32x32", None),
    ("GRU", "bidirectional", 0, 0, 70, 136, "64x32", None),
    ("GRU", "reverse", 1, 1, 20, 256, "32x16", None),
    ("RNN", "bidirectional", 0, 0, 33, 520, "64x64", (("Relu", 0, 0), ("ScaledTanh", 1.5, 0.5))),
    ("RNN", "forward", 1, 0, 64, 128, None, (("Softsign", 0, 0),)),
    ("GRU", "forward", 0, 0, 17, 96, "64x16", (("HardSigmoid", 0.2, 0.5), ("Elu", 0.9, 0))),
]


@pytest.mark.parametrize("cell,direction,layout,opt,B,H,tile,acts", SPLIT_CASES,
                         ids=["-".join(map(str, c[:7])) for c in SPLIT_CASES])
def test_matrix_step_bf16x3(cell, direction, layout, opt, B, H, tile, acts, monkeypatch):
    monkeypatch.setenv("RNN_F32_SPLIT", "1")
    if tile:
        monkeypatch.setenv("RNN_MFMA_TILE", tile)
    spec = LayerSpec(cell, seq=7, batch=B, input=40, hidden=H, direction=direction, layout=layout, dtype="f32",
                     linear_before_reset=opt if cell == "GRU" else 0, input_forget=opt if cell == "LSTM" else 0,
                     init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM", clip=2.0,
                     acts=acts, outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 43, Dists(sequence_lens=("I", 0, 7), W=("U", -0.2, 0.2), R=("U", -0.1, 0.1)))
    check(spec, inp, engine="launch", what=f"bf16x3 step {cell}/{direction}/L{layout}/opt{opt}/B{B}/H{H}/{tile}")


# The persistent form of the matrix-core step (one launch for
# every step, batches of 16 and more): the three modes, every cell, both GRU
# forms (two phases per step), forced tile shapes and column splits, ragged
# batch and hidden sizes, lengths with 0, both layouts and directions.
PERS_MFMA_CASES = [
    # cell, dtype, direction, layout, option, B, H, tile, split
    ("LSTM", "f16", "forward", 1, 1, 64, 128, None, None),
    ("LSTM", "f16", "bidirectional", 0, 0, 37, 136, "32x32", None),
    ("GRU", "f16", "bidirectional", 1, 0, 70, 136, "64x32", None),
    ("GRU", "f16", "reverse", 0, 1, 20, 256, "16x16", None),
    ("RNN", "f16", "forward", 0, 0, 33, 520, "64x64", None),
    ("LSTM", "f32", "bidirectional", 0, 0, 37, 64, "16x16", "0"),
    ("GRU", "f32", "forward", 1, 0, 17, 96, "64x16", "0"),
    ("RNN", "f32", "reverse", 0, 0, 40, 72, None, "0"),
    ("LSTM", "f32", "reverse", 1, 1, 40, 136, "32x32", "1"),
    ("GRU", "f32", "bidirectional", 0, 0, 70, 136, "64x32", "1"),
    ("GRU", "f32", "forward", 0, 1, 20, 256, "32x16", "1"),
    ("RNN", "f32", "bidirectional", 1, 0, 33, 520, "64x64", "1"),
]


@pytest.mark.parametrize("cell,dtype,direction,layout,opt,B,H,tile,split", PERS_MFMA_CASES,
                         ids=["-".join(map(str, c)) for c in PERS_MFMA_CASES])
def test_persistent_matrix_step(cell, dtype, direction, layout, opt, B, H, tile, split, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    if tile:
        monkeypatch.setenv("RNN_MFMA_TILE", tile)
    if split:
        monkeypatch.setenv("RNN_F32_SPLIT", split)
    spec = LayerSpec(cell, seq=9, batch=B, input=40, hidden=H, direction=direction, layout=layout, dtype=dtype,
                     linear_before_reset=opt if cell == "GRU" else 0, input_forget=opt if cell == "LSTM" else 0,
                     init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM", clip=2.0,
                     outputs=("Y", "Y_h", "Y_c"))
    layer = rl.Layer(spec, engine="persistent", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
    inp = make_inputs(spec, 53, Dists(sequence_lens=("I", 0, 9), W=("U", -0.2, 0.2), R=("U", -0.1, 0.1)))
    check(spec, inp, engine="persistent", what=f"persistent mfma {cell}/{dtype}/{direction}/L{layout}/opt{opt}/"
                                                 f"B{B}/H{H}/{tile}/split{split}")


# The persistent matrix-core step with R resident in LDS (f16 mode, one
# phase per step): loaded once per layer, read in the same layout and order
# as the streamed chunks, so the outputs must be bit-identical to the
# streamed form (RNN_MFMA_RRES=0), and within the bar of the oracle.
RRES = [("LSTM", 0, 16, 64, 0, 1), ("LSTM", 1, 16, 200, 1, 0), ("GRU", 1, 32, 96, 0, 1), ("RNN", 0, 20, 1000, 1, 0),
        ("LSTM", 1, 40, 136, 0, 1)]


@pytest.mark.parametrize("cell,opt,B,H,layout,bidir", RRES, ids=[f"{c}-{o}-B{b}-H{h}-L{l}-{d}" for c, o, b, h, l, d in RRES])
def test_persistent_matrix_step_resident_r(cell, opt, B, H, layout, bidir, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=7, batch=B, input=24, hidden=H, direction="bidirectional" if bidir else "forward",
                     layout=layout, dtype="f16", linear_before_reset=opt if cell == "GRU" else 0,
                     input_forget=opt if cell == "LSTM" else 0, init_h=True, init_c=cell == "LSTM", lens=True,
                     peephole=cell == "LSTM", clip=2.0, outputs=("Y", "Y_h", "Y_c"))
    layer = rl.Layer(spec, engine="persistent", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
    inp = make_inputs(spec, 71, Dists(sequence_lens=("I", 0, 7), W=("U", -0.2, 0.2), R=("U", -0.1, 0.1)))
    note(f"case resident R {cell}/opt{opt}/B{B}/H{H}/L{layout}/bidir{bidir}")
    got = check(spec, inp, engine="persistent", what=f"resident R {cell} B{B} H{H}")
    res = gpu_layer(spec, inp, engine="persistent")
    monkeypatch.setenv("RNN_MFMA_RRES", "0")
    streamed = gpu_layer(spec, inp, engine="persistent")
    for n in res:
        assert np.array_equal(res[n].view(np.uint8), streamed[n].view(np.uint8)), f"{n}: resident R differs"


# The persistent matrix-core step's fallback (its grid not all running at
# once, forced with RNN_PERSISTENT_FALLBACK = k): the workgroups that arrived
# take the groups of tiles (one batch tile of one direction each) and run
# every tile of a group in turn through the same tile body.  Every mode: f16
# with split h (resident R and streamed R, both GRU forms), f32, and f32 on
# the bf16 matrix cores.  Bit-identical to the fast path.
MFALL = [("LSTM", 1, "f16", 0, None), ("GRU", 0, "f16", 1, None), ("GRU", 1, "f16", 0, None),
         ("RNN", 0, "f32", 0, None), ("LSTM", 0, "f32", 1, "1"), ("LSTM", 0, "f16", 1, None)]


@pytest.mark.parametrize("cell,opt,dtype,layout,split", MFALL,
                         ids=[f"{c}-{o}-{d}-L{l}-split{s}" for c, o, d, l, s in MFALL])
@pytest.mark.parametrize("forced", ["1", "2"])
def test_persistent_matrix_step_fallback(cell, opt, dtype, layout, split, forced, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    if split is not None:
        monkeypatch.setenv("RNN_F32_SPLIT", split)
    spec = LayerSpec(cell, seq=6, batch=20, input=24, hidden=40, direction="bidirectional", layout=layout,
                     dtype=dtype, linear_before_reset=opt if cell == "GRU" else 0,
                     input_forget=opt if cell == "LSTM" else 0, init_h=True, init_c=cell == "LSTM", lens=True,
                     peephole=cell == "LSTM", clip=2.0, outputs=("Y", "Y_h", "Y_c"))
    layer = rl.Layer(spec, engine="persistent", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
    inp = make_inputs(spec, 83, Dists(sequence_lens=("I", 0, 6), W=("U", -0.2, 0.2), R=("U", -0.1, 0.1)))
    note(f"case matrix-core fallback {forced} {cell}/opt{opt}/{dtype}/L{layout}/split{split}")
    fast = check(spec, inp, engine="persistent", what=f"matrix-core fast {cell}")
    fast = gpu_layer(spec, inp, layer=layer)
    assert layer.run_status().fallback_workgroups == 0
    monkeypatch.setenv("RNN_PERSISTENT_FALLBACK", forced)
    slow = gpu_layer(spec, inp, layer=layer)
    run = layer.run_status()
    assert run.persistent == 1 and run.fallback_workgroups == int(forced) and run.timed_out == 0
    for n in fast:
        assert np.array_equal(fast[n].view(np.uint8), slow[n].view(np.uint8)), f"fallback {forced} {cell} {n}: bits differ"


def test_large_batch_general_activations():
    """The matrix-core step kernel with non-default activations (f16 tensors
    then take the f32 path, f32 tensors always do)."""
    for cell, acts in (("LSTM", (("HardSigmoid", 0.2, 0.5), ("Softsign", 0, 0), ("Elu", 0.9, 0))),
                       ("GRU", (("Sigmoid", 0, 0), ("LeakyRelu", 0.05, 0))),
                       ("RNN", (("Relu", 0, 0),))):
        for dtype in ("f16", "f32"):
            spec = LayerSpec(cell, seq=6, batch=33, input=20, hidden=48, direction="bidirectional", dtype=dtype,
                             acts=acts, init_h=True, lens=True, linear_before_reset=1 if cell == "GRU" else 0)
            check(spec, make_inputs(spec, 29, Dists(sequence_lens=("I", 0, 6))), engine="launch",
                  what=f"large general acts {cell} {dtype}")


ALL_ACTS = [("Relu", 0, 0), ("Tanh", 0, 0), ("Sigmoid", 0, 0), ("Affine", 0.7, -0.2), ("LeakyRelu", 0.03, 0),
            ("ThresholdedRelu", 0.2, 0), ("ScaledTanh", 1.5, 0.5), ("HardSigmoid", 0.2, 0.5), ("Elu", 0.8, 0),
            ("Softsign", 0, 0), ("Softplus", 0, 0)]


# A plain RNN cell on tiles with several elements per thread (64x64 and
# 32x16 tiles, forced) takes, in the one-launch-per-step kernel, an epilogue
# loop compiled for its activation kind, and with hidden a multiple of 4 its
# four-units-per-thread form (vector stores of h, its halves and Y): every
# kind, in each direction, in the f32 matrix-core mode and the bf16 split
# mode, f32 and f16 tensors, ragged batch, hidden not a multiple of 4, and Y
# and Y_h at odd element offsets (no vector store of Y).
RNN_TILE_ACTS = [(k, ALL_ACTS[k], ALL_ACTS[(k + 5) % len(ALL_ACTS)]) for k in range(len(ALL_ACTS))]


@pytest.mark.parametrize("k,fwd,rev", RNN_TILE_ACTS, ids=[f"{a[0]}-{b[0]}" for _, a, b in RNN_TILE_ACTS])
def test_rnn_large_tile_activations(k, fwd, rev, monkeypatch):
    monkeypatch.setenv("RNN_MFMA_TILE", "64x64" if k % 2 == 0 else "32x16")
    monkeypatch.setenv("RNN_F32_SPLIT", "1" if k % 3 == 0 else "0")
    hidden = (100, 92, 98)[k % 3]
    dtype = "f16" if k % 4 == 3 else "f32"
    spec = LayerSpec("RNN", seq=5, batch=70, input=24, hidden=hidden, direction="bidirectional", dtype=dtype,
                     acts=(fwd, rev), init_h=True, lens=True, clip=3.0 if k % 4 == 1 else None,
                     outputs=("Y", "Y_h"))
    inp = make_inputs(spec, 61 + k, Dists(sequence_lens=("I", 0, 5), W=("U", -0.3, 0.3), R=("U", -0.2, 0.2)))
    offsets = {"Y": 3, "Y_h": 5} if k % 5 == 2 else None
    check(spec, inp, engine="launch", offsets=offsets, what=f"RNN large tile {fwd[0]}/{rev[0]} {dtype} H{hidden}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("cell", ["LSTM", "GRU", "RNN"])
def test_every_activation_in_every_slot(cell, engine):
    slots = synth.SLOTS[cell]
    for i, act in enumerate(ALL_ACTS):
        for slot in range(2 * slots):
            acts = list(synth.DEFAULT_ACTS[cell]) * 2
            acts[slot] = act
            acts[(slot + 3) % (2 * slots)] = ALL_ACTS[(i + 5) % len(ALL_ACTS)]
            spec = LayerSpec(cell, seq=4, batch=3, input=5, hidden=19, direction="bidirectional", acts=acts,
                             init_h=True, dtype="f32" if (i + slot) % 2 == 0 else "f16",
                             linear_before_reset=slot % 2 if cell == "GRU" else 0)
            check(spec, make_inputs(spec, 100 + i), engine=engine, twice=False,
                  what=f"{cell} act {act[0]} slot {slot}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_odd_offsets_with_sentinels(dtype, engine):
    offs = {n: 3 for n in ("X", "W", "R", "B", "sequence_lens", "initial_h", "initial_c", "P", "Y", "Y_h", "Y_c")}
    for cell in ("LSTM", "GRU", "RNN"):
        spec = LayerSpec(cell, seq=5, batch=3, input=7, hidden=13, direction="bidirectional", dtype=dtype,
                         init_h=True, init_c=cell == "LSTM", peephole=cell == "LSTM", lens=True)
        inp = make_inputs(spec, 7)
        check(spec, inp, engine=engine, offsets={k: v for k, v in offs.items() if k in inp or k.startswith("Y")},
              what=f"offsets {cell} {dtype}")


@pytest.mark.parametrize("engine", ENGINES)
def test_empty_sequence_and_batch(engine):
    for cell in ("LSTM", "GRU", "RNN"):
        spec = LayerSpec(cell, seq=0, batch=3, input=4, hidden=5, init_h=True, init_c=cell == "LSTM",
                         direction="bidirectional")
        inp = make_inputs(spec, 3)
        got = gpu_layer(spec, inp, engine=engine)
        ref = oracle.run(spec, inp)
        compare(spec, got, ref, what=f"seq0 {cell}")
        spec = LayerSpec(cell, seq=4, batch=0, input=4, hidden=5)
        got = gpu_layer(spec, make_inputs(spec, 3), engine=engine)
        for v in got.values():
            assert v.size == 0


@pytest.mark.parametrize("engine", ENGINES)
def test_lengths_edge_cases_and_max_length(engine):
    for cell in ("LSTM", "GRU", "RNN"):
        spec = LayerSpec(cell, seq=6, batch=5, input=4, hidden=9, direction="bidirectional", init_h=True,
                         init_c=cell == "LSTM", lens=True)
        inp = make_inputs(spec, 9)
        inp["sequence_lens"] = np.array([0, 6, 3, 17, -2], np.int32)  # > Seq acts as Seq; < 0 as 0
        check(spec, inp, engine=engine, what=f"lens edges {cell}")
        inp["sequence_lens"] = np.array([0, 4, 3, 1, 2], np.int32)
        check(spec.replace(max_length=4), inp, engine=engine, what=f"max_length {cell}")


# MaxLength ("Recurrent layers" page: a host-side bound on the sequence
# lengths that shortens the step loop) below some rows' lengths, and below
# Seq with no lengths at all, on every step engine: the vector-ALU persistent
# engine, one launch per step, the matrix-core step (18 rows, f32) and its
# persistent form (16 rows, f16, default activations).
MAXLEN_CASES = [("launch", 5, "f32", None), ("persistent", 5, "f32", None), ("auto", 18, "f32", None),
                ("persistent", 16, "f16", "default")]


@pytest.mark.parametrize("engine,B,dtype,acts", MAXLEN_CASES, ids=[f"{e}-B{b}-{d}" for e, b, d, _ in MAXLEN_CASES])
def test_max_length_cuts_rows(engine, B, dtype, acts):
    for cell in ("LSTM", "GRU", "RNN"):
        for lbr in ((0, 1) if cell == "GRU" else (0,)):
            spec = LayerSpec(cell, seq=6, batch=B, input=12, hidden=48, direction="bidirectional", dtype=dtype,
                             init_h=True, init_c=cell == "LSTM", lens=True, linear_before_reset=lbr, max_length=4)
            inp = make_inputs(spec, 13)
            lens = np.array([6, 0, 5, 17, -2, 4, 3, 1] * 3, np.int32)[:B]   # rows above, at and below 4
            inp["sequence_lens"] = lens
            check(spec, inp, engine=engine, what=f"max_length 4 rows cut {cell} lbr{lbr}")
            nolens = spec.replace(lens=False)
            inp.pop("sequence_lens")
            check(nolens, inp, engine=engine, what=f"max_length 4 < Seq 6 without lengths {cell} lbr{lbr}")


# f16 outputs are rounded to nearest even once ("How a layer runs", item 4).
# With W = R = 0 and Affine activations, a unit's output is exactly the f32
# sum Wb + Rb (forward, alpha 1) or half of it (reverse, alpha 0.5); the bias
# pairs put that value on ties between binary16 neighbours (both parities),
# just off them, past the largest finite value, in the subnormal range and at
# its edge.  Every output must carry exactly the bits of the oracle's
# round-to-nearest-even of the same value.
_HALF_PAIRS = [(1.0, 2.0 ** -11), (1.0 + 2.0 ** -10, 2.0 ** -11), (1.0, 2.0 ** -12), (1.0, 3 * 2.0 ** -12),
               (65504.0, 16.0), (65504.0, 16.0 - 2.0 ** -7), (-1.0, -(2.0 ** -11)), (3 * 2.0 ** -24, 0.0),
               (2.0 ** -24, 0.0), (2.0 ** -14, -(2.0 ** -24)), (2048.0, 1.0), (2048.0, 3.0), (-65504.0, -32.0),
               (0.0, -0.0), (-(2.0 ** -24), 0.0)]


def _half_bias_pairs(n_random, seed):
    rng = np.random.default_rng(seed)
    pairs = list(_HALF_PAIRS)
    # random pairs within eleven binades, so that their sum is exact in f32
    mag = rng.uniform(-8, 2, size=(n_random, 2))
    v = (np.sign(rng.uniform(-1, 1, size=(n_random, 2))) * 2.0 ** mag).astype(np.float16).astype(np.float64)
    pairs += [tuple(r) for r in v]
    return np.array(pairs, np.float64)


@pytest.mark.parametrize("engine,B,layout", [("persistent", 1, 0), ("launch", 3, 1), ("auto", 16, 0)])
def test_f16_outputs_round_to_nearest_even(engine, B, layout):
    pairs = _half_bias_pairs(49, 5)
    H = len(pairs)
    spec = LayerSpec("RNN", seq=3, batch=B, input=7, hidden=H, direction="bidirectional", layout=layout,
                     dtype="f16", acts=(("Affine", 1.0, 0.0), ("Affine", 0.5, 0.0)), outputs=("Y", "Y_h"))
    inp = make_inputs(spec, 3)
    inp["W"] = np.zeros_like(inp["W"])
    inp["R"] = np.zeros_like(inp["R"])
    bias = np.concatenate([pairs[:, 0], pairs[:, 1]]).astype(np.float16)
    assert np.array_equal(bias.astype(np.float64), np.concatenate([pairs[:, 0], pairs[:, 1]])), "pairs not in f16"
    inp["B"] = np.stack([bias, bias])
    note(f"case f16 rounding engine={engine} B={B} L{layout} H={H}")
    got = gpu_layer(spec, inp, engine=engine)
    ref = oracle.run(spec, inp, outputs=spec.outputs)
    for n in ("Y", "Y_h"):
        want = oracle.round_half(ref[n])
        have = got[n].view(np.uint16)
        bad = np.argwhere(have != want)
        assert bad.size == 0, (f"{n}{tuple(bad[0])}: value {ref[n][tuple(bad[0])]!r} gave bits "
                               f"{have[tuple(bad[0])]:#06x}, nearest-even is {want[tuple(bad[0])]:#06x}")


# Batches of 9 to 15 run on the matrix-core step with one 16-row block whose
# rows past the batch read as zeros: every cell and GRU form, both dtypes,
# lengths with 0, peepholes, clip, input_forget; the automatic choice (the
# persistent form for these small layers) and one launch per step.
B9 = [(c, o, dt, b) for c, o in (("LSTM", 0), ("LSTM", 1), ("GRU", 0), ("GRU", 1), ("RNN", 0))
      for dt in ("f32", "f16") for b in (9, 15)]


@pytest.mark.parametrize("cell,opt,dtype,B", B9, ids=[f"{c}-{o}-{d}-B{b}" for c, o, d, b in B9])
def test_batches_nine_to_fifteen(cell, opt, dtype, B):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=9, batch=B, input=40, hidden=64, direction="bidirectional", layout=opt, dtype=dtype,
                     linear_before_reset=opt if cell == "GRU" else 0, input_forget=opt if cell == "LSTM" else 0,
                     init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM", clip=2.5,
                     outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 113, Dists(sequence_lens=("I", 0, 9), W=("U", -0.2, 0.2), R=("U", -0.2, 0.2)))
    layer = rl.Layer(spec, engine="auto", device="cuda:0")
    assert rl.PRODUCTS[layer.plan.step_products] != "f32 vector ALU"
    for engine in ("auto", "launch"):
        check(spec, inp, engine=engine, what=f"B{B} {cell} opt{opt} {dtype} {engine}")


@pytest.mark.parametrize("engine", ENGINES)
def test_batch_above_eight_and_hidden_not_dividing(engine):
    for cell, H in (("LSTM", 65), ("GRU", 127), ("RNN", 129)):
        spec = LayerSpec(cell, seq=5, batch=19 if engine == "launch" else 8, input=31, hidden=H,
                         direction="bidirectional", init_h=True, lens=True, linear_before_reset=0)
        check(spec, make_inputs(spec, 21), engine=engine, what=f"B{spec.batch} H{H} {cell}")


# ---------------------------------------------------------------------------
# the five seeded workloads at full size
# ---------------------------------------------------------------------------
FULL = [("C1", {}), ("C2", {}), ("C3", {"linear_before_reset": 0}), ("C3", {"linear_before_reset": 1}),
        ("C4", {}), ("C5", {}), ("C4", {"engine": "launch"}), ("C5", {"engine": "persistent"})]
# one row in each batch tile of the step kernels (C4: 16-row tiles; C5:
# 64-row tiles), every unit of each sampled row
SAMPLE_ROWS = {"C4": [0, 21, 42, 63], "C5": [0, 100, 170, 255]}


# The recognizer shapes of the "Recurrent layers" page: both layer shapes,
# both tensor types, every engine, both layouts, with every operand and output
# at an odd element offset and sentinels around every output (H = 96 does not
# divide the persistent engine's 32-wide padding nor the 64-unit tiles).
REC_CASES = [(n, dt, e, lay) for n in ("REC80", "REC48") for dt in ("f32", "f16")
             for e in ("auto", "launch", "persistent") for lay in (0, 1)]


@pytest.mark.parametrize("name,dtype,engine,layout", REC_CASES, ids=["-".join(map(str, c)) for c in REC_CASES])
def test_recognizer_shapes(name, dtype, engine, layout):
    spec, inp = synth.config(name, dtype=dtype, layout=layout)
    offs = {n: 5 for n in list(inp) + list(spec.outputs)}
    check(spec, inp, engine=engine, offsets=offs, what=f"recognizer {name} {dtype} L{layout}")


def test_engine_choice_and_plan():
    import onnx_recurrent_layers_amd as rl
    for name in ("C1", "C2", "C3"):
        spec, _ = synth.config(name)
        layer = rl.Layer(spec, engine="auto", device="cuda:0")
        assert layer.plan.engine == rl.ENGINES["persistent"], name
        assert layer.plan.step_launches == 1
    # C4 (f16, split h): the matrix-core step in one persistent launch; C5
    # (f32): one launch per step, unless the persistent engine is asked for
    spec, _ = synth.config("C4")
    layer = rl.Layer(spec, engine="auto", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"]
    assert layer.plan.step_launches == 1 and layer.plan.step_blocks == 256
    spec, _ = synth.config("C5")
    layer = rl.Layer(spec, engine="auto", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["launch"] and layer.plan.step_launches == 1024
    layer = rl.Layer(spec, engine="persistent", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_blocks == 256


@pytest.mark.parametrize("name,over", FULL + [("C2", {"engine": "launch"}), ("C3", {"engine": "launch"})],
                         ids=[f"{n}-{o}" for n, o in FULL + [("C2", {"engine": "launch"}), ("C3", {"engine": "launch"})]])
def test_full_config(name, over):
    over = dict(over)
    engine = over.pop("engine", "auto")
    spec, inp = synth.config(name, **over)
    note(f"case {name} {over} engine={engine}")
    got = gpu_layer(spec, inp, engine=engine)
    again = gpu_layer(spec, inp, engine=engine)
    for n in got:
        assert np.array_equal(got[n].view(np.uint8), again[n].view(np.uint8)), f"{name} {n}: runs differ"
    rows = SAMPLE_ROWS.get(name)
    if rows is None:
        ref = oracle.run(spec, inp, outputs=spec.outputs)
        rep = compare(spec, got, ref, what=name)
    else:
        ref = oracle_rows(spec, inp, rows, outputs=spec.outputs)
        rep = compare(spec, select_rows(spec, got, rows), ref, what=name)
    note(f"{name} {over}: " + ", ".join(f"{k} abs {v[0]:.3g} scaled {v[1]:.3g}" for k, v in rep.items()))


# ---------------------------------------------------------------------------
# stacked layers and streaming continuation
# ---------------------------------------------------------------------------
def test_stacked_layers_without_transpose():
    """A bidirectional layout-1 layer's Y [B, S, 2, H] is the next layer's X
    [B, S, 2H] as it lies in memory: the second layer reads the first one's
    output buffer in place, no transpose and no copy."""
    import onnx_recurrent_layers_amd as rl
    B, S, H1 = 3, 9, 12
    s1 = LayerSpec("LSTM", seq=S, batch=B, input=10, hidden=H1, direction="bidirectional", layout=1, dtype="f32",
                   init_h=True, init_c=True, peephole=True, outputs=("Y",))
    in1 = make_inputs(s1, 91)
    y1 = rl.run(s1, in1, engine="persistent", outputs=("Y",))["Y"]
    assert tuple(y1.shape) == (B, S, 2, H1)
    compare(s1, {"Y": y1.cpu().numpy()}, oracle.run(s1, in1, outputs=("Y",)), what="stacked layer 1")
    for engine in ("persistent", "launch"):
        s2 = LayerSpec("GRU", seq=S, batch=B, input=2 * H1, hidden=8, direction="bidirectional", layout=1,
                       dtype="f32", linear_before_reset=1, outputs=("Y", "Y_h"))
        in2 = make_inputs(s2, 92)
        dev = rl.to_device({k: v for k, v in in2.items() if k != "X"})
        dev["X"] = y1.view(B, S, 2 * H1)   # the first layer's output, read in place
        got = rl.run(s2, dev, engine=engine, outputs=s2.outputs)
        ref = oracle.run(s2, {**in2, "X": y1.view(B, S, 2 * H1).cpu().numpy()}, outputs=s2.outputs)
        compare(s2, {k: v.cpu().numpy() for k, v in got.items()}, ref, what=f"stacked layer 2 {engine}")


# Two stacked bidirectional layout-0 layers (the recognizer's stack): the
# second reads the first's Y [S, 2, B, H'] in place as its X [S, B, 2H'], each
# row gathered by the projection from two pieces (x_bidirectional_y = 1).
# Cases reach every projection kernel (small layers, 64/128 tiles, the
# 256x256 direct-to-LDS tiles in f16 and in bf16-split f32, the
# register-staged bf16 split kernel) and the element-wise path (H' not a
# whole number of 16-byte segments).  Checked against the oracle fed the
# first layer's Y transposed on the host, and bit for bit against the same
# second layer run on that transposed copy.
STACK0 = [("f32", 48, 5, {}), ("f16", 48, 5, {}), ("f32", 37, 5, {}), ("f16", 37, 3, {}),
          ("f16", 64, 8, {"RNN_SMALL_PROJECTION": "0"}), ("f32", 36, 7, {"RNN_SMALL_PROJECTION": "0"}),
          ("f16", 64, 8, {"RNN_PROJ_LDS_MIN_TILES": "1"}),
          ("f32", 64, 8, {"RNN_F32_SPLIT": "1", "RNN_PROJ_LDS_MIN_TILES": "1"}),
          ("f32", 64, 8, {"RNN_F32_SPLIT": "1", "RNN_PROJ_LDS_MIN_TILES": "1000000000"}),
          ("f32", 40, 1, {})]


@pytest.mark.parametrize("dtype,H1,B,env", STACK0, ids=[f"{d}-H{h}-B{b}-{'-'.join(e) or 'auto'}"
                                                       for d, h, b, e in STACK0])
def test_stacked_bidirectional_layout0(dtype, H1, B, env, monkeypatch):
    import torch
    import onnx_recurrent_layers_amd as rl
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    S = 11
    s1 = LayerSpec("LSTM", seq=S, batch=B, input=20, hidden=H1, direction="bidirectional", layout=0, dtype=dtype,
                   init_h=True, init_c=True, lens=True, outputs=("Y",))
    in1 = make_inputs(s1, 95, Dists(sequence_lens=("I", 1, S)))
    y1 = rl.run(s1, in1, outputs=("Y",))["Y"]
    assert tuple(y1.shape) == (S, 2, B, H1)
    compare(s1, {"Y": y1.cpu().numpy()}, oracle.run(s1, in1, outputs=("Y",)), what="stacked layer 1")
    xt = y1.permute(0, 2, 1, 3).contiguous().view(S, B, 2 * H1)   # the same values as one X row each
    for cell in ("LSTM", "GRU"):
        s2 = LayerSpec(cell, seq=S, batch=B, input=2 * H1, hidden=24, direction="bidirectional", layout=0,
                       dtype=dtype, init_h=True, init_c=cell == "LSTM", lens=True, outputs=("Y", "Y_h"))
        in2 = make_inputs(s2, 96)
        in2["sequence_lens"] = in1["sequence_lens"]
        dev = rl.to_device({k: v for k, v in in2.items() if k != "X"})
        note(f"case stacked layout 0 {cell} {dtype} H'={H1} B={B} {env}")
        got = rl.run(s2.replace(x_bidirectional_y=1), {**dev, "X": y1}, outputs=s2.outputs)   # Y read in place
        ref = oracle.run(s2, {**in2, "X": xt.cpu().numpy()}, outputs=s2.outputs)
        compare(s2, {k: v.cpu().numpy() for k, v in got.items()}, ref, what=f"stacked layer 2 {cell}")
        plain = rl.run(s2, {**dev, "X": xt}, outputs=s2.outputs)
        for n in got:
            assert torch.equal(got[n].view(torch.int16 if dtype == "f16" else torch.int32),
                               plain[n].view(torch.int16 if dtype == "f16" else torch.int32)), f"{cell} {n}: bits differ"


def test_bidirectional_y_flag_is_a_no_op_in_layout_1():
    """Layout 1: Y [B, S, 2, H'] is X [B, S, 2H'] already; x_bidirectional_y = 1
    reads it exactly as a plain X."""
    import torch
    import onnx_recurrent_layers_amd as rl
    s2 = LayerSpec("GRU", seq=6, batch=4, input=30, hidden=16, direction="bidirectional", layout=1, dtype="f32",
                   init_h=True, outputs=("Y", "Y_h"))
    inp = make_inputs(s2, 97)
    a = rl.run(s2.replace(x_bidirectional_y=1), inp, outputs=s2.outputs)
    b = rl.run(s2, inp, outputs=s2.outputs)
    for n in a:
        assert torch.equal(a[n].view(torch.int32), b[n].view(torch.int32)), n


@pytest.mark.parametrize("cell,engine", [("LSTM", "persistent"), ("GRU", "launch"), ("RNN", "persistent"),
                                         ("LSTM", "launch")])
def test_streaming_continuation(cell, engine):
    """A sequence run in two pieces, the second starting from the first's
    Y_h (and Y_c), gives the same bits as one run over the whole sequence: the
    projection of a row and the arithmetic of a step do not depend on the
    sequence length, and f32 final states carry the state exactly."""
    import torch
    import onnx_recurrent_layers_amd as rl
    S1, S2, B = 5, 7, 4 if engine == "persistent" else 19
    lstm = cell == "LSTM"
    outs = ("Y", "Y_h", "Y_c") if lstm else ("Y", "Y_h")

    def spec(seq):
        return LayerSpec(cell, seq=seq, batch=B, input=11, hidden=20, direction="forward", layout=0, dtype="f32",
                         init_h=True, init_c=lstm, peephole=lstm, clip=3.0, outputs=outs)

    full = spec(S1 + S2)
    inp = make_inputs(full, 93)
    rf = rl.run(full, inp, engine=engine, outputs=outs)
    compare(full, {k: v.cpu().numpy() for k, v in rf.items()}, oracle.run(full, inp, outputs=outs),
            what=f"continuation reference {cell}")
    ra = rl.run(spec(S1), {**inp, "X": inp["X"][:S1]}, engine=engine, outputs=outs)
    inb = {**inp, "X": inp["X"][S1:], "initial_h": ra["Y_h"].cpu().numpy()}
    if lstm:
        inb["initial_c"] = ra["Y_c"].cpu().numpy()
    rb = rl.run(spec(S2), inb, engine=engine, outputs=outs)
    y = torch.cat([ra["Y"], rb["Y"]], dim=0)
    assert torch.equal(y.view(torch.int32), rf["Y"].view(torch.int32)), f"{cell}: Y differs"
    for n in outs[1:]:
        assert torch.equal(rb[n].view(torch.int32), rf[n].view(torch.int32)), f"{cell}: {n} differs"


# The persistent engine's units per workgroup, set with RNN_PERSISTENT_UNITS
# (the tuning switch): every choice is the same layer, spread over a
# different number of workgroups.
UNITS = [("LSTM", "f32", 1, 40, (1, 3, 8)), ("GRU", "f16", 5, 72, (2, 12)), ("RNN", "f32", 8, 100, (1, 8))]


@pytest.mark.parametrize("cell,dtype,B,H,units", UNITS, ids=[f"{c}-{d}-B{b}-H{h}" for c, d, b, h, _ in UNITS])
def test_persistent_units_per_workgroup(cell, dtype, B, H, units, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=9, batch=B, input=24, hidden=H, direction="bidirectional", dtype=dtype,
                     init_h=True, init_c=cell == "LSTM", lens=True, outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 83, Dists(sequence_lens=("I", 0, 9)))
    blocks = set()
    for u in units:
        monkeypatch.setenv("RNN_PERSISTENT_UNITS", str(u))
        layer = rl.Layer(spec, engine="persistent", device="cuda:0")
        assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
        blocks.add(layer.plan.step_blocks)
        note(f"case persistent units {u} {cell} {dtype} B{B} H{H} blocks {layer.plan.step_blocks}")
        check(spec, inp, engine="persistent", what=f"units {u} {cell} {dtype} B{B} H{H}")
    assert len(blocks) == len(units), blocks       # each choice spreads the layer differently


# Both persistent kernels launched with the cooperative API
# (RNN_COOPERATIVE_LAUNCH = 1) instead of the plain launch with the
# workgroups' own residency decision: the same kernels and arithmetic, so the
# outputs are bit-identical to the plain launch and within the oracle's bar.
COOP = [("LSTM", "f32", 1, 40), ("GRU", "f16", 3, 64), ("LSTM", "f16", 16, 64)]


@pytest.mark.parametrize("cell,dtype,B,H", COOP, ids=[f"{c}-{d}-B{b}-H{h}" for c, d, b, h in COOP])
def test_cooperative_launch(cell, dtype, B, H, monkeypatch):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=8, batch=B, input=24, hidden=H, direction="bidirectional", dtype=dtype,
                     init_h=True, init_c=cell == "LSTM", lens=True, peephole=cell == "LSTM",
                     outputs=("Y", "Y_h", "Y_c"))
    inp = make_inputs(spec, 89, Dists(sequence_lens=("I", 0, 8), W=("U", -0.2, 0.2), R=("U", -0.1, 0.1)))
    layer = rl.Layer(spec, engine="persistent", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
    plain = gpu_layer(spec, inp, engine="persistent")
    monkeypatch.setenv("RNN_COOPERATIVE_LAUNCH", "1")
    note(f"case cooperative launch {cell} {dtype} B{B} H{H}")
    check(spec, inp, engine="persistent", what=f"cooperative {cell} {dtype} B{B} H{H}")
    coop = gpu_layer(spec, inp, engine="persistent")
    for n in plain:
        assert np.array_equal(plain[n].view(np.uint8), coop[n].view(np.uint8)), f"{n}: cooperative launch differs"


# The largest hidden sizes the persistent engine takes (one more unit and the
# automatic choice is one launch per step): every compute unit or nearly
# every one holds a slice of R, and the layer is still exact.
LARGEST = [("LSTM", "f32", 1, 1088), ("LSTM", "f16", 8, 1024), ("GRU", "f32", 4, 1184), ("RNN", "f32", 1, 2176)]


@pytest.mark.parametrize("cell,dtype,B,H", LARGEST, ids=[f"{c}-{d}-B{b}-H{h}" for c, d, b, h in LARGEST])
def test_persistent_largest_shapes(cell, dtype, B, H):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=6, batch=B, input=40, hidden=H, direction="bidirectional", dtype=dtype,
                     init_h=True, init_c=cell == "LSTM", lens=B > 1, outputs=("Y", "Y_h", "Y_c"))
    layer = rl.Layer(spec, engine="auto", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
    bigger = rl.Layer(spec.replace(hidden=H + 1), engine="auto", device="cuda:0")
    assert bigger.plan.engine == rl.ENGINES["launch"]
    s = 1.0 / np.sqrt(H)
    inp = make_inputs(spec, 97, Dists(W=("U", -s, s), R=("U", -s, s), sequence_lens=("I", 1, 6)))
    note(f"case persistent largest {cell} {dtype} B{B} H{H} blocks {layer.plan.step_blocks}")
    check(spec, inp, engine="auto", what=f"largest persistent {cell} {dtype} B{B} H{H}")


# The persistent matrix-core step at its largest sizes (batches of 16 and
# more, f16): hidden 4096 with R streamed, and the last hidden size before
# the automatic choice turns to one launch per step for a GRU of batch 32.
MLARGEST = [("LSTM", 16, 4096, "forward", False), ("RNN", 16, 4096, "bidirectional", False),
            ("GRU", 32, 1024, "bidirectional", True)]


@pytest.mark.parametrize("cell,B,H,direction,edge", MLARGEST, ids=[f"{c}-B{b}-H{h}" for c, b, h, _, _ in MLARGEST])
def test_persistent_matrix_step_largest_shapes(cell, B, H, direction, edge):
    import onnx_recurrent_layers_amd as rl
    spec = LayerSpec(cell, seq=3, batch=B, input=40, hidden=H, direction=direction, dtype="f16",
                     init_h=True, init_c=cell == "LSTM", lens=True, outputs=("Y", "Y_h", "Y_c"))
    layer = rl.Layer(spec, engine="auto", device="cuda:0")
    assert layer.plan.engine == rl.ENGINES["persistent"] and layer.plan.step_launches == 1
    if edge:
        assert rl.Layer(spec.replace(hidden=H + 8), engine="auto", device="cuda:0").plan.engine == rl.ENGINES["launch"]
    s = 1.0 / np.sqrt(H)
    inp = make_inputs(spec, 101, Dists(W=("U", -s, s), R=("U", -s, s), sequence_lens=("I", 1, 3)))
    note(f"case persistent matrix-core largest {cell} B{B} H{H} blocks {layer.plan.step_blocks}")
    check(spec, inp, engine="auto", what=f"largest persistent matrix-core {cell} B{B} H{H}")

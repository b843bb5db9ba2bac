"""GPU-side test harness: run a layer through the C ABI with sentinels around
every tensor, and compare against the CPU oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

import onnx_recurrent_layers_amd as rl
from oracle import oracle

SENTINEL = -777.0          # exact in f16 and f32
ABS_TOL = {"f32": 1e-4, "f16": 5e-3}


def note(msg: str):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def gpu_layer(spec, inputs, engine="auto", offsets=None, outputs=None, layer=None, return_layer=False):
    """Run on cuda:0.  Every input/output sits at its element offset inside a
    larger buffer; output padding holds SENTINEL and is checked afterwards."""
    import torch
    dev = torch.device("cuda", 0)
    dt = torch.float32 if spec.dtype == "f32" else torch.float16
    offs = dict(offsets or {})
    tens = {}
    for k, v in inputs.items():
        off = offs.get(k, 0)
        flat = torch.from_numpy(np.ascontiguousarray(v).reshape(-1))
        buf = torch.zeros(flat.numel() + off + 5, dtype=flat.dtype)
        buf[off:off + flat.numel()] = flat
        tens[k] = buf.to(dev)
    shapes = rl.output_shapes(spec)
    want = outputs if outputs is not None else spec.outputs
    outs = {}
    for n in want:
        if n == "Y_c" and spec.cell != "LSTM":
            continue
        numel = int(np.prod(shapes[n]))
        off = offs.get(n, 0)
        buf = torch.full((numel + off + 7,), SENTINEL, dtype=dt, device=dev)
        outs[n] = (buf, off, numel, shapes[n])
    if layer is None:
        layer = rl.Layer(spec, engine=engine, device="cuda:0")
    layer.encode({**tens, **{n: o[0] for n, o in outs.items()}}, offsets=offs)
    torch.cuda.synchronize()
    # a persistent step kernel must never end on its safety bound, and takes
    # its fallback only when a test forces it
    run = layer.run_status()
    assert not run.timed_out, "a wait of the persistent step kernel passed its safety bound"
    if not os.environ.get("RNN_PERSISTENT_FALLBACK"):
        assert run.fallback_workgroups == 0, f"the fallback ran ({run.fallback_workgroups} workgroups)"
    res = {}
    for n, (buf, off, numel, shape) in outs.items():
        host = buf.cpu()
        pad = torch.cat([host[:off], host[off + numel:]])
        assert bool((pad == SENTINEL).all()), f"{n}: a value outside the output was written"
        res[n] = host[off:off + numel].view(shape).numpy()
    if return_layer:
        return res, layer
    return res


def compare(spec, got: dict, ref: dict, tol=None, what="", rows=None):
    """Max abs error per output within the tolerance; returns {name: (abs, scaled)}."""
    tol = tol if tol is not None else ABS_TOL[spec.dtype]
    report = {}
    for n, g in got.items():
        r = ref[n]
        if r is None:
            continue
        g64 = g.astype(np.float64)
        assert g64.shape == r.shape, (n, g64.shape, r.shape)
        err = np.abs(g64 - r)
        both_nan = np.isnan(g64) & np.isnan(r)
        err = np.where(both_nan, 0.0, err)
        m = float(np.max(err)) if err.size else 0.0
        scale = float(np.max(np.abs(np.where(np.isnan(r), 0.0, r)))) if r.size else 0.0
        report[n] = (m, m / scale if scale > 0 else m)
        assert not np.isnan(m) and m <= tol, f"{what} {n}: max abs error {m} > {tol}"
    return report


def oracle_rows(spec, inputs, rows, outputs=None):
    """Oracle on a subset of batch rows (rows are independent sequences)."""
    rows = list(rows)
    sub = dict(inputs)
    if spec.layout == 0:
        sub["X"] = inputs["X"][:, rows]
        for k in ("initial_h", "initial_c"):
            if k in inputs:
                sub[k] = inputs[k][:, rows]
    else:
        sub["X"] = inputs["X"][rows]
        for k in ("initial_h", "initial_c"):
            if k in inputs:
                sub[k] = inputs[k][rows]
    if "sequence_lens" in inputs:
        sub["sequence_lens"] = inputs["sequence_lens"][rows]
    s2 = spec.replace(batch=len(rows))
    return oracle.run(s2, sub, outputs=outputs)


def select_rows(spec, out: dict, rows):
    rows = list(rows)
    res = {}
    for n, v in out.items():
        if n == "Y":
            res[n] = v[:, :, rows] if spec.layout == 0 else v[rows]
        else:
            res[n] = v[:, rows] if spec.layout == 0 else v[rows]
    return res

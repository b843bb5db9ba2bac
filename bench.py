#!/usr/bin/env python3
"""Benchmark of one ONNX recurrent layer on one MI355X.

Default workload: bidirectional LSTM, seq 80, batch 1, input 256, hidden 256,
f32, layout 0 (the five seeded workloads are in onnx_recurrent_layers_amd.synth;
``--config`` picks another).  A step of this benchmark is one whole layer
(projection, state setup, every recurrent step, the outputs) through
``rnn_encode`` with inputs resident in device memory.

Prints one JSON line: timesteps/s (value), layer latency (ms_per_step), the
roofline of the dominant kernel (the recurrent-step kernel, timed with HIP
events recorded by the library at the stage boundaries on the layer's stream),
and the CPU oracle timed on the host on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "f32": 157.3}


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API."""

    def __init__(self, n: int):
        import onnx_recurrent_layers_amd as rl
        self.hip = rl.hip_runtime()
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev.append(e.value)

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


# Measured HBM traffic per launch of the step kernel on a workload, from two
# rocprofv3 counter runs (see each profile file); it is reported only while
# the kernel sources still hash to what was profiled.
TRAFFIC_PROFILES = {
    ("C2", "persistent"): os.path.join(ROOT, "profiles", "persistent_step_bilstm_s80_b1_h256_f32.md"),
    ("C4", "persistent"): os.path.join(ROOT, "profiles", "persistent_mfma_step_lstm_s256_b64_h1024_f16.md"),
    ("C5", "launch"): os.path.join(ROOT, "profiles", "mfma_step_rnn_s1024_b256_h2048_f32.md"),
}


def row_subset(spec, inputs, rows: int):
    """The first `rows` batch rows of a layer (rows are independent sequences)."""
    sub = dict(inputs)
    if spec.layout == 0:
        sub["X"] = inputs["X"][:, :rows]
        for k in ("initial_h", "initial_c"):
            if k in inputs:
                sub[k] = inputs[k][:, :rows]
    else:
        sub["X"] = inputs["X"][:rows]
        for k in ("initial_h", "initial_c"):
            if k in inputs:
                sub[k] = inputs[k][:rows]
    if "sequence_lens" in inputs:
        sub["sequence_lens"] = inputs["sequence_lens"][:rows]
    return spec.replace(batch=rows), sub


def profiled_traffic(path: str):
    import hashlib
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(ln.split(": ", 1) for ln in text.splitlines()
                  if ln.startswith(("traffic_bytes_per_launch", "kernel_sources_sha256_16", "kernel_sources")))
    try:
        h = hashlib.sha256()
        for f in fields["kernel_sources"].split(", "):
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] != fields["kernel_sources_sha256_16"].strip():
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, OSError, ValueError):
        return None


def step_bytes(spec) -> int:
    """Algorithmic bytes of one recurrent step (both directions): R once, the
    step's slice of Xw, the previous h read and the new h written (plus the
    cell state read and written for an LSTM)."""
    D, H, B = spec.num_directions, spec.hidden, spec.batch
    G = spec.gates - (1 if (spec.cell == "LSTM" and spec.input_forget) else 0)
    e = 4 if spec.dtype == "f32" else 2
    b = D * G * H * H * e + D * B * G * H * 4 + 2 * D * B * H * 4
    if spec.cell == "LSTM":
        b += 2 * D * B * H * 4
    return b


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed layer runs")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--engine", default="auto", choices=["auto", "launch", "persistent"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floors", action="store_true",
                    help="skip the step-floor layers (for profiler runs, whose kernel statistics then cover the "
                         "workload alone)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the layer, run a plain device copy of this many bytes (a known-size "
                         "kernel against which the HBM byte counters of a profiler are scaled)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library runs a layer on a single MI355X "
              "(see the design notes for how batch rows or directions would shard); use --gpus 1",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import onnx_recurrent_layers_amd as rl
    from onnx_recurrent_layers_amd import synth

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 3}))
        return 0

    spec, inputs = synth.config(args.config)
    name = synth.CONFIGS[args.config]["name"]
    dev = torch.device("cuda", 0)
    dt = torch.float32 if spec.dtype == "f32" else torch.float16
    tens = rl.to_device(inputs, "cuda:0")
    shapes = rl.output_shapes(spec)
    outs = {n: torch.empty(shapes[n], dtype=dt, device=dev) for n in spec.outputs
            if not (n == "Y_c" and spec.cell != "LSTM")}
    layer = rl.Layer(spec, engine=args.engine, device="cuda:0")
    plan = layer.plan
    engine_name = {v: k for k, v in rl.ENGINES.items()}[plan.engine]
    stream = torch.cuda.current_stream(dev)
    allt = {**tens, **outs}

    for _ in range(args.warmup):
        layer.encode(allt)
    torch.cuda.synchronize()

    # timed region: exactly K layers through rnn_encode, nothing else on the stream
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        layer.encode(allt, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # a second pass with the library's stage-boundary events, for the per-stage
    # breakdown and the step kernel's duration (each mark adds a small gap)
    ev = HipEvents(5 * K)
    torch.cuda.synchronize()
    for i in range(K):
        layer.encode(allt, events=ev.ev[5 * i:5 * i + 5], stream=stream)
    torch.cuda.synchronize()

    lat = [ev.ms(5 * i, 5 * i + 4) for i in range(K)]
    stage = {k: [ev.ms(5 * i + a, 5 * i + b) for i in range(K)]
             for k, (a, b) in {"projection": (0, 1), "setup": (1, 2), "steps": (2, 3), "output": (3, 4)}.items()}
    ev.close()
    med = {k: statistics.median(v) for k, v in stage.items()}
    ms_per_step = wall * 1000.0 / K
    n_steps = plan.steps
    value = n_steps / (ms_per_step / 1000.0)

    # roofline of the recurrent-step kernel (dominant): algorithmic bytes per launch / launch time
    step_launches = max(1, plan.step_launches)
    steps_per_launch = n_steps / step_launches
    launch_ms = med["steps"] / step_launches
    bytes_per_launch = step_bytes(spec) * steps_per_launch
    achieved = bytes_per_launch / (launch_ms / 1000.0) / 1e9
    # projection flops (f rows skipped under input_forget)
    G = spec.gates - (1 if (spec.cell == "LSTM" and spec.input_forget) else 0)
    proj_flops = 2.0 * spec.num_directions * spec.seq * spec.batch * G * spec.hidden * spec.input
    proj_tflops = proj_flops / (med["projection"] / 1000.0) / 1e12 if med["projection"] > 0 else 0.0

    line = {
        "metric": "bidir LSTM layer latency (ms) + timesteps/s; R-stream GB/s vs HBM peak",
        "value": round(value, 1),
        "unit": "timesteps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if spec.dtype == "f32" else "f16 tensors, f32 arithmetic",
        "data": "synthetic",
        "config": {"workload": name, "seq": spec.seq, "batch": spec.batch, "input": spec.input,
                   "hidden": spec.hidden, "directions": spec.num_directions, "engine": engine_name,
                   "timesteps_per_layer": n_steps},
        "latency_ms_median_with_stage_events": round(statistics.median(lat), 5),
        "stage_ms_median": {k: round(v, 5) for k, v in med.items()},
        "per_step_us": round(med["steps"] * 1000.0 / max(1, n_steps), 3),
        "roofline": {
            "bound": "hbm", "kernel": "recurrent step", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
            "traffic": (profiled_traffic(TRAFFIC_PROFILES[(args.config, engine_name)])
                        if (args.config, engine_name) in TRAFFIC_PROFILES else None),
            "bytes_per_launch": int(bytes_per_launch), "launch_us": round(launch_ms * 1000.0, 3),
            "launches_per_layer": step_launches,
        },
        "projection": {"tflops": round(proj_tflops, 3), "peak_tflops": MFMA_PEAK_TFLOPS[spec.dtype],
                       "frac": round(proj_tflops / MFMA_PEAK_TFLOPS[spec.dtype], 5)},
    }

    # floors of a step on this device, measured with the library itself on a
    # layer too small to have any arithmetic to speak of (the workload's
    # cell, seq, one batch row, input and hidden 8): one launch per step, and
    # the persistent engine's exchange between workgroups
    floors = {}
    for eng in (() if args.no_floors else ("launch", "persistent")):
        fspec = spec.replace(batch=1, input=8, hidden=8, lens=False, max_length=0, layout=0,
                             direction=spec.direction)
        finp = synth.make_inputs(fspec, 1)
        ften = rl.to_device(finp, "cuda:0")
        fouts = {n: torch.empty(rl.output_shapes(fspec)[n], dtype=dt, device=dev) for n in fspec.outputs
                 if not (n == "Y_c" and fspec.cell != "LSTM")}
        flayer = rl.Layer(fspec, engine=eng, device="cuda:0")
        fall = {**ften, **fouts}
        for _ in range(3):
            flayer.encode(fall)
        fev = HipEvents(5 * 10)
        for i in range(10):
            flayer.encode(fall, events=fev.ev[5 * i:5 * i + 5])
        torch.cuda.synchronize()
        fsteps = statistics.median([fev.ms(5 * i + 2, 5 * i + 3) for i in range(10)])
        fev.close()
        floors[eng + "_per_step_us"] = round(fsteps * 1000.0 / max(1, flayer.plan.steps), 3)
        del flayer
    if floors:
        line["step_floor"] = {**floors, "layer": f"{spec.cell} seq {spec.seq}, batch 1, input 8, hidden 8"}

    if not args.no_cpu_baseline:
        # the oracle on a bounded sample: whole layers while one takes under
        # the time target, else the first r batch rows (independent
        # sequences), r doubling until the target is reached, with the
        # layer's time scaled by B / r
        from oracle import oracle
        rows = 1
        while True:
            sspec, sinp = row_subset(spec, inputs, rows)
            t1 = time.perf_counter()
            o = oracle.run(sspec, sinp, outputs=spec.outputs)
            t_sub = time.perf_counter() - t1
            if rows == spec.batch or t_sub * 2 >= args.cpu_seconds:
                break
            rows = min(spec.batch, rows * 2)
        runs, t_cpu = 1, t_sub
        while rows == spec.batch and t_cpu < args.cpu_seconds:
            t1 = time.perf_counter()
            o = oracle.run(sspec, sinp, outputs=spec.outputs)
            t_cpu += time.perf_counter() - t1
            runs += 1
        layer_s = t_cpu / runs * spec.batch / rows
        what = (f"the whole {args.config} layer, {runs} run(s) in {t_cpu:.1f} s" if rows == spec.batch else
                f"the first {rows} of {spec.batch} batch rows of {args.config} in {t_cpu:.1f} s, scaled by "
                f"{spec.batch}/{rows} to the whole layer")
        line["cpu_baseline"] = {
            "value": round(n_steps / layer_s, 2), "unit": "timesteps/s", "cores": o["threads"], "kind": "oracle",
            "sample": f"{what} (float64, threaded over the {spec.num_directions * rows} independent sequences)",
        }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())

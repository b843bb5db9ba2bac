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
# MI355X dense peaks per arithmetic unit (TFLOP/s): f16 and bf16 matrix cores,
# f32 matrix cores, f32 vector ALUs
PEAK_TFLOPS = {"f16 matrix cores": 2500.0, "bf16x3 matrix cores": 2500.0, "f32 matrix cores": 157.3,
               "f32 vector ALU": 157.3}
# products issued per product of the method: h as two f16 halves in the steps
# (the projection reads f16 operands as they are), three bf16 products per f32
# product
ISSUED_PER_PRODUCT = {"f16 matrix cores": 1, "bf16x3 matrix cores": 3, "f32 matrix cores": 1, "f32 vector ALU": 1}
EXTRA_CONFIGS = ("C1", "C3", "C3L1", "C4", "C5")


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


def row_subset(spec, inputs, rows: int, steps: int = 0):
    """The first `rows` batch rows of a layer (rows are independent sequences),
    and with `steps` > 0 only the first `steps` time steps of each (lengths cut
    to them)."""
    import numpy as np
    sub = dict(inputs)
    S = spec.seq if steps <= 0 else min(steps, spec.seq)
    if spec.layout == 0:
        sub["X"] = inputs["X"][:S, :rows]
        for k in ("initial_h", "initial_c"):
            if k in inputs:
                sub[k] = inputs[k][:, :rows]
    else:
        sub["X"] = inputs["X"][:rows, :S]
        for k in ("initial_h", "initial_c"):
            if k in inputs:
                sub[k] = inputs[k][:rows]
    if "sequence_lens" in inputs:
        sub["sequence_lens"] = np.minimum(inputs["sequence_lens"][:rows], S).astype(np.int32)
    return spec.replace(batch=rows, seq=S, max_length=min(spec.max_length, S) if spec.max_length else 0), sub


def row_steps(spec, inputs) -> int:
    """Steps run summed over every (direction, batch row) sequence."""
    import numpy as np
    L = spec.max_length or spec.seq
    if "sequence_lens" in inputs:
        lens = np.clip(inputs["sequence_lens"].astype(np.int64), 0, spec.seq)
    else:
        lens = np.full(spec.batch, spec.seq, np.int64)
    return int(np.minimum(lens, L).sum()) * spec.num_directions


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def step_flops(spec) -> float:
    """Flops of the method's recurrent products in one step (both directions,
    every batch row): 2 * D * B * Gp * H * H (Gp: gate blocks computed)."""
    G = spec.gates - (1 if (spec.cell == "LSTM" and spec.input_forget) else 0)
    return 2.0 * spec.num_directions * spec.batch * G * spec.hidden * spec.hidden


def proj_flops(spec) -> float:
    G = spec.gates - (1 if (spec.cell == "LSTM" and spec.input_forget) else 0)
    return 2.0 * spec.num_directions * spec.seq * spec.batch * G * spec.hidden * spec.input


def time_layer(layer, allt, stream, K: int, warmup: int):
    """K layers through rnn_encode between synchronisations (wall clock), then
    K more with the library's stage-boundary events; returns (ms per layer,
    median stage times in ms)."""
    import torch
    for _ in range(warmup):
        layer.encode(allt, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        layer.encode(allt, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = HipEvents(5 * K)
    torch.cuda.synchronize()
    for i in range(K):
        layer.encode(allt, events=ev.ev[5 * i:5 * i + 5], stream=stream)
    torch.cuda.synchronize()
    stage = {k: statistics.median([ev.ms(5 * i + a, 5 * i + b) for i in range(K)])
             for k, (a, b) in {"projection": (0, 1), "setup": (1, 2), "steps": (2, 3), "output": (3, 4),
                               "layer": (0, 4)}.items()}
    ev.close()
    return wall * 1000.0 / K, stage


def step_floors(spec, dt, engines=("launch", "persistent")) -> dict:
    """Per-step time of a layer of the same cell, direction and length with
    one batch row, input 8 and hidden 8 (nothing to compute to speak of): one
    launch per step, and the persistent engine's exchange between workgroups
    with its gate chain."""
    import torch
    import onnx_recurrent_layers_amd as rl
    from onnx_recurrent_layers_amd import synth
    dev = torch.device("cuda", 0)
    out = {}
    for eng in engines:
        fspec = spec.replace(batch=1, input=8, hidden=8, lens=False, max_length=0, layout=0)
        finp = synth.make_inputs(fspec, 1)
        ften = rl.to_device(finp, "cuda:0")
        fouts = {n: torch.empty(rl.output_shapes(fspec)[n], dtype=dt, device=dev) for n in fspec.outputs
                 if not (n == "Y_c" and fspec.cell != "LSTM")}
        flayer = rl.Layer(fspec, engine=eng, device="cuda:0")
        _, st = time_layer(flayer, {**ften, **fouts}, torch.cuda.current_stream(dev), 30, 5)
        out[eng + "_per_step_us"] = round(st["steps"] * 1000.0 / max(1, flayer.plan.steps), 3)
        del flayer
    out["layer"] = f"{spec.cell} {spec.direction} seq {spec.seq}, batch 1, input 8, hidden 8"
    return out


def cpu_baseline(name, spec, inputs, cpu_seconds: float, single_thread: bool = False) -> dict:
    """The oracle (as it stands) on a bounded sample of the layer: the first r
    batch rows and the first s time steps, grown until the sample takes about
    `cpu_seconds`, its time scaled to the whole layer by the ratio of
    (direction, row) steps; threaded over the sample's independent
    sequences."""
    from oracle import oracle
    host = os.cpu_count() or 1
    # the threads this process may use: its CPU affinity, or OMP_NUM_THREADS
    # where that is set lower
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else host
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = 1 if single_thread else max(1, min(avail, omp) if omp > 0 else avail)
    rows = 1 if single_thread else min(spec.batch, max(1, threads // spec.num_directions))
    steps = min(spec.seq, 4)
    while True:
        sspec, sinp = row_subset(spec, inputs, rows, steps)
        t1 = time.perf_counter()
        o = oracle.run(sspec, sinp, nthreads=threads, outputs=spec.outputs)
        t_sub = time.perf_counter() - t1
        if t_sub * 2 >= cpu_seconds or (steps == spec.seq and rows == spec.batch):
            break
        if steps < spec.seq:
            steps = min(spec.seq, steps * 2)
        else:
            rows = min(spec.batch, rows * 2)
    runs, t_cpu = 1, t_sub
    while t_cpu < cpu_seconds and t_sub * 4 < cpu_seconds:
        t1 = time.perf_counter()
        oracle.run(sspec, sinp, nthreads=threads, outputs=spec.outputs)
        t_cpu += time.perf_counter() - t1
        runs += 1
    full, part = row_steps(spec, inputs), max(1, row_steps(sspec, sinp))
    layer_s = t_cpu / runs * full / part
    whole = rows == spec.batch and steps == spec.seq
    what = (f"the whole {name} layer, {runs} run(s) in {t_cpu:.1f} s" if whole else
            f"the first {rows} of {spec.batch} batch rows and the first {steps} of {spec.seq} steps of {name}, "
            f"{runs} run(s) in {t_cpu:.1f} s, scaled by the ratio of (direction, row) steps, {full}/{part}, "
            f"to the whole layer")
    return {"value": round((spec.max_length or spec.seq) / layer_s, 2), "unit": "timesteps/s",
            "cores": o["threads"], "host_cores": host, "cpu_model": cpu_model(), "kind": "oracle",
            "layer_s": round(layer_s, 4),
            "sample": f"{what} (float64, {o['threads']} thread(s) over the sample's "
                      f"{sspec.num_directions * sspec.batch} independent sequences)"}


def measure(name: str, engine: str, K: int, warmup: int, floors: bool, cpu_seconds: float,
            single_thread: bool = False, xw_chunk_steps: int = 0) -> dict:
    """One workload: latency, throughput, stage times, the step kernel against
    the bounds that apply to it, the projection against the peak of the units
    it runs on, and the oracle baseline."""
    import torch
    import onnx_recurrent_layers_amd as rl
    from onnx_recurrent_layers_amd import synth

    spec, inputs = synth.config(name)
    if xw_chunk_steps:
        spec = spec.replace(xw_chunk_steps=xw_chunk_steps)
    dev = torch.device("cuda", 0)
    dt = torch.float32 if spec.dtype == "f32" else torch.float16
    tens = rl.to_device(inputs, "cuda:0")
    shapes = rl.output_shapes(spec)
    outs = {n: torch.empty(shapes[n], dtype=dt, device=dev) for n in spec.outputs
            if not (n == "Y_c" and spec.cell != "LSTM")}
    layer = rl.Layer(spec, engine=engine, device="cuda:0")
    plan = layer.plan
    engine_name = {v: k for k, v in rl.ENGINES.items()}[plan.engine]
    stream = torch.cuda.current_stream(dev)
    ms, st = time_layer(layer, {**tens, **outs}, stream, K, warmup)
    run = layer.run_status()
    n_steps = plan.steps
    step_kind = rl.PRODUCTS[plan.step_products]
    proj_kind = rl.PRODUCTS[plan.proj_products]

    step_launches = max(1, plan.step_launches)
    # A projection in chunks: the projection stage times the first chunk; the
    # later ones run inside the steps stage, each about as long as the first.
    tc = plan.xw_chunk_steps
    nchunks = -(-n_steps // tc) if 0 < tc < n_steps else 1
    steps_only_ms = st["steps"] - (nchunks - 1) * st["projection"]
    launch_ms = steps_only_ms / step_launches
    per_step_us = st["steps"] * 1000.0 / max(1, n_steps)
    bytes_per_launch = step_bytes(spec) * n_steps / step_launches
    hbm = bytes_per_launch / (launch_ms / 1000.0) / 1e9
    method = step_flops(spec) * n_steps / step_launches
    issued = method * (2 if step_kind == "f16 matrix cores" else ISSUED_PER_PRODUCT[step_kind])
    mf = issued / (launch_ms / 1000.0) / 1e12
    prof = TRAFFIC_PROFILES.get((name, engine_name))
    bounds = {
        "hbm": {"achieved": round(hbm, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(hbm / HBM_PEAK_GBS, 5),
                "bytes_per_launch": int(bytes_per_launch),
                "traffic": profiled_traffic(prof) if prof else None,
                "what": "algorithmic bytes: R once per step, the step's Xw slice, h (and c) read and written; "
                        "traffic: measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a "
                        "plain copy) while the kernel sources match the profiled ones"},
        "arith": {"achieved": round(mf, 3), "peak": PEAK_TFLOPS[step_kind], "unit": "TFLOP/s",
                  "frac": round(mf / PEAK_TFLOPS[step_kind], 5), "units": step_kind,
                  "method_flops_per_launch": method, "issued_flops_per_launch": issued},
    }
    res = {
        "workload": synth.CONFIGS[name]["name"], "engine": engine_name, "dtype": spec.dtype,
        "timesteps_per_layer": n_steps, "layer_ms": round(ms, 5), "timesteps_per_s": round(n_steps / (ms / 1e3), 1),
        "row_steps_per_s": round(row_steps(spec, inputs) / (ms / 1e3), 1),
        "stage_ms_median": {k: round(v, 5) for k, v in st.items()},
        "per_step_us": round(per_step_us, 3), "step_launches": plan.step_launches, "step_launch_us": round(launch_ms * 1e3, 3),
        "step_products": step_kind, "step_bounds": bounds, "fallback_workgroups": run.fallback_workgroups,
        "xw_chunk_steps": plan.xw_chunk_steps, "xw_slots": plan.xw_slots, "xw_scratch_bytes": layer.xw_bytes,
    }
    if nchunks > 1:
        res["step_launch_us_what"] = ("steps stage less the %d later projection chunks (each taken as long as the "
                                      "first, which the projection stage times), over the step launches" % (nchunks - 1))
    if floors and engine_name == "persistent" and plan.step_products in (0, 2) and spec.batch <= 8:
        fl = step_floors(spec, dt)
        res["step_floor"] = fl
        # the minimal layer runs fewer workgroups than this one, so a step can
        # match it within the timing noise: the fraction stops at 1
        res["step_bounds"]["exchange"] = {
            "floor_us": fl["persistent_per_step_us"], "per_step_us": round(per_step_us, 3),
            "frac": round(min(1.0, fl["persistent_per_step_us"] / per_step_us), 5),
            "at_floor": fl["persistent_per_step_us"] >= per_step_us,
            "what": "per-step time of the persistent engine on a layer with nothing to compute (same cell, "
                    "direction and length; batch 1, input 8, hidden 8): the exchange between workgroups, two "
                    "workgroup barriers and the gate chain; a step at or below it (at_floor) reports 1"}
    # the binding bound: the largest fraction
    res["binding"] = max(res["step_bounds"], key=lambda k: res["step_bounds"][k]["frac"])
    pm = proj_flops(spec) * (min(tc, n_steps) / n_steps if nchunks > 1 else 1.0)
    pi = pm * ISSUED_PER_PRODUCT[proj_kind]
    pt = st["projection"]
    res["projection"] = {
        "units": proj_kind, "method_flops": pm, "issued_flops": pi, "ms": round(pt, 5),
        "chunks": nchunks,
        "what": ("the first of %d chunks of %d steps (its flops over the projection stage's time; the later "
                 "chunks run between the steps)" % (nchunks, tc)) if nchunks > 1 else "the whole projection",
        "method_tflops": round(pm / (pt / 1e3) / 1e12, 3) if pt > 0 else 0.0,
        "issued_tflops": round(pi / (pt / 1e3) / 1e12, 3) if pt > 0 else 0.0,
        "peak_tflops": PEAK_TFLOPS[proj_kind],
        "frac": round(pi / (pt / 1e3) / 1e12 / PEAK_TFLOPS[proj_kind], 5) if pt > 0 else 0.0,
    }
    del layer, tens, outs
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(name, spec, inputs, cpu_seconds)
        if single_thread:
            res["cpu_baseline_single_thread"] = cpu_baseline(name, spec, inputs, cpu_seconds, single_thread=True)
    res["_spec"] = spec
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed layer runs")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--engine", default="auto", choices=["auto", "launch", "persistent"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--extra-cpu-seconds", type=float, default=4.0,
                    help="target CPU time of each other workload's oracle baseline")
    ap.add_argument("--extra", default=",".join(EXTRA_CONFIGS),
                    help="other workloads measured after the main one and reported under 'configs' "
                         "(comma-separated; empty for none)")
    ap.add_argument("--xw-chunk-steps", type=int, default=0,
                    help="the main workload's projection in chunks of this many steps (0: the library chooses)")
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

    import torch
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

    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    m = measure(args.config, args.engine, args.steps, args.warmup, not args.no_floors, cpu_s,
                single_thread=args.config in ("C1", "C2") and not args.no_cpu_baseline,
                xw_chunk_steps=args.xw_chunk_steps)
    spec = m.pop("_spec")
    hb = m["step_bounds"]["hbm"]
    line = {
        "metric": "bidir LSTM layer latency (ms) + timesteps/s; R-stream GB/s vs HBM peak",
        "value": m["timesteps_per_s"],
        "unit": "timesteps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["layer_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if spec.dtype == "f32" else "f16 tensors, f32 arithmetic",
        "data": "synthetic",
        "config": {"workload": m["workload"], "seq": spec.seq, "batch": spec.batch, "input": spec.input,
                   "hidden": spec.hidden, "directions": spec.num_directions, "engine": m["engine"],
                   "timesteps_per_layer": m["timesteps_per_layer"]},
        "latency_ms_median_with_stage_events": m["stage_ms_median"]["layer"],
        "stage_ms_median": {k: v for k, v in m["stage_ms_median"].items() if k != "layer"},
        "per_step_us": m["per_step_us"],
        "roofline": {
            "bound": "hbm", "kernel": "recurrent step", "achieved": hb["achieved"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": hb["frac"],
            "traffic": hb["traffic"],
            "bytes_per_launch": hb["bytes_per_launch"], "launch_us": m["step_launch_us"],
            "launches_per_layer": max(1, m["step_launches"]),
            "binding": m["binding"],
        },
        "step_bounds": m["step_bounds"],
        "projection": m["projection"],
    }
    if "step_floor" in m:
        line["step_floor"] = m["step_floor"]
    for k in ("cpu_baseline", "cpu_baseline_single_thread"):
        if k in m:
            line[k] = m[k]
    extras = [c for c in args.extra.split(",") if c and c != args.config]
    if extras:
        line["configs"] = {}
        for c in extras:
            r = measure(c, "auto", max(3, min(args.steps, 20)), max(1, min(args.warmup, 3)), not args.no_floors,
                        0.0 if args.no_cpu_baseline else args.extra_cpu_seconds, single_thread=c in ("C1", "C2"))
            r.pop("_spec")
            line["configs"][c] = r
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())

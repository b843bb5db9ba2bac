"""The benchmark's JSON line on the GPU: a short run of the default workload
(the bidirectional LSTM, seq 80, batch 1, 256/256, f32) through bench.main(),
with every derived figure checked against the figures it is derived from."""
import json
import sys

import pytest

import bench
from onnx_recurrent_layers_amd import synth
from tests.gpu_harness import note

pytestmark = pytest.mark.gpu


def test_bench_line(monkeypatch, capsys):
    note("case bench.main() C2 steps 3 warmup 1 cpu-seconds 0.5")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"])
    assert bench.main() == 0
    out = capsys.readouterr().out.strip().splitlines()
    d = json.loads(out[-1])
    spec = synth.CONFIGS["C2"]["spec"]

    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "timesteps/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["dtype"] == "f32" and d["vs_baseline"] is None
    assert d["config"]["workload"] == synth.CONFIGS["C2"]["name"]
    assert d["config"]["timesteps_per_layer"] == spec.seq
    # throughput is timesteps over the layer latency
    assert d["value"] == pytest.approx(spec.seq / (d["ms_per_step"] / 1000.0), rel=1e-3)

    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["bytes_per_launch"] == bench.step_bytes(spec) * spec.seq // r["launches_per_layer"]
    assert r["achieved"] == pytest.approx(r["bytes_per_launch"] / (r["launch_us"] * 1e3), rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["traffic"] is None or r["traffic"] > 0
    assert 0 < r["launch_us"] <= d["ms_per_step"] * 1000.0 * 1.5

    assert set(d["stage_ms_median"]) == {"projection", "setup", "steps", "output"}
    assert all(v >= 0 for v in d["stage_ms_median"].values())
    assert d["step_floor"]["launch_per_step_us"] > 0 and d["step_floor"]["persistent_per_step_us"] > 0

    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "timesteps/s" and c["cores"] >= 1 and c["value"] > 0

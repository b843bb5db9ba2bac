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
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5",
                                      "--extra", "C1,C3", "--extra-cpu-seconds", "0.3"])
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
    assert c["host_cores"] >= 1 and c["cpu_model"]
    assert d["cpu_baseline_single_thread"]["cores"] == 1

    # every fraction against a peak or a floor is at most 1
    for b in d["step_bounds"].values():
        assert 0 < b["frac"] <= 1.0, b
    assert d["roofline"]["binding"] in d["step_bounds"]
    p = d["projection"]
    assert p["units"] == "f32 matrix cores" and p["issued_flops"] == p["method_flops"]
    assert 0 < p["frac"] <= 1.0
    assert p["method_flops"] == 2.0 * 2 * spec.seq * spec.batch * 4 * spec.hidden * spec.input

    # the other workloads, each with the same figures
    assert set(d["configs"]) == {"C1", "C3"}
    c3 = d["configs"]["C3"]
    s3 = synth.CONFIGS["C3"]["spec"]
    assert c3["timesteps_per_layer"] == s3.seq and c3["step_products"] == "f16 matrix cores"
    assert c3["timesteps_per_s"] == pytest.approx(s3.seq / (c3["layer_ms"] / 1000.0), rel=1e-3)
    for r in d["configs"].values():
        for b in r["step_bounds"].values():
            assert 0 < b["frac"] <= 1.0, b
        assert 0 < r["projection"]["frac"] <= 1.0
        assert r["cpu_baseline"]["value"] > 0 and r["fallback_workgroups"] == 0

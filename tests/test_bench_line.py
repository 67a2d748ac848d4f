"""bench.py's output: one JSON line whose fields are consistent with one
another (the roofline's fraction is achieved over peak, the step's rate is
its bytes over its time), with the CPU oracle timed beside the GPU; and the
refusal of a multi-GPU run, which this library has no path for."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    res = run_bench("--gpus", "2", timeout=60)
    assert res.returncode == 2
    assert b"one GPU" in res.stderr and not res.stdout.strip()


@pytest.mark.gpu
def test_json_line_is_consistent():
    print("[bench] fp32 1000x1003, 3 steps, 1 s of oracle", flush=True)
    res = run_bench("--workload", "fp32_1000x1003_nd4", "--steps", "3", "--warmup", "1",
                    "--cpu-seconds", "1", "--only")
    assert res.returncode == 0, res.stderr.decode()[-2000:]
    lines = [l for l in res.stdout.decode().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["unit"] == "GB/s"
    assert d["config"]["workload"] == "fp32_1000x1003_nd4"
    cfg = d["config"]
    assert d["value"] == pytest.approx(cfg["bytes_per_step"] / d["ms_per_step"] / 1e6, rel=5e-3)
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert roof["achieved"] == pytest.approx(
        roof["bytes_per_launch"] / roof["avg_launch_us"] / 1e3, rel=2e-3)
    if roof["traffic"] is None:
        assert roof["traffic_GBps"] is None
    else:
        assert roof["traffic_GBps"] == pytest.approx(
            roof["traffic"] / roof["avg_launch_us"] / 1e3, rel=2e-3)
    fused = d["kernels"]["fused"]
    assert fused["launches"] == 3 and fused["min_us"] <= fused["median_us"]
    # the roofline names the kind of launch with the most time per step
    ks = d["kernels"]
    step_kinds = [k for k in ks if "us_per_step" in ks[k]]
    assert roof["kind"] == max(step_kinds, key=lambda k: ks[k]["us_per_step"])
    assert roof["step_frac"] == pytest.approx(d["value"] / roof["peak"], abs=2e-4)
    assert list(d["workloads"]) == ["fp32_1000x1003_nd4"]
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert cpu["cores"] >= 1 and cpu["single_core"]["cores"] == 1

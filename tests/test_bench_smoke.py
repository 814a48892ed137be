"""bench.py end to end: the tiny workload on the GPU emits one JSON line
with the fields the driver reads; a multi-GPU request is refused on any
machine."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_forced_persistent_path_checks_its_outputs():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "2",
                        "--assign-path", "3", "--steps", "5", "--warmup", "2",
                        "--settle-ms", "20", "--cpu-seconds", "0.2", "--no-ceiling"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["config"]["path"].startswith("persistent")
    assert "assign_queue_kernel" in d["roofline"]["kernel"]
    assert d["parity"]["bad"] == 0 and d["parity"]["points"] > 0


@pytest.mark.gpu
def test_bench_tiny_workload_emits_the_json_line():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "1",
                        "--steps", "5", "--warmup", "2", "--settle-ms", "20",
                        "--cpu-seconds", "0.2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "mfma_ceiling"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["unit"] == "points/s" and d["dtype"] == "bf16"
    assert d["config"]["N"] == 4096 and d["config"]["D"] == 64 and d["config"]["K"] == 256
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == 2516.6 and 0 < rf["frac"] < 1
    assert abs(rf["achieved"] / rf["peak"] - rf["frac"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert d["mfma_ceiling"]["tflops"] > 0


@pytest.mark.gpu
@pytest.mark.parametrize("path", [1, 2])
def test_bench_update_emits_the_json_line_and_checks_its_outputs(path):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--update",
                        "--update-path", str(path), "--config", "1", "--steps", "6",
                        "--warmup", "2", "--settle-ms", "20", "--cpu-seconds", "0.2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["config"]["path"] == {1: "sort", 2: "buckets"}[path]
    assert d["roofline"]["bound"] == "hbm" and d["value"] > 0
    p = d["parity"]
    assert p["bad_sets"] == 0 and len(p["per_seed"]) == 3
    assert all(v["ok"] for v in p["per_seed"].values())

"""bench.py's host-side contract, on the CPU: argument checks that end the run
before any GPU work, the counter lookup that feeds `roofline.traffic`, and a
complete JSON line from the CPU-offload leg."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args, timeout=300):
    env = dict(os.environ, CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_workload_is_refused():
    r = _run("--workload", "no_such_workload")
    assert r.returncode == 2 and "unknown workload" in r.stderr


@pytest.mark.parametrize("wl", ["llama3_8b_p8", "edge_p16_literal"])
def test_unfused_needs_a_single_tensor_slice_workload(wl):
    r = _run("--unfused", "--workload", wl)
    assert r.returncode == 2 and "--unfused" in r.stderr


def test_traffic_only_for_the_measured_workload_and_form():
    with open(bench.COUNTERS_FILE) as fh:
        data = json.load(fh)
    rec = data["zero_7p5b_p64"]
    got = bench.measured_traffic("zero_7p5b_p64", rec.get("form", "standard"))
    if rec["kernel_source_hash"] == bench.kernel_source_hash():
        assert got == rec["hbm_bytes_per_launch"]
        # read and write bytes within 10% of the algorithmic bytes of the launch
        assert abs(got / rec["algorithmic_bytes_per_launch"] - 1.0) < 0.10
    else:
        assert got is None  # counters taken on other kernel sources are not reported
    assert bench.measured_traffic("zero_7p5b_p64", "sgd") is None
    assert bench.measured_traffic("tiny_p4", "standard") is None


def test_cpu_offload_json_line():
    r = _run("--cpu-offload", "--workload", "tiny_p4", "--steps", "3", "--warmup", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in d, key
    assert d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["workload"] == "tiny_p4"

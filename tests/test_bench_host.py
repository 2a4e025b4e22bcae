"""Host-side pieces of bench.py: the one-GPU refusal, the HBM-traffic lookup
keyed to the kernel sources, and the CPU-baseline leg (the oracle on host
processes).  No GPU is touched."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as WL  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        entry = json.load(f)["4k"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: entry["kernel_sha"])
    assert bench.measured_traffic("4k") == entry["bytes_per_launch"]
    assert abs(entry["bytes_per_launch"] - entry["fetch_bytes"] - entry["write_bytes"]) <= 1  # each rounded
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.measured_traffic("4k") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_kernel_hash_covers_the_attention_sources():
    assert [os.path.basename(p) for p in bench.KERNEL_SRCS] == ["kernels.hip", "plan.cpp"]
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0


@pytest.mark.timeout(300)
def test_cpu_baseline_times_whole_heads_of_the_oracle():
    w = WL.WORKLOADS["tiny"]
    cpu = bench.cpu_baseline(w, max_procs=2)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s"
    assert cpu["value"] > 0 and cpu["seconds"] > 0
    assert cpu["processes"] == cpu["cores"] == min(2, os.cpu_count() or 1, w.heads)
    assert cpu["nproc"] == (os.cpu_count() or 1) and cpu["blas_threads_per_process"] == 1
    assert isinstance(cpu["cpu_model"], str) and cpu["cpu_model"]
    assert f"of {w.heads} heads of the {w.name} layer" in cpu["sample"]

"""Host logic of bench.py (no GPU): the one-GPU guard, the stored-traffic lookup that keeps
HBM bytes only while the kernel source is the one they were measured on, and the per-class
kernel figures."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.fixture
def traffic_files(tmp_path, monkeypatch):
    src = tmp_path / "kernels.hip"
    src.write_bytes(b"// kernels\n")
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNELS_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC", str(rec))
    return src, rec


def test_stored_traffic_only_for_the_measured_source(traffic_files):
    src, rec = traffic_files
    assert bench.stored_traffic() is None  # no measurement
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    rec.write_text(json.dumps({"kernels_hip_sha256": sha, "hbm_bytes_per_launch": 1234}))
    assert bench.stored_traffic() == 1234
    src.write_bytes(b"// kernels, changed\n")  # any edit, a comment included
    assert bench.stored_traffic() is None


def test_committed_traffic_record_is_consistent():
    """The stored counter summary: bytes per launch = (fetched + written) / launches, taken with
    commands that run bench.py only."""
    with open(os.path.join(ROOT, "profiles", "conv_traffic_704x1280_bf16.json")) as f:
        t = json.load(f)
    assert t["launches"] > 0 and t["launches"] % 1208 == 0  # whole decodes of 1,208 conv launches
    assert t["hbm_bytes_per_launch"] == int((t["fetch_bytes"] + t["write_bytes"]) / t["launches"])
    assert all("bench.py" in c and "_work" not in c for c in t["commands"])
    assert len(t["kernels_hip_sha256"]) == 64


def test_kernel_classes_figures():
    prof = {"conv": {"ms": 300.0, "launches": 30, "flops": 3e14, "bytes": 0.0},
            "norm": {"ms": 10.0, "launches": 20, "flops": 0.0, "bytes": 4e10}}
    k = bench.kernel_classes(prof, 3)
    assert k["conv"] == {"ms_per_step": 100.0, "launches_per_step": 10, "TFLOP/s": 1000.0}
    assert k["norm"]["GB/s"] == 4000.0 and k["norm"]["frac_of_peak"] == 0.5
    assert k["norm"]["launches_per_step"] == 6

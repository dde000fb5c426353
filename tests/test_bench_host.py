"""Host-side logic of bench.py (no GPU): the work and byte counts behind the
throughput and roofline figures, the traffic record's source-hash gate and
the single-GPU guard."""
import json
import subprocess
import sys

import pytest

import bench


def test_flop_count_of_the_headline_workload():
    # 4 B H N^2 d: two N x N x d products of two FLOPs per multiply-add
    assert bench.flops(8, 32, 1024, 64, False) == 4 * 8 * 32 * 1024 * 1024 * 64
    assert bench.flops(8, 32, 1024, 64, True) == bench.flops(8, 32, 1024, 64, False) / 2


def test_algorithmic_bytes_of_the_headline_workload():
    # Q, K, V read and O written once in binary16, lse written once in float32
    n = 8 * 32 * 1024 * 64
    assert bench.algorithmic_bytes(8, 32, 1024, 64, 2, 2) == 4 * 2 * n + 4 * 8 * 32 * 1024 == 135266304
    # fp8 inputs with bfloat16 output
    assert bench.algorithmic_bytes(8, 32, 1024, 64, 1, 2) == 5 * n + 4 * 8 * 32 * 1024


def test_traffic_record_is_used_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "bytes_per_launch": 123}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic() == 123
    rec["kernel_source_sha256_16"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.load_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic() is None


def test_committed_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for key in ("kernel", "kernel_source_sha256_16", "fetch_bytes_per_launch", "write_bytes_per_launch",
                "bytes_per_launch", "algorithmic_bytes_per_launch", "calibration", "commands"):
        assert key in t, key
    assert t["bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert t["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(8, 32, 1024, 64, 2, 2)


def test_kernel_source_hash_changes_with_the_source(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("one")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a)])
    h1 = bench.kernel_source_hash()
    a.write_text("two")
    assert bench.kernel_source_hash() != h1


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    out = subprocess.run([sys.executable, bench.__file__, "--gpus", n], capture_output=True, text=True, timeout=120)
    assert out.returncode != 0
    assert "one GPU" in (out.stdout + out.stderr)

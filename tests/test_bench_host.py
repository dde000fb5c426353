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


def test_every_configuration_has_a_current_record_where_committed():
    """c2-c5 carry committed counter records taken on the current kernel
    sources (bench.py reports their traffic and instruction ceilings)."""
    for tag, B, H, N, d, dt, causal in bench.CONFIGS[1:]:
        rec = bench.load_record(bench.record_tag(B, H, N, d, dt, causal))
        assert rec is not None, tag
        assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(B, H, N, d, 1 if dt == "fp8" else 2, 2)
        for key in ("valu", "valu_trans", "mfma", "lds", "lds_load_64b"):
            assert rec["instructions"][key] > 0, (tag, key)


def test_lds_bytes_per_score_follow_the_tile_shape():
    assert bench.lds_bytes_per_score(64, "f16", "32x8x64x0x4") == 8.0      # K and V once per 32 rows
    assert bench.lds_bytes_per_score(64, "bf16", "64x8x64x1x2") == 4.0     # 64-row waves halve it
    assert bench.lds_bytes_per_score(64, "fp8", "64x4x64x0x2") == 2.0      # 8-bit K and V
    assert bench.lds_bytes_per_score(128, "bf16", "64x8x32x1x2") == 12.0   # + the second block's Q from LDS
    assert bench.lds_bytes_per_score(128, "fp8", "64x8x32x1x2") == 4.0     # fp8 Q stays in registers


def test_secondary_ceilings_from_instruction_counts():
    d, fl = 64, bench.flops(8, 32, 1024, 64, False)
    scores = fl / (4 * d)
    rec = {"instructions": {"valu": 3.0 * scores / 64 + 100, "valu_trans": scores / 64, "mfma": 100}}
    c = bench.secondary_ceilings(d, "f16", False, fl, "32x8x64x0x4", rec)
    assert abs(c["valu_insts_per_score"] - 2.0) < 1e-6 and abs(c["trans_insts_per_score"] - 1.0) < 1e-6
    # 2 plain instructions at 4 cycles and 1 exponential at 8 per score on 1024 SIMDs at 2.4 GHz
    t = scores / 64 * (2 * 4 + 8) / 1024 / 2.4e9
    assert abs(c["valu_ceiling_tflops"] - fl / t / 1e12) < 0.1
    assert "valu_ceiling_tflops" not in bench.secondary_ceilings(d, "f16", False, fl, "32x8x64x0x4", None)


def test_sampled_cpu_baseline_extrapolates_by_slices(monkeypatch):
    import oracle
    from io_aware_attention_fwd_amd import gen

    x = gen.make(2, 4, 64, 64, "f16", seed=1)
    calls = []
    monkeypatch.setattr(oracle, "attention_slice", lambda *a, **k: calls.append(1))
    r = bench.cpu_baseline_sampled(x, False, 0.125, 0.0, oracle.slice_sample(2, 4, count=3))
    assert len(calls) == 1  # a zero budget still times one slice
    assert r["kind"] == "oracle" and r["cores"] >= 1 and "x8" in r["sample"]


def test_oracle_threads_follow_affinity_and_share(monkeypatch):
    import os

    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    assert 1 <= bench.oracle_threads() <= min(2, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.oracle_threads() >= 1  # back to the whole affinity mask for the tests that follow

"""Host-side checks of the measurement tools (no GPU): the tile sweep reads
every compiled tile shape from the kernel source, the GPU tile test covers
each of them, and the profile recorder names its files and commands as
documented."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from io_aware_attention_fwd_amd import record, sweep  # noqa: E402


def test_sweep_reads_every_compiled_shape():
    v = sweep.variants()
    assert len(v) == len(set(v)) >= 5
    for t in v:
        qw, nw, bc, sched, wpe = (int(x) for x in t.split("x"))
        assert qw in (32, 64) and bc in (32, 64) and sched in (0, 1, 2) and 1 <= wpe <= 4
        assert sched == 0 or nw in (8, 16)  # the ping-pong groups hold NW/8 waves of every SIMD


def test_gpu_tile_test_covers_every_compiled_shape():
    from tests import test_tiles_gpu

    listed = test_tiles_gpu.TILES
    assert sorted(listed) == sorted(sweep.variants_per_d())
    assert {t for _, t in listed} == set(sweep.variants())
    for d, t in listed:  # a shape compiled for one head dimension only is tested there only
        assert (d, t) in sweep.variants_per_d()


def test_sweep_reads_the_instance_that_ran():
    name = ("void fa::fa_fwd_kernel<fa::(anonymous namespace)::TrBF16, 128, true, 64, 8, 32, 1, 2, false>"
            "(fa::FwdParams) [clone .kd]")
    assert sweep.tile_of_kernel(name) == "64x8x32x1x2"
    assert sweep.tile_of_kernel("void fa::fa_bwd_dq_kernel<...>") is None


def test_profiler_crash_is_recorded_not_hidden(monkeypatch):
    """A profiler run that ends with SIGSEGV is kept (its CSVs are complete)
    but its exit status lands in the sweep row and the recorded summary;
    any other failure raises."""
    import subprocess

    class P:
        def __init__(self, rc):
            self.returncode, self.stdout = rc, "{}"

    for rc in (-11, 139):
        monkeypatch.setattr(subprocess, "run", lambda *a, rc=rc, **k: P(rc))
        crashes = []
        sweep._run(["rocprofv3"], {}, 1, crashes)
        assert crashes == [rc]
        record.PROFILER_CRASHES.clear()
        record._profile(["--kernel-trace"], [], "/tmp/x", "t")
        assert record.PROFILER_CRASHES == [("--kernel-trace", rc)]
        assert str(rc) in record._crash_note()
    record.PROFILER_CRASHES.clear()
    assert "0 for every run" in record._crash_note()
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: P(1))
    import pytest

    with pytest.raises(RuntimeError):
        sweep._run(["rocprofv3"], {}, 1, [])
    with pytest.raises(RuntimeError):
        record._profile(["--kernel-trace"], [], "/tmp/x", "t")


def test_record_tags_and_commands():
    assert record.tag_of((8, 32, 1024, 64, "f16", False)) == "fa_fwd_f16_b8h32n1024d64"
    assert record.tag_of((2, 16, 16384, 128, "bf16", True)) == "fa_fwd_bf16_b2h16n16384d128_causal"
    assert "--shape" not in record._bench_args(record.HEADLINE, 20, 5)
    args = record._bench_args((4, 32, 8192, 128, "fp8", False), 3, 1, ["--copy-calib-mib", "256"])
    assert args[args.index("--shape") + 1] == "4,32,8192,128,fp8,0"
    assert args[args.index("--copy-calib-mib") + 1] == "256"
    cmd = record._display("--pmc FETCH_SIZE", ["--steps", "3"])
    assert cmd.startswith("cd /tmp && rocprofv3 --pmc FETCH_SIZE") and cmd.endswith("bench.py --steps 3")

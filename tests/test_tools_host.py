"""Host-side checks of the measurement tools (no GPU): the tile sweep reads
every compiled tile shape from the kernel source, the GPU tile test covers
each of them, and the profile recorder names its files and commands as
documented."""
import ast
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
        assert qw in (32, 64) and bc in (32, 64) and sched in (0, 1) and 1 <= wpe <= 4
        assert sched == 0 or nw in (8, 16)  # the ping-pong groups hold NW/8 waves of every SIMD


def test_gpu_tile_test_covers_every_compiled_shape():
    src = open(os.path.join(ROOT, "tests", "test_tiles_gpu.py")).read()
    line = next(l for l in src.splitlines() if l.startswith("TILES = "))
    listed = ast.literal_eval(line.split("=", 1)[1].strip())
    assert sorted(listed) == sorted(sweep.variants())


def test_record_tags_and_commands():
    assert record.tag_of((8, 32, 1024, 64, "f16", False)) == "fa_fwd_f16_b8h32n1024d64"
    assert record.tag_of((2, 16, 16384, 128, "bf16", True)) == "fa_fwd_bf16_b2h16n16384d128_causal"
    assert "--shape" not in record._bench_args(record.HEADLINE, 20, 5)
    args = record._bench_args((4, 32, 8192, 128, "fp8", False), 3, 1, ["--copy-calib-mib", "256"])
    assert args[args.index("--shape") + 1] == "4,32,8192,128,fp8,0"
    assert args[args.index("--copy-calib-mib") + 1] == "256"
    cmd = record._display("--pmc FETCH_SIZE", ["--steps", "3"])
    assert cmd.startswith("cd /tmp && rocprofv3 --pmc FETCH_SIZE") and cmd.endswith("bench.py --steps 3")

"""Record the rocprofv3 evidence behind bench.py's roofline figures.

    python -m io_aware_attention_fwd_amd.record --out-dir DIR [--shape B,H,N,d,dtype,causal]

Runs ``bench.py`` under ``rocprofv3`` (each run a child process started from
/tmp with a time limit) and writes short text summaries into DIR:

* ``<tag>_kernel_stats.md``: ``--kernel-trace --stats`` of the bench command
  with its default warm-up and step counts (the same command bench.py's line
  comes from), the forward kernel's average duration and the TFLOP/s it
  implies;
* unless ``--no-counters``: ``<tag>_counters.md`` and ``<tag>_traffic.json``
  from four counter runs, ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (one
  counter per run, each next to a 256 MiB device copy whose known size
  calibrates the counter), one run of SQ counters and one of instruction
  counts.  The JSON carries the hash of the kernel sources it was taken on;
  bench.py reports its traffic and instruction-based ceiling only while that
  hash matches the sources.

``tag`` names the kernel and workload, e.g. ``fa_fwd_f16_b8h32n1024d64``.

    python -m io_aware_attention_fwd_amd.record --out-dir DIR --mode MODE --mode-arg ARG --tag TAG

profiles another bench.py mode (``varlen``, ``dropout``, ``bwd``, ``proj``;
``--MODE ARG`` on bench.py's command line) the same way: ``TAG_kernel_stats.md``
with every kernel of the run, and the FLOP per step that bench.py reports
divided by the summed average durations of the kernels one step launches.
It needs a GPU and rocprofv3.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (host-side helpers: FLOP and byte counts, kernel source hash)

COPY_MIB = 256
HEADLINE = (8, 32, 1024, 64, "f16", False)
SQ_COUNTERS = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
               "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE"]
# instruction counts (per wave, summed over the dispatch) behind the vector-ALU ceiling bench.py reports:
# vector ALU instructions, the transcendental ones among them, matrix instructions, LDS instructions, and
# the bytes LDS loads returned (in 64-byte units)
INSTR_COUNTERS = {"valu": "SQ_INSTS_VALU", "valu_trans": "SQ_INSTS_VALU_TRANS_F32", "mfma": "SQ_INSTS_MFMA",
                  "lds": "SQ_INSTS_LDS", "lds_load_64b": "SQ_INSTS_LDS_LOAD_BANDWIDTH"}
MODE_FAMILY = {"varlen": "fwd", "dropout": "fwd", "bwd": "bwd", "proj": "proj"}


def _bench_args(shape, steps=None, warmup=None, extra=()):
    args = ["--no-sweep", "--no-cpu"] + list(extra)
    if steps is not None:
        args += ["--steps", str(steps), "--warmup", str(warmup)]
    if shape != HEADLINE:
        B, H, N, d, dt, causal = shape
        args += ["--shape", f"{B},{H},{N},{d},{dt},{int(causal)}"]
    return args


def _profile(prof_args, bench_args, out_dir, tag, timeout=300):
    cmd = (["rocprofv3"] + prof_args + ["--output-format", "csv", "-d", out_dir, "-o", tag, "--",
                                        sys.executable, os.path.join(ROOT, "bench.py")] + bench_args)
    proc = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"), timeout=timeout,
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # rocprofv3 can end with SIGSEGV after the profiled program has finished
    # and its CSVs are complete: the run is used (the caller still needs its
    # CSVs) but the exit status is kept and written into the summary
    if proc.returncode in (-11, 139):
        PROFILER_CRASHES.append((" ".join(prof_args), proc.returncode))
    elif proc.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed ({proc.returncode}):\n{proc.stdout[-2000:]}")
    lines = [l for l in proc.stdout.splitlines() if l.startswith("{")]
    return " ".join(prof_args), (json.loads(lines[-1]) if lines else None)


# (profiler arguments, exit status) of every profiler run of this process that ended with SIGSEGV
PROFILER_CRASHES = []


def _crash_note():
    if not PROFILER_CRASHES:
        return "Profiler exit status: 0 for every run.\n"
    runs = "; ".join(f"`{a}` exited {rc}" for a, rc in PROFILER_CRASHES)
    return (f"Profiler exit status: {runs} (SIGSEGV of rocprofv3 after the program finished; the CSVs it "
            f"had written were complete and are the ones used).\n")


def _counter_means(out_dir):
    """{(is_attention_kernel, is_copy_kernel, counter): mean value per dispatch}."""
    vals = {}
    for f in glob.glob(os.path.join(out_dir, "**", "*_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            key = ("fa_fwd_kernel" in r["Kernel_Name"], "copyBuffer" in r["Kernel_Name"], r["Counter_Name"])
            vals.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def _display(cmd_args, bench_args):
    return ("cd /tmp && rocprofv3 " + cmd_args + " --output-format csv -d <out> -o <tag> -- python3 <repo>/bench.py "
            + " ".join(bench_args))


def tag_of(shape):
    B, H, N, d, dt, causal = shape
    return f"fa_fwd_{dt}_b{B}h{H}n{N}d{d}" + ("_causal" if causal else "")


def record(shape, out_dir, counters=True):
    os.makedirs(out_dir, exist_ok=True)
    B, H, N, d, dt, causal = shape
    tag = tag_of(shape)
    flop = bench.flops(B, H, N, d, causal)
    e_in, e_out = (1, 2) if dt == "fp8" else (2, 2)
    algo = bench.algorithmic_bytes(B, H, N, d, e_in, e_out)
    desc = f"B={B} H={H} N={N} d={d} {dt} " + ("causal" if causal else "non-causal")

    with tempfile.TemporaryDirectory(dir="/tmp") as wd:
        bargs = _bench_args(shape)
        pargs, line = _profile(["--kernel-trace", "--stats"], bargs, os.path.join(wd, "trace"), "trace")
        stats = glob.glob(os.path.join(wd, "trace", "**", "*_kernel_stats.csv"), recursive=True)[0]
        text = open(stats).read().strip()
        row = [r for r in csv.DictReader(open(stats)) if "fa_fwd_kernel" in r["Name"]][0]
        avg_ns = float(row["AverageNs"])
        with open(os.path.join(out_dir, f"{tag}_kernel_stats.md"), "w") as f:
            f.write(f"# rocprofv3 kernel statistics: attention forward {desc}\n\n")
            f.write(f"Command (MI355X, repository root as `<repo>`):\n\n```\n{_display(pargs, bargs)}\n```\n\n")
            f.write(f"`kernel_stats.csv` as written by rocprofv3:\n\n```\n{text}\n```\n\n")
            f.write(f"Average duration of the attention kernel {avg_ns / 1e3:.1f} us -> "
                    f"{flop / avg_ns / 1e3:.1f} TFLOP/s ({flop / 1e9:.1f} GFLOP per launch).")
            if line:
                f.write(f"  The same command's bench.py line (HIP events over the timed region, profiler attached) "
                        f"reported {line['ms_per_step'] * 1e3:.1f} us per step, {line['value']:.1f} TFLOP/s.")
            f.write(f"\n\nKernel source hash (bench.kernel_source_hash): {bench.kernel_source_hash()}\n")
            f.write(_crash_note())
        if not counters:
            return

        raw, factor, cmds = {}, {}, []
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            bargs = _bench_args(shape, 3, 1, ["--copy-calib-mib", str(COPY_MIB)])
            pargs, _ = _profile(["--pmc", counter], bargs, os.path.join(wd, counter), counter.lower())
            cmds.append(_display(pargs, bargs))
            c = _counter_means(os.path.join(wd, counter))
            raw[counter] = c[(True, False, counter)]
            raw[counter + "_copy"] = c[(False, True, counter)]
            factor[counter] = COPY_MIB * 1024 / raw[counter + "_copy"]
        bargs = _bench_args(shape, 3, 1)
        pargs, _ = _profile(["--pmc"] + SQ_COUNTERS, bargs, os.path.join(wd, "sq"), "sq")
        sq_cmd = _display(pargs, bargs)
        sq = {k[2]: v for k, v in _counter_means(os.path.join(wd, "sq")).items() if k[0]}
        pargs, _ = _profile(["--pmc"] + list(INSTR_COUNTERS.values()), bargs, os.path.join(wd, "insts"), "insts")
        inst_cmd = _display(pargs, bargs)
        ic = {k[2]: v for k, v in _counter_means(os.path.join(wd, "insts")).items() if k[0]}
        instructions = {key: ic.get(name) for key, name in INSTR_COUNTERS.items()}

    fetch = round(raw["FETCH_SIZE"] * 1024 * factor["FETCH_SIZE"])
    write = round(raw["WRITE_SIZE"] * 1024 * factor["WRITE_SIZE"])
    traffic = {
        "kernel": row["Name"], "workload": f"attention forward {desc}",
        "kernel_source_sha256_16": bench.kernel_source_hash("fwd"),
        "fetch_size_kib_per_dispatch_raw": raw["FETCH_SIZE"], "write_size_kib_per_dispatch_raw": raw["WRITE_SIZE"],
        "calibration": {"reference_kernel": f"__amd_rocclr_copyBuffer (device copy of {COPY_MIB} MiB)",
                        "expected_kib_each_way": COPY_MIB * 1024,
                        "fetch_size_kib_raw": raw["FETCH_SIZE_copy"], "write_size_kib_raw": raw["WRITE_SIZE_copy"],
                        "fetch_factor": round(factor["FETCH_SIZE"], 5), "write_factor": round(factor["WRITE_SIZE"], 5)},
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write, "bytes_per_launch": fetch + write,
        "algorithmic_bytes_per_launch": algo, "ratio_to_algorithmic": round((fetch + write) / algo, 4),
        "commands": cmds,
        "instructions": instructions, "instruction_counters": INSTR_COUNTERS, "instruction_command": inst_cmd,
    }
    with open(os.path.join(out_dir, f"{tag}_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    grbm = sq.get("GRBM_GUI_ACTIVE", float("nan"))
    mfma = sq.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
    with open(os.path.join(out_dir, f"{tag}_counters.md"), "w") as f:
        f.write(f"# rocprofv3 counters: attention forward {desc}\n\nKernel: `{row['Name']}`\n\n")
        f.write("## HBM traffic (FETCH_SIZE, WRITE_SIZE; one counter per run)\n\n")
        for c in cmds:
            f.write(f"```\n{c}\n```\n\n")
        f.write(f"Calibration: the same run performs one {COPY_MIB} MiB device copy (`__amd_rocclr_copyBuffer`), "
                f"which must read and write {COPY_MIB * 1024} KiB.  It reads FETCH_SIZE = {raw['FETCH_SIZE_copy']:.1f} "
                f"KiB and WRITE_SIZE = {raw['WRITE_SIZE_copy']:.1f} KiB, so FETCH_SIZE is scaled by "
                f"{factor['FETCH_SIZE']:.4f} and WRITE_SIZE by {factor['WRITE_SIZE']:.4f}.\n\n")
        f.write("| | raw KiB per dispatch | scaled bytes per launch |\n|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {raw['FETCH_SIZE']:.1f} | {fetch} |\n| WRITE_SIZE | {raw['WRITE_SIZE']:.1f} | {write} |\n")
        f.write(f"| total | | {fetch + write} |\n\n")
        f.write(f"Algorithmic bytes per launch (Q, K, V read once, O and lse written once): {algo}.  "
                f"Measured / algorithmic = {(fetch + write) / algo:.4f}.\n\n")
        f.write(f"## SQ counters (one run)\n\n```\n{sq_cmd}\n```\n\n| counter | mean per dispatch |\n|---|---|\n")
        for k in sorted(sq):
            f.write(f"| {k} | {sq[k]:.0f} |\n")
        f.write(f"\n## Instruction counts (one run; per-wave instructions summed over the dispatch)\n\n"
                f"```\n{inst_cmd}\n```\n\n| counter | mean per dispatch |\n|---|---|\n")
        for k, name in INSTR_COUNTERS.items():
            v = instructions.get(k)
            f.write(f"| {name} | {'n/a' if v is None else f'{v:.0f}'} |\n")
        f.write(f"\nGRBM_GUI_ACTIVE is summed over the 8 XCDs ({grbm / 8:.0f} cycles each); MFMA busy / "
                f"(cycles x 1024 SIMDs) = {100 * mfma / (grbm / 8 * 1024):.1f}% under the counter run.\n")
        f.write(_crash_note())


def record_mode(mode, mode_arg, tag, out_dir):
    """Kernel statistics of bench.py --MODE ARG (one step may launch several kernels)."""
    os.makedirs(out_dir, exist_ok=True)
    bargs = ["--no-sweep", "--no-cpu", f"--{mode}", mode_arg]
    with tempfile.TemporaryDirectory(dir="/tmp") as wd:
        pargs, line = _profile(["--kernel-trace", "--stats"], bargs, os.path.join(wd, "trace"), "trace")
        stats = glob.glob(os.path.join(wd, "trace", "**", "*_kernel_stats.csv"), recursive=True)[0]
        text = open(stats).read().strip()
        rows = [r for r in csv.DictReader(open(stats)) if r["Name"].startswith("void fa::")]
    # the kernels launched once per step are the most-called ones (a kernel
    # called once, like the forward pass that feeds the backward, is set-up)
    most = max(int(r["Calls"]) for r in rows)
    per_step_ns = sum(float(r["AverageNs"]) for r in rows if int(r["Calls"]) == most)
    with open(os.path.join(out_dir, f"{tag}_kernel_stats.md"), "w") as f:
        f.write(f"# rocprofv3 kernel statistics: bench.py --{mode} {mode_arg}\n\n")
        f.write(f"Command (MI355X, repository root as `<repo>`):\n\n```\n{_display(pargs, bargs)}\n```\n\n")
        f.write(f"`kernel_stats.csv` as written by rocprofv3:\n\n```\n{text}\n```\n\n")
        for r in rows:
            f.write(f"* `{r['Name']}`: {int(r['Calls'])} calls, average {float(r['AverageNs']) / 1e3:.1f} us\n")
        if line:
            flop = line["value"] * 1e12 * line["ms_per_step"] * 1e-3
            f.write(f"\nThe kernels of one step take {per_step_ns / 1e3:.1f} us on average -> "
                    f"{flop / per_step_ns / 1e3:.1f} TFLOP/s at bench.py's {flop / 1e9:.1f} GFLOP per step.  The same "
                    f"command's bench.py line (HIP events over the timed region, profiler attached) reported "
                    f"{line['ms_per_step'] * 1e3:.1f} us per step, {line['value']:.1f} TFLOP/s.\n")
        fam = MODE_FAMILY[mode]
        f.write(f"\nKernel source hash (bench.kernel_source_hash(\"{fam}\")): {bench.kernel_source_hash(fam)}\n")
        f.write(_crash_note())


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out-dir", required=True)
    ap.add_argument("--shape", default=None, help="B,H,N,d,dtype,causal (default: the headline workload)")
    ap.add_argument("--mode", default=None, choices=["varlen", "dropout", "bwd", "proj"])
    ap.add_argument("--mode-arg", default=None, help="the argument bench.py takes for --MODE")
    ap.add_argument("--tag", default=None, help="file name stem for --mode")
    ap.add_argument("--no-counters", action="store_true",
                    help="kernel statistics only (no FETCH_SIZE / WRITE_SIZE / SQ / instruction counter runs)")
    args = ap.parse_args(argv)
    if args.mode:
        record_mode(args.mode, args.mode_arg, args.tag, args.out_dir)
        print(f"recorded {args.tag} into {args.out_dir}", flush=True)
        return 0
    shape = HEADLINE
    if args.shape:
        B, H, N, d, dt, causal = args.shape.split(",")
        shape = (int(B), int(H), int(N), int(d), dt, causal in ("1", "true"))
    record(shape, args.out_dir, counters=not args.no_counters)
    print(f"recorded {tag_of(shape)} into {args.out_dir}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

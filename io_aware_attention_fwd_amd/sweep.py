"""Tile-shape / occupancy sweep of the forward kernel, recorded with rocprofv3.

    python -m io_aware_attention_fwd_amd.sweep [--workloads ...] [--out DIR]

For every tile variant compiled into libfa.so (the ``kVariants`` table of
``csrc/fa_fwd.hip``, selected per call with ``FA_TILE``) and every workload,
this runs ``bench.py --shape ...`` three times under ``rocprofv3``:

1. ``--kernel-trace --stats`` with bench.py's default warm-up and step counts
   (the clock needs tens of milliseconds of load to leave its idle level):
   average kernel duration -> TFLOP/s;
2. ``--pmc`` SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_LDS_BANK_CONFLICT
   SQ_LDS_IDX_ACTIVE: matrix-core utilisation and LDS bank conflicts;
3. ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (one counter per run), the
   same run also timing a 256 MiB device copy whose known size calibrates
   the counters.

It prints one JSON object per (variant, workload) and writes a markdown
table.  It needs a GPU and rocprofv3; each profiler run is a child process
started from /tmp with a time limit.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BENCH = os.path.join(ROOT, "bench.py")
DEFAULT_WORKLOADS = ["8,32,1024,64,f16,0", "8,32,8192,64,f16,0", "8,32,4096,64,bf16,1",
                     "8,32,8192,64,fp8,0", "4,32,8192,128,bf16,0", "2,16,16384,128,bf16,1", "4,32,8192,128,fp8,0"]
COPY_MIB = 256


VARIANTS_H = os.path.join(HERE, "csrc", "fa_variants.h")


def variants():
    """FA_TILE strings of the compiled variants, read from the variant table."""
    src = open(VARIANTS_H).read()
    body = re.search(r"kVariants\[\] = \{(.*?)\};", src, re.S).group(1)
    return ["x".join(t.split(",")).replace(" ", "") for t in re.findall(r"\{([\d,\s]+)\}", body)]


def variants_per_d():
    """(d, FA_TILE) of every shape compiled for head dimension d."""
    src = open(VARIANTS_H).read()
    only = {n: {int(i) for i in re.findall(r"v == (\d+)", re.search(n + r"\(int v\) \{(.*?)\}", src).group(1))}
            for n in ("d64_only", "d128_only")}
    return [(d, t) for d in (64, 128) for i, t in enumerate(variants())
            if not (i in only["d64_only"] and d != 64) and not (i in only["d128_only"] and d != 128)]


def _rocprof(args, out_dir, tag, env, timeout):
    cmd = ["rocprofv3"] + args + ["--output-format", "csv", "-d", out_dir, "-o", tag, "--",
                                  sys.executable, BENCH, "--no-sweep", "--no-cpu"]
    return cmd


def _run(cmd, env, timeout, crashes):
    """Run one profiler command.  rocprofv3 can end with SIGSEGV (-11 / 139)
    after the profiled program has finished and its CSVs are complete; such a
    run is kept (the caller still needs its CSVs, or raises without them) but
    its exit status is appended to ``crashes``, so the row it feeds says so."""
    proc = subprocess.run(cmd, cwd="/tmp", env=env, timeout=timeout, stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True)
    if proc.returncode in (-11, 139):
        crashes.append(proc.returncode)
    elif proc.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed ({proc.returncode}):\n{proc.stdout[-2000:]}")
    return proc.stdout


KERNEL_RE = re.compile(r"fa_fwd_kernel<[^,]+, (\d+), (?:true|false), (\d+), (\d+), (\d+), (\d+), (\d+)")


def tile_of_kernel(name):
    """The FA_TILE string (QWxNWxBCxSCHEDxWPE) of a forward kernel instance name, or None."""
    m = KERNEL_RE.search(name)
    return "x".join(m.groups()[1:]) if m else None


def _counters(path, kernel_substr="fa_fwd_kernel"):
    vals = {}
    for f in glob.glob(os.path.join(path, "*_counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            vals.setdefault((kernel_substr in r["Kernel_Name"], "copyBuffer" in r["Kernel_Name"], r["Counter_Name"]),
                            []).append(float(r["Counter_Value"]))
    return vals


def _mean(v):
    return sum(v) / len(v) if v else float("nan")


def measure(tile, workload, workdir, timeout=300):
    B, H, N, d, dtype, causal = workload.split(",")
    B, H, N, d = int(B), int(H), int(N), int(d)
    causal = causal in ("1", "true")
    env = dict(os.environ, FA_TILE=tile, TMPDIR="/tmp")
    shape = ["--shape", workload]
    res = {"tile": tile, "workload": workload}
    crashes = []
    # 1. duration
    out = os.path.join(workdir, "trace")
    # bench.py's default warm-up and steps, so the clock has left its idle level
    _run(_rocprof(["--kernel-trace", "--stats"], out, "t", env, timeout) + shape, env, timeout, crashes)
    rows = [r for f in glob.glob(os.path.join(out, "*_kernel_stats.csv")) for r in csv.DictReader(open(f))
            if "fa_fwd_kernel" in r["Name"]]
    if not rows:
        raise RuntimeError(f"no forward kernel in the kernel trace of {workload} with FA_TILE={tile}")
    avg_ns = float(rows[0]["AverageNs"])
    flop = 4.0 * B * H * N * N * d / (2 if causal else 1)
    res["kernel"] = rows[0]["Name"]
    # the instance that ran, from its name: a request the library did not honour shows here
    res["tile_ran"] = tile_of_kernel(rows[0]["Name"])
    res["avg_us"] = round(avg_ns / 1e3, 2)
    res["tflops"] = round(flop / avg_ns / 1e3, 1)
    # 2. SQ counters
    out = os.path.join(workdir, "sq")
    _run(_rocprof(["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"],
                  out, "s", env, timeout) + shape + ["--steps", "2", "--warmup", "1"], env, timeout, crashes)
    c = _counters(out)
    mfma = _mean(c.get((True, False, "SQ_VALU_MFMA_BUSY_CYCLES"), []))
    grbm = _mean(c.get((True, False, "GRBM_GUI_ACTIVE"), []))  # summed over the 8 XCDs
    res["mfma_util"] = round(mfma / (grbm / 8 * 1024), 4) if grbm == grbm and grbm > 0 else None
    res["lds_bank_conflict_cycles"] = _mean(c.get((True, False, "SQ_LDS_BANK_CONFLICT"), []))
    res["lds_active_cycles"] = _mean(c.get((True, False, "SQ_LDS_IDX_ACTIVE"), []))
    # 3. HBM traffic, calibrated on a device copy of known size
    traffic = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = os.path.join(workdir, counter.lower())
        _run(_rocprof(["--pmc", counter], out, counter.lower(), env, timeout) + shape +
             ["--steps", "2", "--warmup", "1", "--copy-calib-mib", str(COPY_MIB)], env, timeout, crashes)
        c = _counters(out)
        copy = _mean(c.get((False, True, counter), []))
        factor = COPY_MIB * 1024 / copy if copy > 0 else float("nan")
        traffic[counter] = _mean(c.get((True, False, counter), [])) * 1024 * factor
    res["hbm_bytes"] = round(traffic["FETCH_SIZE"] + traffic["WRITE_SIZE"])
    res["hbm_gbs"] = round(res["hbm_bytes"] / (avg_ns * 1e-9) / 1e9, 1)
    res["profiler_crashes"] = crashes  # exit statuses of profiler runs that ended with SIGSEGV
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workloads", nargs="*", default=DEFAULT_WORKLOADS, help="B,H,N,d,dtype,causal ...")
    ap.add_argument("--tiles", nargs="*", default=None, help="FA_TILE strings (default: every compiled variant)")
    ap.add_argument("--out", default=None, help="write a markdown table here")
    args = ap.parse_args(argv)
    tiles = args.tiles or variants()
    compiled = set(variants_per_d())
    results = []
    for w in args.workloads:
        for t in tiles:
            d = int(w.split(",")[3])
            if (d, t) not in compiled:
                continue  # not compiled for this head dimension
            with tempfile.TemporaryDirectory(dir="/tmp") as wd:
                r = measure(t, w, wd)
            print(json.dumps(r), flush=True)
            results.append(r)
    if args.out:
        with open(args.out, "w") as f:
            f.write("| workload (B,H,N,d,dtype,causal) | FA_TILE (QW x NW x BC x schedule x waves/SIMD) | instance "
                    "that ran | us | TFLOP/s | MFMA busy | LDS bank-conflict cycles | LDS active cycles | HBM bytes "
                    "| HBM GB/s | profiler SIGSEGV |\n")
            f.write("|---|---|---|---|---|---|---|---|---|---|---|\n")
            for r in results:
                ran = r["tile_ran"] if r["tile_ran"] == r["tile"] else f"**{r['tile_ran']}** (not the request)"
                crash = ", ".join(str(c) for c in r["profiler_crashes"]) or "none"
                f.write(f"| {r['workload']} | {r['tile']} | {ran} | {r['avg_us']} | {r['tflops']} | {r['mfma_util']} | "
                        f"{r['lds_bank_conflict_cycles']:.0f} | {r['lds_active_cycles']:.0f} | {r['hbm_bytes']} | "
                        f"{r['hbm_gbs']} | {crash} |\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())

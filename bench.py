"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  A step is one ``fa_fwd`` call (the whole forward pass:
Q tile load, K/V streaming, Q K^T, mask, online softmax, P V, epilogue) on
B=8, H=32, N=1024, d=64 binary16 inputs, non-causal, scale 1/8, drawn i.i.d.
N(0,1) from seed 0.  Inputs are resident in device memory before the timed
region.  The shader clock needs tens of milliseconds of load to leave its
idle level, so the GPU is first kept busy with plain device matmuls
(``--clock-ms``, 150 by default; not the benchmarked call); then come W
untimed warm-up steps (500 by default) and K timed steps (200 by default),
timed with HIP events on the stream the kernel runs on, between two device
synchronisations.

Throughput is 4*B*H*N^2*d FLOP per step (halved for causal) / time.  The line
also carries per-call median / min / p90 times; the five configurations
(B1 H2 N128 d64 f16; B8 H32 N1024 d64 f16; B8 H32 N4096 d64 bf16 causal;
B8 H32 N8192 d64 fp8 in, bf16 out; B2 H16 N16384 d128 bf16 causal) as
entries of their own, each with its fraction of the dtype's dense
matrix-core peak, algorithmic HBM GB/s, HBM traffic from committed
rocprofv3 counters when they were taken on the current kernel source, the
LDS and vector-ALU ceilings, and the float64 CPU oracle timed on the host
cores (in full where that takes seconds, else on sampled (b, h) slices,
extrapolated); the sequence-length sweep N = 512..8192 at B=8, H=32, d=64
(the shape of the benchmark page's forward-time tables) plus d=128 and
causal points at N >= 4096, each after a 50 ms warm-up of its own; and the
shader and memory clock levels in use under load.

Other modes print one line each for the other entry points instead of the
headline: ``--shape`` (another dense forward shape), ``--varlen`` (packed
sequences), ``--dropout``, ``--bwd`` (the backward pass) and ``--proj`` (the
fused QKV projection); ``--copy-calib-mib`` adds a plain device copy used to
calibrate the HBM counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0}  # MI355X dense matrix-core peaks
HBM_PEAK_GBS = 8000.0
CLOCK_GHZ = 2.4          # the clock the MI355X peaks are quoted at
N_CU = 256
LDS_BYTES_PER_CLK = 128  # LDS read bandwidth per CU assumed for the LDS ceiling (CDNA3's documented figure)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "fa_fwd_f16_b8h32n1024d64_traffic.json")
_CSRC = os.path.join(ROOT, "io_aware_attention_fwd_amd", "csrc")
# the sources each kernel family is built from (a profile is current while their hash is unchanged)
KERNEL_FAMILIES = {
    "fwd": ["fa_fwd.hip", "fa_device.h", "fa_launch.h", "fa_variants.h"],
    "bwd": ["fa_bwd.hip", "fa_device.h", "fa_launch.h"],
    "proj": ["fa_proj.hip", "fa_device.h", "fa_launch.h"],
}
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in KERNEL_FAMILIES["fwd"]]

# The five configurations of the benchmark: (tag, B, H, N, d, dtype, causal); scale 1/sqrt(d).
CONFIGS = [("c1", 1, 2, 128, 64, "f16", False), ("c2", 8, 32, 1024, 64, "f16", False),
           ("c3", 8, 32, 4096, 64, "bf16", True), ("c4", 8, 32, 8192, 64, "fp8", False),
           ("c5", 2, 16, 16384, 128, "bf16", True)]


def flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def algorithmic_bytes(B, H, N, d, in_bytes, out_bytes):
    # Q, K, V read once, O written once, lse written once
    return (3 * in_bytes + out_bytes) * B * H * N * d + 4 * B * H * N


def kernel_source_hash(family="fwd"):
    """Hash of the sources one kernel family is built from ("fwd", "bwd" or "proj")."""
    paths = KERNEL_SOURCES if family == "fwd" else [os.path.join(_CSRC, f) for f in KERNEL_FAMILIES[family]]
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def record_tag(B, H, N, d, dtype, causal):
    """File stem of a forward workload's profiles under profiles/."""
    return f"fa_fwd_{dtype}_b{B}h{H}n{N}d{d}" + ("_causal" if causal else "")


def load_record(tag):
    """The committed rocprofv3 counter record of a workload, if it was taken on the current kernel source."""
    path = TRAFFIC_FILE if tag == record_tag(8, 32, 1024, 64, "f16", False) else os.path.join(PROFILES, f"{tag}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t


def lds_bytes_per_score(d, dtype, tile):
    """LDS operand bytes one score costs with the tile shape (QWxNWxBCxSCHEDxWPE) that runs: each wave
    reads the whole K and V tile once per tile for its QW query rows (and, with 64-row waves at d = 128
    and 16-bit values, its second 32-row block's Q operands)."""
    qw, _, bc = (int(x) for x in tile.split("x")[:3])
    e = 1 if dtype == "fp8" else 2
    b = d * 2 * e / qw
    if qw == 64 and d == 128 and dtype != "fp8":
        b += 32 * d * 2 / (qw * bc)
    return b


def secondary_ceilings(d, dtype, causal, fl, tile, rec):
    """Ceilings other than the matrix cores, in TFLOP/s at the quoted 2.4 GHz: the LDS operand reads
    (from the tile shape) and, where the counter record holds instruction counts, the vector ALU issue
    (4 cycles per wave64 instruction, 8 for an exponential or logarithm) per launch."""
    out = {"lds_bytes_per_score": round(lds_bytes_per_score(d, dtype, tile), 3),
           "lds_ceiling_tflops": round(N_CU * LDS_BYTES_PER_CLK * CLOCK_GHZ * 1e9 / lds_bytes_per_score(d, dtype, tile)
                                       * 4 * d / 1e12, 1),
           "lds_assumption": f"{LDS_BYTES_PER_CLK} B/clk per CU, {N_CU} CUs, {CLOCK_GHZ} GHz"}
    counts = (rec or {}).get("instructions")
    if counts and counts.get("valu") is not None:
        trans = counts.get("valu_trans") or 0
        other = counts["valu"] - trans - (counts.get("mfma") or 0)
        cycles = 4 * other + 8 * trans
        t = cycles / (4 * N_CU) / (CLOCK_GHZ * 1e9)
        scores = fl / (4 * d)
        out.update({"valu_insts_per_score": round(64 * other / scores, 3),
                    "trans_insts_per_score": round(64 * trans / scores, 3),
                    "valu_ceiling_tflops": round(fl / t / 1e12, 1)})
    return out


def progress(msg):
    """One line per stage on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_calls(fn, warmup, steps, stream):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def warm(fn, seconds=0.05):
    """Untimed back-to-back calls for at least `seconds` of wall time, so that
    the shader clock has left its idle level (it needs tens of milliseconds
    of load) before a measurement, e.g. after inputs were built on the host."""
    import torch

    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def condition_clock(ms):
    """Keep the GPU busy with plain device matmuls (not the benchmarked call) for about ``ms``
    milliseconds: the shader clock needs tens of milliseconds of load to leave its idle level, and
    a timed region of a few milliseconds that starts on an idle clock reads ~20 % low."""
    import torch

    if ms <= 0:
        return
    a = torch.randn(2048, 2048, device="cuda", dtype=torch.float16)
    b = torch.empty_like(a)
    torch.mm(a, a, out=b)  # the matmul library's first call sets itself up: kept out of the window
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            torch.mm(a, a, out=b)
        torch.cuda.synchronize()
    del a, b


def time_each(fn, warmup, steps, stream):
    """Per-call durations (ms) from an event pair around every call."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def summarize(ms_list, fl, peak):
    ms = sorted(ms_list)
    med = float(np.median(ms))
    p90 = float(np.percentile(ms, 90))
    t = fl / (med * 1e-3) / 1e12
    return {"ms_median": round(med, 4), "ms_min": round(ms[0], 4), "ms_p90": round(p90, 4),
            "tflops": round(t, 1), "frac_of_peak": round(t / peak, 4)}


def gpu_clock_state(busy_fn=None):
    """Shader and memory clock levels from the amdgpu sysfs tables (the source rocm-smi reads),
    sampled while ``busy_fn`` keeps the GPU loaded, so the level in use under load is the one marked."""
    import glob

    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return None
    if busy_fn is not None:
        busy_fn()
        time.sleep(0.05)
    out = {}
    for p in paths:
        dev = p.split("/")[4]
        st = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(os.path.dirname(p), name)) as f:
                    lines = f.read().split("\n")
                cur = [l for l in lines if l.rstrip().endswith("*")]
                st[name[7:]] = cur[0].split(":", 1)[1].strip(" *") if cur else None
                st[name[7:] + "_levels"] = [l.split(":", 1)[1].strip(" *") for l in lines if ":" in l]
            except OSError:
                st[name[7:]] = None
        out[dev] = st
    return out


def make_call(B, H, N, d, dtype, causal, scale, seed=0, x=None):
    import torch

    from io_aware_attention_fwd_amd import _lib, gen

    if x is None:
        x = gen.make(B, H, N, d, dtype, seed=seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]

    def dev(a):
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        if dtype == "fp8":
            return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16 if dtype == "fp8" else tdt, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    ds = x.descale
    dt = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16, "fp8": _lib.FA_DTYPE_FP8_E4M3}[dtype]
    qp, kp, vp, op, lp = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()
    lib = _lib.load()

    if dtype == "fp8":
        def call():
            rc = lib.fa_fwd_fp8(qp, kp, vp, op, lp, B, H, N, d, scale, int(causal), ds["q"], ds["k"], ds["v"], s)
            if rc:
                raise _lib.FaError(rc)
    else:
        def call():
            rc = lib.fa_fwd(qp, kp, vp, op, lp, B, H, N, d, scale, int(causal), dt, s)
            if rc:
                raise _lib.FaError(rc)
    return call, stream, (x, q, k, v, o, lse)


def make_call_varlen(lengths, H, d, dtype, causal, scale, seed=0):
    """fa_fwd_varlen on packed [total, H, d] sequences of the given lengths."""
    import torch

    from io_aware_attention_fwd_amd import _lib, gen

    x, cu = gen.make_packed(lengths, H, d, dtype, seed=seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]

    def dev(a):
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        if dtype == "fp8":
            return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
        return torch.from_numpy(a).cuda()

    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    total = q.shape[0]
    o = torch.empty((total, H, d), dtype=torch.bfloat16 if dtype == "fp8" else tdt, device="cuda")
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    cu_t = torch.from_numpy(cu).cuda()
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    dt = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16, "fp8": _lib.FA_DTYPE_FP8_E4M3}[dtype]
    eff = scale * (x.descale["q"] * x.descale["k"] if dtype == "fp8" else 1.0)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu_t.data_ptr(), len(lengths), H,
            total, max(lengths), d, eff, int(causal), dt, s)
    lib = _lib.load()

    def call():
        rc = lib.fa_fwd_varlen(*args)
        if rc:
            raise _lib.FaError(rc, "fa_fwd_varlen")
    return call, stream, (x, cu, q, k, v, o, lse, cu_t)


def oracle_threads():
    """BLAS threads for the oracle: the CPUs this process may run on (sched_getaffinity), capped by
    OMP_NUM_THREADS where the host sets it to its share; returns the count actually in use."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        threadpool_limits(limits=n, user_api="blas")
        used = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(used) if used else n
    except Exception:  # pragma: no cover
        return n


def cpu_baseline_varlen(x, cu, causal, scale, budget_s):
    """The float64 oracle on (sequence, head) slices of a packed batch for about
    ``budget_s`` seconds, extrapolated to the whole batch by FLOPs."""
    import oracle

    H, d = x.q.shape[1], x.q.shape[2]
    cores = oracle_threads()
    lengths = np.diff(cu)
    total_fl = sum(flops(1, H, int(n), d, causal) for n in lengths)
    done_fl, n_slices, t0 = 0.0, 0, time.perf_counter()
    for b in range(len(lengths)):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        for h in range(H):
            qkv = [oracle.dequantize(a[r0:r1, h], x.dtype, x.descale[n]) for a, n in ((x.q, "q"), (x.k, "k"), (x.v, "v"))]
            oracle.attention_slice(qkv[0], qkv[1], qkv[2], scale, causal)
            done_fl += flops(1, 1, r1 - r0, d, causal)
            n_slices += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    rate = done_fl / el
    return {"value": rate / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"{n_slices} (sequence, head) slices of the packed batch ({done_fl / 1e9:.1f} GFLOP, "
                      f"{x.dtype} inputs, float64 math) timed in {el:.1f} s; whole batch extrapolated by FLOPs to "
                      f"{total_fl / rate:.1f} s"}


def cpu_baseline(x, causal, scale, budget_s):
    """The float64 oracle on the (b, h) slices of ``x``, cycling through them
    until ``budget_s`` seconds have passed (or one pass, if that takes longer)."""
    import oracle

    B, H, N, d = x.shape
    dtype = x.dtype
    cores = oracle_threads()
    done, t0 = 0, time.perf_counter()
    while True:
        b, h = divmod(done % (B * H), H)
        qkv = [oracle.dequantize(a[b, h], dtype, x.descale[n]) for a, n in ((x.q, "q"), (x.k, "k"), (x.v, "v"))]
        oracle.attention_slice(qkv[0], qkv[1], qkv[2], scale, causal)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_slice = el / done
    full_s = per_slice * B * H
    tflops = flops(B, H, N, d, causal) / full_s / 1e12
    return {"value": tflops, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"{done} slice evaluations ({done / (B * H):.2f} passes over the {B * H} (b,h) slices) of N={N}, "
                      f"d={d} ({dtype} inputs, float64 math) in {el:.1f} s; one full workload = {full_s:.2f} s "
                      f"({full_s * 1e3:.0f} ms per step)"}


def cpu_baseline_sampled(x, causal, scale, budget_s, slices):
    """The float64 oracle on the given (b, h) slices, in order, until ``budget_s`` seconds have passed
    (at least one slice), extrapolated to all B*H slices: the whole workload takes hours of host time
    at N >= 4096, so only a bounded sample is timed."""
    import oracle

    B, H, N, d = x.shape
    cores = oracle_threads()
    done, t0 = 0, time.perf_counter()
    for b, h in slices:
        qkv = [oracle.dequantize(a[b, h], x.dtype, x.descale[n]) for a, n in ((x.q, "q"), (x.k, "k"), (x.v, "v"))]
        oracle.attention_slice(qkv[0], qkv[1], qkv[2], scale, causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    full_s = el / done * B * H
    return {"value": flops(B, H, N, d, causal) / full_s / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "ms_per_step_extrapolated": round(full_s * 1e3, 1),
            "sample": f"{done} of the sampled (b,h) slices {slices[:done]} of N={N}, d={d} ({x.dtype} inputs, float64 "
                      f"math) timed in {el:.1f} s; the {B * H} slices extrapolated x{B * H / done:g} to "
                      f"{full_s:.1f} s per step"}


def load_traffic(_unused=None):
    """HBM bytes per launch of the headline workload from the committed rocprofv3 counter record, if current."""
    t = load_record(record_tag(8, 32, 1024, 64, "f16", False))
    return None if t is None else t.get("bytes_per_launch")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Untimed warm-up long enough for the shader clock to leave its idle level
    # (about 45 ms of back-to-back calls for the headline workload): with 10
    # calls the timed region starts before the clock has ramped and the
    # headline reads ~20 % low; 500 and 2000 warm-up calls agree within 1 %.
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-sweep", action="store_true", help="skip the configurations and the N=512..8192 sweep")
    ap.add_argument("--clock-ms", type=float, default=150.0,
                    help="milliseconds of device matmuls before the warm-up calls, to bring the shader clock "
                         "up from idle (0: none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--shape", default=None,
                    help="B,H,N,d,dtype,causal to time another shape instead of the headline one "
                         "(e.g. 2,16,16384,128,bf16,1); the JSON line then names that workload")
    ap.add_argument("--varlen", default=None,
                    help="COUNT,LO,HI,H,d,dtype,causal: time fa_fwd_varlen on COUNT packed sequences with lengths "
                         "drawn uniformly from [LO, HI] (seed 0) instead of the headline shape")
    ap.add_argument("--bwd", default=None,
                    help="B,H,N,d,dtype,causal: time the backward pass fa_bwd (after one forward call that "
                         "produces O and lse) instead of the headline shape")
    ap.add_argument("--dropout", default=None,
                    help="B,H,N,d,dtype,causal,p: time fa_fwd_dropout at drop rate p (seed 1234, offset 0) "
                         "instead of the headline shape")
    ap.add_argument("--proj", default=None,
                    help="B,N,D,H,d,dtype: time the fused QKV projection fa_qkv_proj (with bias) instead of the "
                         "headline shape")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (reference kernel for HBM counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward pass has no multi-GPU path in this library)", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.varlen:
        return main_varlen(args)
    if args.bwd:
        return main_bwd(args)
    if args.dropout:
        return main_dropout(args)
    if args.proj:
        return main_proj(args)

    B, H, N, d, dtype, causal = 8, 32, 1024, 64, "f16", False
    if args.shape:
        f = args.shape.split(",")
        B, H, N, d, dtype, causal = int(f[0]), int(f[1]), int(f[2]), int(f[3]), f[4], f[5] in ("1", "true", "True")
    scale = 1.0 / math.sqrt(d)
    progress(f"inputs B={B} H={H} N={N} d={d} {dtype} causal={int(causal)}")
    call, stream, keep = make_call(B, H, N, d, dtype, causal, scale)
    if args.copy_calib_mib:
        n = args.copy_calib_mib * 2 ** 20 // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    condition_clock(args.clock_ms)
    ms = time_calls(call, args.warmup, args.steps, stream)
    fl = flops(B, H, N, d, causal)
    peak = PEAK_TFLOPS[dtype]
    per_call = summarize(time_each(call, 2, min(args.steps, 50), stream), fl, peak)
    tflops = fl / (ms * 1e-3) / 1e12
    algo_bytes = algorithmic_bytes(B, H, N, d, 1 if dtype == "fp8" else 2, 2)

    from io_aware_attention_fwd_amd import _lib

    def point(pb, ph, n, dd, dt, cz, x=None):
        """Time one workload (after a 50 ms warm-up of its own); returns (entry, call, kept), where
        kept holds the host inputs and the device tensors the call's raw pointers refer to: the
        caller keeps it alive for as long as it may launch the call again."""
        c2, st2, keep2 = make_call(pb, ph, n, dd, dt, cz, 1.0 / math.sqrt(dd), x=x)
        warm(c2)
        fl2 = flops(pb, ph, n, dd, cz)
        r = summarize(time_each(c2, 0, 20 if n >= 4096 else 50, st2), fl2, PEAK_TFLOPS[dt])
        ab = algorithmic_bytes(pb, ph, n, dd, 1 if dt == "fp8" else 2, 2)
        tile = _lib.fwd_tile(n, dd, cz, {"f16": 0, "bf16": 1, "fp8": 2}[dt])
        e = {"B": pb, "H": ph, "N": n, "d": dd, "dtype": dt, "causal": cz, "tile": tile, **r,
             "peak_tflops": PEAK_TFLOPS[dt], "algorithmic_bytes": ab,
             "algorithmic_hbm_gbs": round(ab / (r["ms_median"] * 1e-3) / 1e9, 1)}
        return e, c2, keep2

    configs, sweep = [], []
    clocks = None
    if not args.no_sweep and not args.shape:
        # the five configurations, each a first-class entry with its own roofline figures and oracle baseline
        for tag, pb, ph, n, dd, dt, cz in CONFIGS:
            progress(f"config {tag} B={pb} H={ph} N={n} d={dd} {dt} causal={int(cz)}")
            e, c2, kept = point(pb, ph, n, dd, dt, cz)
            x2 = kept[0]
            fl2 = flops(pb, ph, n, dd, cz)
            rec = load_record(record_tag(pb, ph, n, dd, dt, cz))
            e = {"config": tag, **e,
                 "hbm_traffic_bytes": None if rec is None else rec.get("bytes_per_launch"),
                 "hbm_traffic_ratio_to_algorithmic": None if rec is None else rec.get("ratio_to_algorithmic"),
                 "secondary_ceilings": secondary_ceilings(dd, dt, cz, fl2, e["tile"], rec)}
            if dt == "fp8":
                # P V runs on bfloat16 matrix instructions (fp8 Q K^T), so the dtype's own ceiling is the
                # harmonic mix of the two peaks over equal halves of the FLOPs
                e["mixed_peak_tflops"] = round(2 / (1 / PEAK_TFLOPS["fp8"] + 1 / PEAK_TFLOPS["bf16"]), 1)
                e["frac_of_mixed_peak"] = round(e["tflops"] / e["mixed_peak_tflops"], 4)
            if clocks is None and n >= 4096:
                def busy(c=c2):
                    for _ in range(30):
                        c()
                clocks = gpu_clock_state(busy)
                torch.cuda.synchronize()
            if not args.no_cpu:
                progress(f"config {tag}: cpu baseline (oracle)")
                if pb * ph * n <= 8 * 32 * 1024:
                    e["cpu_baseline"] = cpu_baseline(x2, cz, 1.0 / math.sqrt(dd), args.cpu_budget / 3)
                else:
                    import oracle

                    e["cpu_baseline"] = cpu_baseline_sampled(x2, cz, 1.0 / math.sqrt(dd), args.cpu_budget / 3,
                                                             oracle.slice_sample(pb, ph))
            configs.append(e)
            del x2, c2, kept  # the call is not launched again: its tensors may go
            torch.cuda.empty_cache()
        # the benchmark page's forward-time table shape (B=8, H=32, d=64, N=512..8192, no mask) and the
        # N >= 4096 head-dimension 64/128 points, causal and bfloat16 too (c2 and c4 are entries above)
        points = [(B, H, n, 64, dtype, False) for n in (512, 2048, 4096, 8192)]
        points += [(B, H, 8192, 64, "bf16", True), (B, H, 4096, 128, "f16", False),
                   (B, H, 8192, 128, "bf16", False), (B, H, 8192, 128, "bf16", True)]
        for pb, ph, n, dd, dt, cz in points:
            progress(f"sweep point B={pb} H={ph} N={n} d={dd} {dt} causal={int(cz)}")
            e, _, kept = point(pb, ph, n, dd, dt, cz)
            sweep.append(e)
            del kept
            torch.cuda.empty_cache()
    if clocks is None:
        def busy():
            for _ in range(max(1, int(50e-3 / max(ms * 1e-3, 1e-6)))):
                call()
        clocks = gpu_clock_state(busy)
        torch.cuda.synchronize()

    rec = load_record(record_tag(B, H, N, d, dtype, causal))
    traffic = None if rec is None else rec.get("bytes_per_launch")
    line = {
        "metric": "attention fwd TFLOPS + ms at B=8,H=32,d=64,N=512..8192; % of MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "per_call": per_call,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": f"synthetic: i.i.d. N(0,1) inputs from seed 0, stored as {dtype}",
        "config": {"workload": f"attention forward B={B} H={H} N={N} d={d} {dtype} "
                               f"{'causal' if causal else 'non-causal'} scale=1/sqrt({d})",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "tile": _lib.fwd_tile(N, d, causal, {"f16": 0, "bf16": 1, "fp8": 2}[dtype])},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "algorithmic_hbm_gbs": round(algo_bytes / (ms * 1e-3) / 1e9, 1),
                     "secondary_ceilings": secondary_ceilings(d, dtype, causal, fl, _lib.fwd_tile(
                         N, d, causal, {"f16": 0, "bf16": 1, "fp8": 2}[dtype]), rec)},
        "configs": configs,
        "sweep": sweep,
        "timing": "HIP events on the kernel's stream; value = K back-to-back calls / elapsed after "
                  f"{args.clock_ms:g} ms of clock conditioning (device matmuls, not the benchmarked call) and W "
                  "warm-up calls; per_call, configs and sweep = one event pair per call (median, min, p90), each "
                  "after a 50 ms warm-up; no cache flush between calls",
        "gpu_clocks_under_load": clocks,
    }
    if not args.no_cpu:
        progress("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(keep[0], causal, scale, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


def main_bwd(args):
    """The backward pass on one dense shape: FLOPs counted as the five products
    of the method (10*B*H*N^2*d, halved for causal)."""
    import torch

    from io_aware_attention_fwd_amd import _lib, gen

    f = args.bwd.split(",")
    B, H, N, d, dtype, causal = int(f[0]), int(f[1]), int(f[2]), int(f[3]), f[4], f[5] in ("1", "true")
    scale = 1.0 / math.sqrt(d)
    progress(f"backward inputs B={B} H={H} N={N} d={d} {dtype} causal={int(causal)}")
    call_f, stream, keep = make_call(B, H, N, d, dtype, causal, scale)
    _, q, k, v, o, lse = keep
    call_f()
    do = make_call(B, H, N, d, dtype, causal, scale, seed=100)[2][1]  # dO: a seeded N(0,1) draw of the same shape
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dt = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16}[dtype]
    lib = _lib.load()
    a = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
         dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, scale, int(causal), dt, stream.cuda_stream)

    def call():
        rc = lib.fa_bwd(*a)
        if rc:
            raise _lib.FaError(rc, "fa_bwd")
    ms = time_calls(call, args.warmup, args.steps, stream)
    fl = 2.5 * flops(B, H, N, d, causal)
    peak = PEAK_TFLOPS[dtype]
    per_call = summarize(time_each(call, 2, min(args.steps, 50), stream), fl, peak)
    tflops = fl / (ms * 1e-3) / 1e12
    line = {
        "metric": "attention fwd TFLOPS + ms at B=8,H=32,d=64,N=512..8192; % of MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "per_call": per_call, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype,
        "data": f"synthetic: i.i.d. N(0,1) Q, K, V (seed 0) and dO (seed 100), stored as {dtype}",
        "config": {"workload": f"attention backward (dQ, dK, dV) B={B} H={H} N={N} d={d} {dtype} "
                               f"{'causal' if causal else 'non-causal'} scale=1/sqrt({d})",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "flop_count": "10*B*H*N^2*d (five products), halved for causal"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None},
        "timing": "HIP events on the kernels' stream; value = K back-to-back calls / elapsed",
    }
    print(json.dumps(line), flush=True)
    del torch
    return 0


def main_varlen(args):
    """The packed variable-length entry point on a seeded length mix."""
    import torch

    from io_aware_attention_fwd_amd import gen

    f = args.varlen.split(",")
    count, lo, hi, H, d, dtype, causal = int(f[0]), int(f[1]), int(f[2]), int(f[3]), int(f[4]), f[5], f[6] in ("1", "true")
    lengths = gen.length_mix(count, lo, hi, seed=0)
    scale = 1.0 / math.sqrt(d)
    progress(f"packed inputs: {count} sequences in [{lo}, {hi}], H={H} d={d} {dtype} causal={int(causal)}")
    call, stream, keep = make_call_varlen(lengths, H, d, dtype, causal, scale)
    ms = time_calls(call, args.warmup, args.steps, stream)
    fl = sum(flops(1, H, n, d, causal) for n in lengths)
    peak = PEAK_TFLOPS[dtype]
    per_call = summarize(time_each(call, 2, min(args.steps, 50), stream), fl, peak)
    tflops = fl / (ms * 1e-3) / 1e12
    total = sum(lengths)
    algo_bytes = (3 * (1 if dtype == "fp8" else 2) + 2) * total * H * d + 4 * total * H
    line = {
        "metric": "attention fwd TFLOPS + ms at B=8,H=32,d=64,N=512..8192; % of MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "per_call": per_call, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype,
        "data": f"synthetic: i.i.d. N(0,1) inputs from seed 0, stored as {dtype}; lengths from seed 0",
        "config": {"workload": f"packed variable-length attention forward: {count} sequences, lengths uniform in "
                               f"[{lo}, {hi}] (total {total} rows), H={H} d={d} {dtype} "
                               f"{'causal' if causal else 'non-causal'} scale=1/sqrt({d})",
                   "lengths": lengths, "H": H, "d": d, "causal": causal},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "algorithmic_hbm_gbs": round(algo_bytes / (ms * 1e-3) / 1e9, 1)},
        "timing": "HIP events on the kernel's stream; value = K back-to-back calls / elapsed",
    }
    if not args.no_cpu:
        progress("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline_varlen(keep[0], keep[1], causal, scale, args.cpu_budget)
    print(json.dumps(line), flush=True)
    del torch
    return 0


def main_dropout(args):
    """The forward pass with dropout on one dense shape (FLOPs as the forward's)."""
    import torch

    from io_aware_attention_fwd_amd import _lib

    f = args.dropout.split(",")
    B, H, N, d, dtype, causal, p = (int(f[0]), int(f[1]), int(f[2]), int(f[3]), f[4], f[5] in ("1", "true"),
                                    float(f[6]))
    scale = 1.0 / math.sqrt(d)
    progress(f"dropout inputs B={B} H={H} N={N} d={d} {dtype} causal={int(causal)} p={p}")
    _, stream, keep = make_call(B, H, N, d, dtype, causal, scale)
    _, q, k, v, o, lse = keep
    dt = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16}[dtype]
    lib = _lib.load()
    a = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, scale, int(causal), dt,
         p, 1234, 0, stream.cuda_stream)

    def call():
        rc = lib.fa_fwd_dropout(*a)
        if rc:
            raise _lib.FaError(rc, "fa_fwd_dropout")
    ms = time_calls(call, args.warmup, args.steps, stream)
    fl = flops(B, H, N, d, causal)
    peak = PEAK_TFLOPS[dtype]
    per_call = summarize(time_each(call, 2, min(args.steps, 50), stream), fl, peak)
    tflops = fl / (ms * 1e-3) / 1e12
    line = {
        "metric": "attention fwd TFLOPS + ms at B=8,H=32,d=64,N=512..8192; % of MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "per_call": per_call, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype,
        "data": f"synthetic: i.i.d. N(0,1) inputs from seed 0, stored as {dtype}; dropout seed 1234, offset 0",
        "config": {"workload": f"attention forward with dropout p={p} B={B} H={H} N={N} d={d} {dtype} "
                               f"{'causal' if causal else 'non-causal'} scale=1/sqrt({d})",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "p_drop": p},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None},
        "timing": "HIP events on the kernel's stream; value = K back-to-back calls / elapsed",
    }
    print(json.dumps(line), flush=True)
    del torch
    return 0


def main_proj(args):
    """The fused QKV projection: FLOPs 2*M*(3Hd)*D, M = B*N tokens."""
    import torch

    from io_aware_attention_fwd_amd import _lib, gen

    f = args.proj.split(",")
    B, N, D, H, d, dtype = int(f[0]), int(f[1]), int(f[2]), int(f[3]), int(f[4]), f[5]
    progress(f"projection inputs B={B} N={N} D={D} H={H} d={d} {dtype}")
    pi = gen.make_projection(B, N, D, H, d, dtype, seed=0)

    def dev(a):
        if dtype == "f16":
            return torch.from_numpy(a).cuda()
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    x, w, bias = dev(pi.x), dev(pi.w), dev(pi.bias)
    q, k, v = (torch.empty((B, H, N, d), dtype=x.dtype, device="cuda") for _ in range(3))
    stream = torch.cuda.current_stream()
    lib = _lib.load()
    dt = {"f16": _lib.FA_DTYPE_F16, "bf16": _lib.FA_DTYPE_BF16}[dtype]
    a = (x.data_ptr(), w.data_ptr(), bias.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), B, N, D, H, d, dt,
         stream.cuda_stream)

    def call():
        rc = lib.fa_qkv_proj(*a)
        if rc:
            raise _lib.FaError(rc, "fa_qkv_proj")
    ms = time_calls(call, args.warmup, args.steps, stream)
    M, ncol = B * N, 3 * H * d
    fl = 2.0 * M * ncol * D
    peak = PEAK_TFLOPS[dtype]
    per_call = summarize(time_each(call, 2, min(args.steps, 50), stream), fl, peak)
    tflops = fl / (ms * 1e-3) / 1e12
    algo_bytes = 2 * (M * D + ncol * D + ncol + M * ncol)
    line = {
        "metric": "attention fwd TFLOPS + ms at B=8,H=32,d=64,N=512..8192; % of MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "per_call": per_call, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype,
        "data": f"synthetic: x ~ N(0,1), weight ~ N(0,1/D), bias ~ N(0,0.01) from seed 0, stored as {dtype}",
        "config": {"workload": f"fused QKV projection B={B} N={N} D={D} -> Q, K, V [B, H={H}, N, d={d}] {dtype}",
                   "B": B, "N": N, "D": D, "H": H, "d": d},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None, "algorithmic_bytes_per_launch": algo_bytes,
                     "algorithmic_hbm_gbs": round(algo_bytes / (ms * 1e-3) / 1e9, 1)},
        "timing": "HIP events on the kernel's stream; value = K back-to-back calls / elapsed",
    }
    print(json.dumps(line), flush=True)
    del torch
    return 0


if __name__ == "__main__":
    sys.exit(main())

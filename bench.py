"""Benchmark of the per-group fp8 scale + cast hot path on one MI355X.

A step is one pass of the hot path over the (16640, 8192) bf16 token-major
gradient with 64 token groups: the colwise per-group cast of T (groups along
dim0, the operand quantised per (group, column)) followed by the rowwise
per-group cast of T transposed, (8192, 16640) with groups along dim1. These
are the two halves of the shape the rowwise page benchmarks ("[moe fp8
training] test and bench new faster method for per group rowwise scaling",
Benchmarks table, (16640, 8192) with 64 groups).

The single JSON line on stdout: `value` is the algorithmic HBM throughput of
the whole step (read bf16 once, write E4M3 once, write fp32 scales, read
offsets) over the timed steps, with every input already resident in HBM and
the GPU brought to steady clocks by 50 ms of untimed steps first.
`roofline` reports the slower of the two kernels against MI355X's 8 TB/s,
timed with HIP events on the stream the library launches on.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.
Per-config kernel times (each run after a cache flush) go into `kernels`.
Human-readable detail goes to stderr.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("mgs_device.hpp", "mgs_kernels.hpp", "mgs_dim0_layout.hpp", "mgs_dim0.hip", "mgs_dim1.hip",
                  "mgs_mx.hip", "mgs_api.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text):
    """Source text without // comments, trailing blanks and blank lines, so
    that comment edits leave the hash alone (the sources use no string
    literal that holds //)."""
    out = []
    for line in text.splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line:
            out.append(line)
    return "\n".join(out) + "\n"


def kernel_source_hash():
    """Hash of the kernel sources' code, comments left out."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "group_scaling_fp8_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode("utf-8"))
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence: it records a
    timestamp on the stream without the system-scope cache writeback and
    invalidate of a default event, which would otherwise add several
    microseconds between the kernels it separates. Elapsed times are read
    only after a device synchronisation."""
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            # the HIP runtime torch has loaded (one copy per process, by soname)
            HipEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self._c = ctypes
        self.ev = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self, stream):
        rc = HipEvent._hip.hipEventRecord(self.ev, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_ms(self, end):
        ms = self._c.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-config table")
    ap.add_argument("--counter-run", type=int, default=0, metavar="REPS",
                    help="only launch each case of counter_cases() (a 256 MiB calibration copy, "
                         "then the library's kernels) REPS times, for rocprofv3 counter collection; "
                         "with --rocprof-summary, the REPS those runs used")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="print a markdown summary of rocprofv3 output under DIR (trace/, fetch/, "
                         "write/ from the commands in profiles/README.md) and write "
                         "profiles/hbm_traffic.json; needs no GPU")
    ap.add_argument("--cpu-cols", type=int, default=8192,
                    help="columns of T (and rows of T^T) in the oracle's timed sample")
    args = ap.parse_args()

    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary, args.counter_run or 3)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the per-group cast needs no cross-GPU exchange, and "
              "this benchmark runs on one GPU only (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import group_scaling_fp8_amd as mgs
    from group_scaling_fp8_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mgs.lib()
    if args.counter_run:
        counter_run(torch, mgs, wl, dev, args.counter_run)
        return

    log("generating the (16640, 8192) bf16 workload ...")
    T = wl.token_major_gradient()
    off = wl.target_offsets(64)
    Tt = np.ascontiguousarray(T.T)
    M, K = T.shape
    G = len(off)
    x0 = torch.from_numpy(T.view(np.int16)).to(dev)
    x1 = torch.from_numpy(Tt.view(np.int16)).to(dev)
    o = torch.from_numpy(off).to(dev)
    q0 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    s0 = torch.empty((G, K), dtype=torch.float32, device=dev)
    q1 = torch.empty((K, M), dtype=torch.uint8, device=dev)
    s1 = torch.empty((K, G), dtype=torch.float32, device=dev)
    bytes_dim0 = wl.Workload("", "dim0", T, off).algorithmic_bytes()
    bytes_dim1 = wl.Workload("", "dim1", Tt, off).algorithmic_bytes()
    step_bytes = bytes_dim0 + bytes_dim1

    stream = torch.cuda.current_stream()

    def step():
        mgs.mgs_quant_groups_dim0(x0, o, False, q=q0, scales=s0)
        mgs.mgs_quant_groups_dim1(x1, o, False, q=q1, scales=s1)

    # Pre-warm: untimed steps for at least PREWARM_MS of wall clock. From
    # idle, the GPU's clocks take about 15 ms of this load to settle (the step
    # runs at 150-154 us in its first 10 ms and 145 us from then on), longer
    # than a few warmup steps last; the timed steps below then measure the
    # steady state of the same work.
    torch.cuda.synchronize()
    t_pre = time.perf_counter()
    prewarm_steps = 0
    while (time.perf_counter() - t_pre) * 1e3 < PREWARM_MS:
        for _ in range(10):
            step()
        prewarm_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Pass 1 (the contract's timed region): K steps, no event markers between
    # kernels, bracketed by device synchronisation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # Pass 2: per-kernel durations with HIP events on the stream the library
    # launches on. Each kernel runs K times back to back, with events only at
    # the two ends of the block (an event between kernels adds a marker that
    # costs several microseconds), alternating between the input and a copy
    # of it so that no launch reads what the previous one left in the
    # 256 MiB Infinity Cache.
    x0b, x1b = x0.clone(), x1.clone()

    def block_ms(fn, xa, xb):
        a, b = HipEvent(), HipEvent()
        # a few untimed launches first, so that the clones' dirty lines are
        # written back before the timed block starts
        for i in range(3):
            fn(xa if i % 2 == 0 else xb)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            fn(xa if i % 2 == 0 else xb)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_ms(b) / args.steps

    avg0 = block_ms(lambda x: mgs.mgs_quant_groups_dim0(x, o, False, q=q0, scales=s0), x0, x0b)
    avg1 = block_ms(lambda x: mgs.mgs_quant_groups_dim1(x, o, False, q=q1, scales=s1), x1, x1b)
    del x0b, x1b
    log("step: %.1f us; kernels alone: dim0 %.1f us, dim1 %.1f us; %.0f GB/s"
        % (ms_per_step * 1e3, avg0 * 1e3, avg1 * 1e3, value))

    # each entry point launches one kernel here (dim0_kernel, dim1_kernel)
    dominant = "dim0_kernel" if avg0 >= avg1 else "dim1_kernel"
    dom_ms, dom_bytes = (avg0, bytes_dim0) if avg0 >= avg1 else (avg1, bytes_dim1)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dominant), "kernel": dominant,
                "kernel_us": round(dom_ms * 1e3, 2), "algorithmic_bytes": dom_bytes}

    # parity spot check of this run's outputs on one strip / a few rows
    import oracle
    cols = np.arange(0, 128)
    rq, rs = oracle.quant_groups_dim0(np.ascontiguousarray(T[:, cols]), off)
    ok0 = (np.array_equal(q0[:, :128].cpu().numpy(), rq)
           and np.array_equal(s0[:, :128].cpu().numpy().view(np.uint32), rs.view(np.uint32)))
    rows = np.array([0, 4097, K - 1])
    rq1, rs1 = oracle.quant_groups_dim1(np.ascontiguousarray(Tt[rows]), off)
    ok1 = (np.array_equal(q1[rows].cpu().numpy(), rq1)
           and np.array_equal(s1[rows].cpu().numpy().view(np.uint32), rs1.view(np.uint32)))

    kernels = None
    samples = {}
    inputs = {"numpy": np.__version__,
              "generator": "numpy default_rng (PCG64), seeds in group_scaling_fp8_amd/workloads.py",
              "sha256": {"T (16640,8192) bf16, seed 4": hashlib.sha256(T.tobytes()).hexdigest(),
                         "offsets G=64, seed 104": hashlib.sha256(off.tobytes()).hexdigest()}}
    if not args.no_kernels:
        kernels = per_config_table(torch, mgs, wl, dev, T, Tt, inputs["sha256"], samples)
        kernels += host_call_cost(torch, mgs, wl, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(T, Tt, off, args.cpu_cols, samples)

    out = {
        "metric": "achieved HBM GB/s (% of peak) per-group fp8 scale+cast, (16640,8192) bf16 G=64",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "per-group fp8 scale+cast of a (16640, 8192) bf16 token-major "
                               "gradient, G=64: dim0 on T then dim1 on T^T (8192, 16640)",
                   "M": M, "K": K, "groups": G, "in": "bf16", "out": "e4m3 + fp32 scales",
                   "step_bytes": step_bytes, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
                   "parity_spot_check": bool(ok0 and ok1),
                   "prewarm": "%d untimed steps (%.0f ms) before the warmup steps" % (prewarm_steps, PREWARM_MS),
                   "device": torch.cuda.get_device_name(0)
                   or torch.cuda.get_device_properties(0).gcnArchName},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "inputs": inputs,
    }
    print(json.dumps(out), flush=True)


# kernel-name fragments of the library's kernels, and what each one is
# matched as substrings of the demangled names, first match wins: the more
# specific names come first
KERNELS = (("copy_kernel", "copy"), ("mx_dim1_kernel", "mx_dim1_kernel"),
           ("mx_dequant_kernel", "mx_dequant_kernel"), ("mx_kernel", "mx_kernel"),
           ("zero_kernel", "zero_kernel"), ("dim0t_kernel", "dim0t_kernel"),
           ("dim0_kernel", "dim0_kernel"), ("dim1_kernel", "dim1_kernel"))
PREWARM_MS = 50.0          # untimed steps before the warmup steps (clock settling)
COPY_BYTES = 1 << 28      # the counter run's calibration copy: 256 MiB read + 256 MiB written


def _short(name):
    for frag, short in KERNELS:
        if frag in name:
            return short
    return None


def _stats_table(path):
    import csv
    out = ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    if os.path.exists(path):
        for r in csv.DictReader(open(path)):
            k = _short(r["Name"])
            if k:
                out.append("| %s | %s | %.2f | %.2f | %.2f |" % (
                    k, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3))
    return out


def experts_weight(torch, dev):
    """The (16, 5120, 8192) bf16 expert weight, randn * 0.02, drawn on the
    GPU from torch's generator with seed 7."""
    gen = torch.Generator(device=dev).manual_seed(7)
    return (torch.randn((16, 5120, 8192), generator=gen, device=dev) * 0.02).to(torch.bfloat16)


def counter_cases():
    """The counter run's launches in order: (label, kernel, algorithmic bytes
    per launch). Bytes: bf16 read once, E4M3 written once, fp32 scales
    written and int32 offsets read (grouped casts); E8M0 scales (MX);
    for the dequantisation the E4M3 codes and scales read and bf16 written."""
    def dim0(M, K, G):
        return 3 * M * K + 4 * G * K + 4 * G

    def dim1(M, K, G):
        return 3 * M * K + 4 * M * G + 4 * G

    mx = 3 * 131072 * 5120 + 131072 * 5120 // 32
    return [("copy 256 MiB (calibration)", "copy", 2 * COPY_BYTES),
            ("dim0 (16640,8192) G=64", "dim0_kernel", dim0(16640, 8192, 64)),
            ("dim0 (16640,8192) G=1", "dim0_kernel", dim0(16640, 8192, 1)),
            ("dim0 (16640,8192) G=8 even", "dim0_kernel", dim0(16640, 8192, 8)),
            ("dim0 (256,4096) G=4", "dim0_kernel", dim0(256, 4096, 4)),
            ("dim0 (4096,4096) G=16 pow2", "dim0_kernel", dim0(4096, 4096, 16)),
            ("dim0 (65536,4096) G=8 dirichlet", "dim0_kernel", dim0(65536, 4096, 8)),
            ("dim1 (8192,16640) G=64", "dim1_kernel", dim1(8192, 16640, 64)),
            ("dim1 (8192,16640) G=16", "dim1_kernel", dim1(8192, 16640, 16)),
            ("dim1 (8192,16640) G=1", "dim1_kernel", dim1(8192, 16640, 1)),
            ("mx dim0 (131072,5120) FLOOR", "mx_kernel", mx),
            ("mx dim0 (131072,5120) RCEIL", "mx_kernel", mx),
            ("dim0_t (16640,8192) G=64 -> (8192,16640)", "dim0t_kernel", dim0(16640, 8192, 64)),
            ("experts (16,5120,8192) along dim1", "dim0_kernel", 3 * 16 * 5120 * 8192 + 4 * 16 * 8192),
            ("mx dim1 (131072,5120) FLOOR -> (5120,131072)", "mx_dim1_kernel", mx),
            ("mx dequant (131072,5120) -> bf16", "mx_dequant_kernel", mx)]


def _dispatches(path, name_col, reps, extra):
    """Rows of a rocprofv3 CSV for the counter run's measured launches, in
    dispatch order, grouped per case: the last len(cases) * reps rows whose
    kernel is one of the library's."""
    import csv
    rows = [r for r in csv.DictReader(open(path)) if _short(r[name_col])]
    for key in ("Dispatch_Id", "Start_Timestamp"):
        if rows and key in rows[0]:
            rows.sort(key=lambda r: int(r[key]))
            break
    cases = counter_cases()
    rows = rows[-len(cases) * reps:]
    if len(rows) != len(cases) * reps:
        raise SystemExit("%s: %d dispatches, expected %d" % (path, len(rows), len(cases) * reps))
    out = []
    for i, (label, kernel, _) in enumerate(cases):
        mine = rows[i * reps:(i + 1) * reps]
        for r in mine:
            if _short(r[name_col]) != kernel:
                raise SystemExit("%s: case %r ran %s" % (path, label, r[name_col][:60]))
        out.append([extra(r) for r in mine])
    return out


def rocprof_summary(d, reps):
    """Markdown summary of a counter run (kernel trace, FETCH_SIZE and
    WRITE_SIZE passes under d/trace, d/fetch, d/write), one row per case;
    also writes profiles/hbm_traffic.json."""
    bench_stats = os.path.join(d, "bench", "run_kernel_stats.csv")
    if os.path.exists(bench_stats):
        print("\n".join(["## benchmark command (steps after warmup, with and without events)", ""]
                        + _stats_table(bench_stats) + [""]))
    cases = counter_cases()
    dur = _dispatches(os.path.join(d, "trace", "run_kernel_trace.csv"), "Kernel_Name", reps,
                      lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    kib = {}
    for counter in ("fetch", "write"):
        kib[counter] = _dispatches(os.path.join(d, counter, "run_counter_collection.csv"),
                                   "Kernel_Name", reps, lambda r: float(r["Counter_Value"]))
    mean = lambda v: sum(v) / len(v)
    ff = COPY_BYTES / 1024.0 / mean(kib["fetch"][0])
    wf = COPY_BYTES / 1024.0 / mean(kib["write"][0])
    out = ["## counter run (one launch at a time after a 1 GiB read sweep; %d launches per case)" % reps,
           "", "FETCH_SIZE scale %.4f, WRITE_SIZE scale %.4f (the copy kernel reads and writes %d B)"
           % (ff, wf, COPY_BYTES), "",
           "| case | kernel | avg us | algorithmic MB | HBM read MB | HBM written MB | HBM / algorithmic "
           "| algorithmic GB/s |", "|---|---|---|---|---|---|---|---|"]
    traffic = {"source_hash": kernel_source_hash(), "fetch_scale": ff, "write_scale": wf,
               "cases": {}, "kernels": {}}
    for i, (label, kernel, alg) in enumerate(cases):
        us = mean(dur[i])
        rd = mean(kib["fetch"][i]) * 1024 * ff
        wr = mean(kib["write"][i]) * 1024 * wf
        traffic["cases"][label] = {"kernel": kernel, "avg_us": round(us, 2), "algorithmic_bytes": alg,
                                   "fetch_kib": mean(kib["fetch"][i]), "write_kib": mean(kib["write"][i]),
                                   "bytes_per_launch": round(rd + wr)}
        # the first case of each kernel is the one its roofline is quoted on
        traffic["kernels"].setdefault(kernel, traffic["cases"][label])
        out.append("| %s | %s | %.2f | %.1f | %.1f | %.1f | %.3f | %.0f |" % (
            label, kernel, us, alg / 1e6, rd / 1e6, wr / 1e6, (rd + wr) / alg, alg / us / 1e3))
    with open(os.path.join(PROFILES, "hbm_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print("\n".join(out))


def counter_run(torch, mgs, wl, dev, reps):
    """Launches each case of counter_cases() `reps` times, in that order,
    with nothing else on the GPU but a cache-evicting read before each
    launch, so a counter collector sees one dispatch per launch. Every
    output buffer and workspace is made first, by calls outside the
    measured loops."""
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    T = wl.token_major_gradient()
    g64 = torch.from_numpy(wl.target_offsets(64)).to(dev)
    g16 = torch.from_numpy(wl.target_offsets(16)).to(dev)
    g1 = torch.from_numpy(np.array([T.shape[0]], np.int32)).to(dev)
    x0 = torch.from_numpy(T.view(np.int16)).to(dev)
    x1 = torch.from_numpy(np.ascontiguousarray(T.T).view(np.int16)).to(dev)
    del T
    small = []
    for w in (wl.c1_dim0_small(), wl.c2_dim0_pow2(), wl.c3_dim0_large()):
        small.append((torch.from_numpy(w.x.view(np.int16)).to(dev), torch.from_numpy(w.offsets).to(dev),
                      w.pow2))
    c5 = wl.c5_mx()
    x5 = torch.from_numpy(c5.x.view(np.int16)).to(dev)
    del c5

    def grouped(f, x, o, pow2=False):
        q, s = f(x, o, pow2)
        return lambda: f(x, o, pow2, q=q, scales=s)

    dim0, dim1 = mgs.mgs_quant_groups_dim0, mgs.mgs_quant_groups_dim1
    g8 = torch.from_numpy(np.arange(1, 9, dtype=np.int32) * (x0.shape[0] // 8)).to(dev)
    w3 = experts_weight(torch, dev)
    q3, s3 = mgs.mgs_quant_experts_dim1(w3)
    q5, s5 = mgs.mgs_mx_quant_dim0(x5, mgs.MGS_MX_FLOOR)
    qt, st = mgs.mgs_quant_groups_dim0_t(x0, g64)
    qd1, sd1 = mgs.mgs_mx_quant_dim1(x5, mgs.MGS_MX_FLOOR)
    yd = mgs.mgs_mx_dequant_dim0(q5, s5)
    runs = [lambda: mgs.mgs_copy(src, dst),
            grouped(dim0, x0, g64), grouped(dim0, x0, g1), grouped(dim0, x0, g8)] + \
        [grouped(dim0, x, o, p) for x, o, p in small] + \
        [grouped(dim1, x1, g64), grouped(dim1, x1, g16), grouped(dim1, x1, g1),
         lambda: mgs.mgs_mx_quant_dim0(x5, mgs.MGS_MX_FLOOR, q=q5, scales=s5),
         lambda: mgs.mgs_mx_quant_dim0(x5, mgs.MGS_MX_RCEIL, q=q5, scales=s5),
         lambda: mgs.mgs_quant_groups_dim0_t(x0, g64, q_t=qt, scales_t=st),
         lambda: mgs.mgs_quant_experts_dim1(w3, q=q3, scales=s3),
         lambda: mgs.mgs_mx_quant_dim1(x5, mgs.MGS_MX_FLOOR, q_t=qd1, scales_t=sd1),
         lambda: mgs.mgs_mx_dequant_dim0(q5, s5, y=yd)]
    assert len(runs) == len(counter_cases())
    torch.cuda.synchronize()
    for (label, _, _), fn in zip(counter_cases(), runs):
        for _ in range(reps):
            flush.max()
            fn()
            torch.cuda.synchronize()
        log("counter run: %s x%d" % (label, reps))
    log("counter run done: %d launches of each case" % reps)


def timed_us(torch, fn, flush, reps=20):
    """Median and min of `reps` single launches, each after reading a 1 GiB
    buffer (more than L2 plus the 256 MiB Infinity Cache)."""
    st = torch.cuda.current_stream()
    ts = []
    a, b = HipEvent(), HipEvent()
    for _ in range(reps):
        flush.max()          # read-only sweep: evicts caches without leaving dirty lines
        a.record(st)
        fn()
        b.record(st)
        torch.cuda.synchronize()
        ts.append(a.elapsed_ms(b) * 1e3)
    return float(np.median(ts)), float(np.min(ts))


def steady_us(torch, fn, reps=20, lead=3):
    """Average of `reps` back-to-back launches with no flush between them:
    each launch also pays for writing back what the one before left dirty.
    `lead` launches are queued before the first event, so the timed block
    starts on a busy stream: it measures the GPU's time per launch, not the
    submission latency of the first one (the host's cost per call is
    measured on its own in host_call_cost)."""
    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    a, b = HipEvent(), HipEvent()
    for _ in range(lead):
        fn()
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_ms(b) * 1e3 / reps


def counter_traffic():
    """Counter-run cases of profiles/hbm_traffic.json (label -> entry) when
    they were taken on the current kernel sources, else {}."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    return t.get("cases", {}) if t.get("source_hash") == kernel_source_hash() else {}


# elements of each config's input that the oracle is timed on (about a third
# of a second of one core); the rest of the config scales with it
ORACLE_SAMPLE_ELEMS = 1 << 24


def per_config_table(torch, mgs, wl, dev, T, Tt, sha, samples):
    """Per-config kernel times; records each generated input's sha256 in
    `sha` (config name -> digest of x's bytes, then the offsets'), and in
    `samples` a slice of each grouped and MX config's input for the CPU
    oracle's timing (config name -> (kind, slice, offsets or mode, pow2,
    fraction of the config, algorithmic bytes of the config))."""
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)     # 1 GiB
    rows = []
    traffic = counter_traffic()

    def add(name, kind, x, off, bytes_, fn_maker, elems=None):
        fn = fn_maker()
        fn()
        torch.cuda.synchronize()
        med, mn = timed_us(torch, fn, flush)
        sty = steady_us(torch, fn)
        rows.append({"config": name, "kind": kind, "us_median": round(med, 2), "us_min": round(mn, 2),
                     "algorithmic_GBps": round(bytes_ / (med * 1e-6) / 1e9, 1),
                     "pct_hbm_peak": round(100 * bytes_ / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                     "us_steady": round(sty, 2),
                     "steady_GBps": round(bytes_ / (sty * 1e-6) / 1e9, 1)})
        if elems is not None:
            # the rowwise page's bytes convention: bf16 input counted twice
            # (2R + 1W + scales), for a like-for-like look at its table
            rows[-1]["page_convention_GBps"] = round((bytes_ + 2 * elems) / (med * 1e-6) / 1e9, 1)
        if name in traffic:
            # HBM bytes of this case from the rocprofv3 counter run, over this
            # run's cold median
            hb = traffic[name]["bytes_per_launch"]
            rows[-1]["hbm_bytes_measured"] = hb
            rows[-1]["measured_GBps"] = round(hb / (med * 1e-6) / 1e9, 1)
        log("  %-44s %9.2f us  %7.1f GB/s   back-to-back %9.2f us  %7.1f GB/s"
            % (name, med, rows[-1]["algorithmic_GBps"], sty, rows[-1]["steady_GBps"]))

    def keep_sample(w):
        M, K = w.x.shape
        if w.kind == "dim0":      # every row of the first columns
            n = min(K, max(8, ORACLE_SAMPLE_ELEMS // M // 8 * 8))
            part = np.ascontiguousarray(w.x[:, :n])
            frac = n / K
        else:                     # the first rows
            n = min(M, max(1, ORACLE_SAMPLE_ELEMS // K))
            part = np.ascontiguousarray(w.x[:n])
            frac = n / M
        samples[w.name] = (w.kind, part, w.offsets, w.pow2, frac, w.algorithmic_bytes())

    def grouped(w):
        sha[w.name] = w.sha256()
        keep_sample(w)
        x = torch.from_numpy(w.x.view(np.int16)).to(dev)
        o = torch.from_numpy(w.offsets).to(dev)
        f = mgs.mgs_quant_groups_dim0 if w.kind == "dim0" else mgs.mgs_quant_groups_dim1
        q, s = f(x, o, w.pow2)
        return lambda: (lambda: f(x, o, w.pow2, q=q, scales=s))

    log("per-config kernel times (cache flushed before each launch; then back-to-back launches):")
    M = T.shape[0]
    tall = [
        # every row in one group: 19 chunks of up to 896 rows (column maxima through the workspace)
        wl.Workload("dim0 (16640,8192) G=1", "dim0", T, np.array([M], dtype=np.int32)),
        # eight groups of 2080 rows: teams of three 694-row chunks
        wl.Workload("dim0 (16640,8192) G=8 even", "dim0", T,
                    np.arange(1, 9, dtype=np.int32) * (M // 8)),
    ]
    for w in [wl.c1_dim0_small(), wl.c2_dim0_pow2(), wl.c3_dim0_large(),
              wl.c6_dim0_target(64, T)] + tall + [wl.c4_dim1(1, T), wl.c4_dim1(16, T),
                                                  wl.c4_dim1(64, T)]:
        add(w.name, w.kind, w.x, w.offsets, w.algorithmic_bytes(), grouped(w), elems=w.x.size)
        del w
    # the fused quantize + transpose of T: (8192, 16640) e4m3 and (8192, 64)
    # scales, the same bytes as dim0 at this shape
    w = wl.c6_dim0_target(64, T)
    xt6 = torch.from_numpy(T.view(np.int16)).to(dev)
    ot6 = torch.from_numpy(w.offsets).to(dev)
    qt6, st6 = mgs.mgs_quant_groups_dim0_t(xt6, ot6)
    add("dim0_t (16640,8192) G=64 -> (8192,16640)", "dim0_t", T, w.offsets, w.algorithmic_bytes(),
        lambda: (lambda: mgs.mgs_quant_groups_dim0_t(xt6, ot6, q_t=qt6, scales_t=st6)))
    del w, xt6, ot6, qt6, st6
    # per-expert scaling of a 3D weight along dim 1: 16 experts of (5120, 8192),
    # each expert a 5120-row group cut into 6-chunk teams (seeded on the GPU)
    E, D1, D2 = 16, 5120, 8192
    w3 = experts_weight(torch, dev)
    sha["experts (16,5120,8192) bf16, torch seed 7"] = hashlib.sha256(
        w3.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
    q3, s3 = mgs.mgs_quant_experts_dim1(w3)
    add("experts (16,5120,8192) along dim1", "experts", None, None, 3 * E * D1 * D2 + 4 * E * D2,
        lambda: (lambda: mgs.mgs_quant_experts_dim1(w3, q=q3, scales=s3)))
    del w3, q3, s3
    c5 = wl.c5_mx()
    sha[c5.name + ", seed 5"] = c5.sha256()
    x5 = torch.from_numpy(c5.x.view(np.int16)).to(dev)
    n_mx = ORACLE_SAMPLE_ELEMS // c5.x.shape[1]
    for mode, nm in ((mgs.MGS_MX_FLOOR, "FLOOR"), (mgs.MGS_MX_RCEIL, "RCEIL")):
        samples[c5.name + " " + nm] = ("mx", np.ascontiguousarray(c5.x[:n_mx]), mode, False,
                                        n_mx / c5.x.shape[0], c5.algorithmic_bytes())
        q, s = mgs.mgs_mx_quant_dim0(x5, mode)
        add(c5.name + " " + nm, "mx", c5.x, None, c5.algorithmic_bytes(),
            lambda: (lambda: mgs.mgs_mx_quant_dim0(x5, mode, q=q, scales=s)))
    # blocks of 32 along dim0, GEMM-ready transposed outputs (K, M) and (K, M/32)
    qd1, sd1 = mgs.mgs_mx_quant_dim1(x5, mgs.MGS_MX_FLOOR)
    add("mx dim1 (131072,5120) FLOOR -> (5120,131072)", "mx_dim1", c5.x, None, c5.algorithmic_bytes(),
        lambda: (lambda: mgs.mgs_mx_quant_dim1(x5, mgs.MGS_MX_FLOOR, q_t=qd1, scales_t=sd1)))
    del qd1, sd1
    # the receiving side: E4M3 + E8M0 back to bf16 (1 + 1/32 B read, 2 B written
    # per element), then the whole pipeline of the mxfp8 all-to-all with a
    # device copy of q and scales standing in for the all-to-all
    n5 = c5.x.size
    q, s = mgs.mgs_mx_quant_dim0(x5, mgs.MGS_MX_RCEIL)
    y5 = mgs.mgs_mx_dequant_dim0(q, s)
    add("mx dequant (131072,5120) -> bf16", "mx_dequant", None, None, 3 * n5 + n5 // 32,
        lambda: (lambda: mgs.mgs_mx_dequant_dim0(q, s, y=y5)))
    q2, s2 = torch.empty_like(q), torch.empty_like(s)

    def pipeline():
        mgs.mgs_mx_quant_dim0(x5, mgs.MGS_MX_RCEIL, q=q, scales=s)
        mgs.mgs_copy(q, q2)
        mgs.mgs_copy(s, s2)
        mgs.mgs_mx_dequant_dim0(q2, s2, y=y5)
    pipe_bytes = (3 * n5 + n5 // 32) + 2 * (n5 + n5 // 32) + (3 * n5 + n5 // 32)
    add("mx RCEIL quant -> copy -> dequant (131072,5120)", "mx_pipeline", None, None, pipe_bytes,
        lambda: pipeline)
    del q2, s2, y5
    # calibration: plain copy of the same byte count as the target's bf16 input
    src = torch.empty(T.size * 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    add("copy kernel, %d MiB read + write" % (src.numel() >> 20), "copy", None, None,
        2 * src.numel(), lambda: (lambda: mgs.mgs_copy(src, dst)))
    del x5, src, dst, flush
    torch.cuda.empty_cache()
    return rows


def host_call_cost(torch, mgs, wl, dev, n=2000):
    """Host time per call of the C ABI alone: a ctypes loop over
    mgs_quant_groups_dim0 (the library's own workspace) and
    mgs_quant_groups_dim1 on the (256, 4096) G=4 configuration, with device
    pointers and the stream handle prepared once (no torch in the loop), and
    the same launches through the Python binding. The kernels queue up
    behind the host; the device is synchronised only around each loop."""
    import ctypes
    w = wl.c1_dim0_small()
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    o = torch.from_numpy(w.offsets).to(dev)
    M, K = w.x.shape
    G = len(w.offsets)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    s0 = torch.empty((G, K), dtype=torch.float32, device=dev)
    s1 = torch.empty((M, G), dtype=torch.float32, device=dev)
    o1 = torch.from_numpy(wl.uniform_group_offsets(np.random.default_rng(9), K, G)).to(dev)
    L = mgs.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp, op, o1p, qp = x.data_ptr(), o.data_ptr(), o1.data_ptr(), q.data_ptr()
    s0p, s1p = s0.data_ptr(), s1.data_ptr()
    rows = []

    def timed(name, fn):
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        us = (t1 - t0) * 1e6 / n
        rows.append({"config": name, "kind": "host_call", "us_host_per_call": round(us, 2),
                     "us_per_call_with_drain": round((t2 - t0) * 1e6 / n, 2)})
        log("  %-52s %6.2f us host per call (%6.2f with the queue drained)"
            % (name, us, (t2 - t0) * 1e6 / n))

    log("host cost per call, (256, 4096) G=4:")
    f0, f1 = L.mgs_quant_groups_dim0, L.mgs_quant_groups_dim1
    timed("C ABI via ctypes: mgs_quant_groups_dim0",
          lambda: f0(xp, M, K, op, G, 0, qp, s0p, stream))
    timed("C ABI via ctypes: mgs_quant_groups_dim1",
          lambda: f1(xp, M, K, o1p, G, 0, qp, s1p, stream))
    timed("Python binding: mgs_quant_groups_dim0",
          lambda: mgs.mgs_quant_groups_dim0(x, o, q=q, scales=s0))
    return rows


def cpu_baseline(T, Tt, off, ncols, samples):
    """The CPU oracle, untuned and single-threaded, on a bounded sample of
    the step: dim0 on T[:, :ncols] (every row, every group) and dim1 on the
    first ncols rows of T^T. Throughput uses the same algorithmic bytes.
    Then, per config, the oracle on the slice kept in `samples`, with the
    whole config's time estimated from the slice's share of it."""
    import oracle
    from group_scaling_fp8_amd import workloads as wl
    xs0 = np.ascontiguousarray(T[:, :ncols])
    xs1 = np.ascontiguousarray(Tt[:ncols])
    b = (wl.Workload("", "dim0", xs0, off).algorithmic_bytes()
         + wl.Workload("", "dim1", xs1, off).algorithmic_bytes())
    t0 = time.perf_counter()
    oracle.quant_groups_dim0(xs0, off)
    oracle.quant_groups_dim1(xs1, off)
    dt = time.perf_counter() - t0
    gbps = b / dt / 1e9
    log("cpu oracle: %.2f s on the sample, %.3f GB/s" % (dt, gbps))
    per = []
    for name, (kind, part, arg, pow2, frac, full_bytes) in samples.items():
        t0 = time.perf_counter()
        if kind == "dim0":
            oracle.quant_groups_dim0(part, arg, pow2)
        elif kind == "dim1":
            oracle.quant_groups_dim1(part, arg, pow2)
        else:
            oracle.mx_quant_dim0(part, arg)
        d = time.perf_counter() - t0
        per.append({"config": name, "sample": "%s of %.2f%% of the input" % (
                        "columns" if kind == "dim0" else "rows", 100 * frac),
                    "sample_s": round(d, 3), "est_full_ms": round(1e3 * d / frac, 1),
                    "GBps": round(full_bytes * frac / d / 1e9, 4)})
        log("  cpu oracle %-36s %.3f s on %.2f%%, %.3f GB/s" % (name, d, 100 * frac, per[-1]["GBps"]))
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "dim0 on T[:, :%d] + dim1 on T^T[:%d] (%.1f%% of a step), %.2f s; host: %s, %d cpus"
                      % (ncols, ncols, 100.0 * ncols / T.shape[1], dt, cpu_model(), os.cpu_count()),
            "per_config": per}


if __name__ == "__main__":
    main()

"""Tile timeline of the dim0 kernel: where one launch's time goes.

A diagnostic, not part of the quantisation path. It loads libmgs_trace.so
(the same sources as libmgs.so built with MGS_TILE_TRACE, see build.py and
include/mgs_trace.h) in place of libmgs.so, runs one dim0 workload through
the ordinary entry point (or, with --transposed, dim0_t's), reads back the per-tile stamps and prints a
markdown summary:

- phases of a tile (search, loads and column maxima, reduction, cast and
  store issue) by tile class;
- a least-squares fit of a tile's time against its size;
- compute units used, tiles per unit, the gap between a tile's end and the
  next tile starting in its slot;
- tiles alive, tiles loading and the tile bytes in flight over time;
- the launch's tail after the last tile started;
- for chunk teams, how far apart a team's tiles started.

Two launch conditions: "b2b", the last of four launches back to back on one
stream (the condition of a benchmark step, caches holding the previous
launch's data), and "cold", one launch after a 1 GiB read-only sweep. The
kernel time comes from separate timed runs; the launch summarised is then
run between one-thread stamp kernels, which give its start and end on the
clock of the tile stamps. The GPU's clocks are settled first by 50 ms of
untimed launches.

    python -m group_scaling_fp8_amd.tile_trace [--workload NAME ...] [--transposed] [--out FILE]

Workloads: g64 and g1 (16640 x 8192 bf16; 64 groups at sorted uniform
random cut points, multiples of 16 rows / one group), g256 and g1024 (the
first 16640 / 16384 rows of the same tensor in 256 groups of 65 rows / 1024
of 16), c2 (4096 x 4096, 16 groups at random cut points, one of them empty
and one all zero, pow2 scales), c3 (65536 x 4096, 8 Dirichlet(0.5) groups).
"""
from __future__ import annotations

import argparse
import ctypes
import sys
import time

import numpy as np

from . import _lib
from . import build as _build

CLASS_NAMES = {0: "A", 1: "T", 2: "C"}
TICK_US = 0.01          # s_memrealtime runs at 100 MHz
PREWARM_MS = 50.0


def _trace_library():
    """Points the package's loader at the trace build; must run before any
    other call of the package loads libmgs.so."""
    if _lib._lib is not None and _lib._LIB_PATH != _build.LIB_TRACE:
        raise RuntimeError("libmgs.so is already loaded in this process; run the tile trace in a "
                           "process of its own")
    _lib._LIB_PATH = _build.LIB_TRACE
    L = _lib.lib()
    for name in ("mgs_tile_trace_capacity", "mgs_tile_trace_clear"):
        getattr(L, name).argtypes = []
        getattr(L, name).restype = ctypes.c_int
    L.mgs_tile_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    L.mgs_tile_trace_read.restype = ctypes.c_int
    L.mgs_tile_trace_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.mgs_tile_trace_stamp.restype = ctypes.c_int
    return L


def _workload(name):
    from . import workloads as wl
    if name in ("g64", "g1"):
        T = wl.token_major_gradient()
        off = wl.target_offsets(64) if name == "g64" else np.array([T.shape[0]], np.int32)
        return ("(16640, 8192) bf16, %s" % ("64 groups at random cut points (0 to 1136 rows)"
                                             if name == "g64" else "one group"), T, off, False)
    if name in ("g256", "g1024"):
        T = wl.token_major_gradient()
        n, rows = (256, 65) if name == "g256" else (1024, 16)
        x = T[:n * rows]
        return ("(%d, 8192) bf16, %d equal groups of %d rows" % (n * rows, n, rows), x,
                (np.arange(1, n + 1) * rows).astype(np.int32), False)
    if name == "c2":
        w = wl.c2_dim0_pow2()
        return "(4096, 4096) bf16, 16 groups at random cut points, pow2 scales", w.x, w.offsets, True
    if name == "c3":
        w = wl.c3_dim0_large()
        return "(65536, 4096) bf16, 8 Dirichlet(0.5) groups", w.x, w.offsets, False
    raise ValueError("unknown workload %r" % name)


def decode(raw: np.ndarray) -> dict:
    """The recorded items of one launch as columns (times in us from the
    earliest start)."""
    a = raw.reshape(-1, 8)
    a = a[a[:, 0] != 0].astype(np.int64)
    if len(a) == 0:
        raise RuntimeError("no tile was recorded")
    ts = (a[:, :5] - a[:, 0].min()) * TICK_US
    hw = a[:, 5] >> 32
    return {
        "first_tick": int(a[:, 0].min()),
        "last_tick": int(a[:, 4].max()),
        "t": ts,
        "cu": (a[:, 5] & 0xF) << 16 | ((hw >> 8) & 0xFF),     # XCC, then SE / SH / CU of HW_ID
        "cls": (a[:, 6] >> 60) & 0xF,
        "chunk": (a[:, 6] >> 32) & 0xFFFFFFF,
        "rows": a[:, 6] & 0xFFFFFFFF,
        "group": a[:, 7] >> 40,
        "strip": (a[:, 7] >> 16) & 0xFFFFFF,
        "width": a[:, 7] & 0xFFFF,
    }


def _pct(v):
    return "%.2f | %.2f | %.2f | %.2f | %.2f" % (v.mean(), *np.percentile(v, [10, 50, 90]), v.max())


def summarise(d: dict, kernel_us: float, edges=None) -> list:
    """Markdown lines for one launch; edges = (us from the stamp before the
    launch to its first tile start, us from its last store issue to the
    stamp after it), or None."""
    t = d["t"]
    n = len(t)
    byt = d["rows"] * d["width"] * 3                # 2 B read + 1 B written per element
    end = t[:, 4].max()
    out = ["- tiles recorded: %d (%s); tile bytes %.1f MB (2 B read + 1 B written per element)" % (
        n, ", ".join("class %s %d" % (CLASS_NAMES.get(c, c), np.sum(d["cls"] == c))
                     for c in np.unique(d["cls"])), byt.sum() / 1e6),
           "- kernel time %.2f us (median of 5; cold: HIP events around the launch; back to back: stamp "
           "kernels around three launches, per launch); first tile start to last store issue %.2f us; "
           "last tile start at %.2f us" % (kernel_us, end, t[:, 0].max()),
           ""]
    phases = (("search", t[:, 1] - t[:, 0]), ("loads + column maxima", t[:, 2] - t[:, 1]),
              ("reduction", t[:, 3] - t[:, 2]), ("cast + store issue", t[:, 4] - t[:, 3]),
              ("whole item", t[:, 4] - t[:, 0]))
    out += ["| phase (us) | class | tiles | mean | p10 | p50 | p90 | max |",
            "|---|---|---|---|---|---|---|---|"]
    for name, v in phases:
        for c in np.unique(d["cls"]):
            m = d["cls"] == c
            out.append("| %s | %s | %d | %s |" % (name, CLASS_NAMES.get(c, c), m.sum(), _pct(v[m])))
    kib = d["rows"] * d["width"] * 2 / 1024.0
    tile = t[:, 4] - t[:, 1]
    a = d["cls"] == 0
    if a.sum() >= 8 and np.ptp(kib[a]) > 0:
        slope, icpt = np.polyfit(kib[a], tile[a], 1)
        out += ["", "- class A tile, found to stores issued: %.2f us fixed + %.4f us per KiB of bf16 input "
                "(least squares over %d tiles of %.0f..%.0f KiB)" % (icpt, slope, a.sum(), kib[a].min(),
                                                                     kib[a].max())]
    elif a.sum():
        out += ["", "- class A tile, found to stores issued: %.2f us mean at %.0f KiB" % (
            tile[a].mean(), kib[a].mean())]
    # compute units and their slots
    keys, inv = np.unique(d["cu"], return_inverse=True)
    per_cu = np.bincount(inv)
    slots, gaps = [], []
    for k in range(len(keys)):
        m = np.where(inv == k)[0]
        st, en = np.sort(t[m, 0]), np.sort(t[m, 4])
        ev = np.concatenate([np.stack([t[m, 0], np.ones(len(m))], 1), np.stack([t[m, 4], -np.ones(len(m))], 1)])
        ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]
        s = int(np.cumsum(ev[:, 1]).max())
        slots.append(s)
        # a slot freed by the i-th end is refilled by the (i + s)-th start
        gaps += list(st[s:] - en[:len(st) - s])
    gaps = np.array(gaps) if gaps else np.zeros(1)
    out += ["- compute units used %d; tiles per unit min %d / median %d / max %d; tiles at once per unit "
            "(max) %d; refill gap (a tile's end to the next start in its slot) p50 %.2f p90 %.2f us" % (
                len(keys), per_cu.min(), int(np.median(per_cu)), per_cu.max(), max(slots),
                *np.percentile(gaps, [50, 90]))]
    # timeline, in about 24 bins
    bin_us = 4 * max(1, int(np.ceil(end / 96.0)))
    grid = np.arange(0.0, end + bin_us, 1.0)
    alive = np.array([np.sum((t[:, 0] <= g) & (t[:, 4] > g)) for g in grid])
    loading = np.array([np.sum((t[:, 1] <= g) & (t[:, 2] > g)) for g in grid])
    rate = np.zeros_like(grid)
    for i in range(n):
        m = (grid >= t[i, 1]) & (grid < t[i, 4])
        rate[m] += byt[i] / max(t[i, 4] - t[i, 1], 1e-3) / 1e6
    step = bin_us
    out += ["", "Per %d us from the first tile start (sampled at each bin's start; TB/s spreads each "
            "tile's bytes evenly from its tile found to its stores issued):" % bin_us, "",
            "| us | " + " | ".join("%d" % g for g in grid[::step]) + " |",
            "|---|" + "---|" * len(grid[::step]),
            "| tiles alive | " + " | ".join("%d" % v for v in alive[::step]) + " |",
            "| tiles loading | " + " | ".join("%d" % v for v in loading[::step]) + " |",
            "| TB/s in flight | " + " | ".join("%.1f" % v for v in rate[::step]) + " |", ""]
    if edges is not None:
        out += ["- launch edges (one-thread stamp kernels right before and after this launch on its "
                "stream): first tile start %.2f us after the first stamp; last store issue %.2f us "
                "before the second" % edges]
    late = t[:, 0] > t[:, 0].max() - 15.0
    out += ["- tail: %d tiles start in the last 15 us of starts; last store issue %.2f us after the last "
            "start; kernel time minus the recorded span %.2f us (launch, first-wave start, store drain)" % (
                late.sum(), end - t[:, 0].max(), kernel_us - end)]
    team = d["cls"] != 0
    if team.any():
        key = d["group"][team] * (1 << 24) + d["strip"][team]
        t0 = t[team, 0]
        tw = t[team, 2] - t[team, 1]
        spread = np.array([np.ptp(t0[key == k]) for k in np.unique(key)])
        out += ["- chunk teams: %d; start spread of a team's tiles p50 %.2f p90 %.2f max %.2f us; "
                "team tiles' loads + maxima + team wait p50 %.2f p90 %.2f us" % (
                    len(spread), *np.percentile(spread, [50, 90]), spread.max(), *np.percentile(tw, [50, 90]))]
    return out


def run(names, out_path=None, transposed=False):
    import torch
    L = _trace_library()
    from . import api as mgs
    cap = L.mgs_tile_trace_capacity()
    dev = torch.device("cuda:0")
    sweep = torch.ones(1 << 28, dtype=torch.int32, device=dev)      # 1 GiB, read-only sweeps
    stamps = torch.zeros(2, dtype=torch.int64, device=dev)

    def stamp(i):
        rc = L.mgs_tile_trace_stamp(ctypes.c_void_p(stamps.data_ptr() + 8 * i),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError("mgs_tile_trace_stamp failed: %d" % rc)

    def event_us(fn, cold):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if cold:
            sweep.max()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    # the fixed cost of a launch: a one-thread kernel between HIP events, and
    # two such kernels back to back
    t_pre = time.perf_counter()
    while (time.perf_counter() - t_pre) * 1e3 < PREWARM_MS:
        stamp(0)
    torch.cuda.synchronize()
    fixed_cold = np.median([event_us(lambda: stamp(0), True) for _ in range(20)])
    fixed_idle = np.median([event_us(lambda: stamp(0), False) for _ in range(20)])
    gaps = []
    for _ in range(10):
        stamp(1)            # wakes the queue
        stamp(0)
        stamp(1)
        torch.cuda.synchronize()
        sv = stamps.cpu().numpy()
        gaps.append((sv[1] - sv[0]) * TICK_US)
    props = torch.cuda.get_device_properties(0)
    lines = ["# dim0%s tile timeline" % ("_t" if transposed else ""), "",
             "Command: `python -m group_scaling_fp8_amd.tile_trace %s%s%s` (%s, %s, %d compute units)." % (
                 " ".join("--workload %s" % n for n in names), " --transposed" if transposed else "",
                 " --out FILE" if out_path else "",
                 props.name, getattr(props, "gcnArchName", "?"), props.multi_processor_count), "",
             "The trace build runs the product kernel plus a few stores per tile, so its launches "
             "take a few us longer than libmgs.so's. Times are in us from the launch's first tile "
             "start; classes: A a tile of its own, T a chunk of a team, C column-maximum casting.", "",
             "Fixed cost of any launch: a one-thread kernel takes %.2f us between HIP events right "
             "after a 1 GiB read sweep and %.2f us on an idle queue (medians of 20); two of them "
             "back to back on a busy queue run %.2f us apart (median of 10)." % (
                 fixed_cold, fixed_idle, np.median(gaps)), ""]
    for name in names:
        desc, x_np, off_np, pow2 = _workload(name)
        x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(dev)
        x2 = x.clone()          # alternate inputs so back-to-back launches do not reread cached data
        off = torch.from_numpy(np.asarray(off_np, np.int32)).to(dev)
        M, K = x.shape
        ws = mgs.dim0_workspace(M, K)
        if transposed:
            q, s = mgs.mgs_quant_groups_dim0_t(x, off, pow2, workspace=ws)

            def call(xx):
                mgs.mgs_quant_groups_dim0_t(xx, off, pow2, q_t=q, scales_t=s, workspace=ws)
        else:
            q, s = mgs.mgs_quant_groups_dim0(x, off, pow2, workspace=ws)

            def call(xx):
                mgs.mgs_quant_groups_dim0(xx, off, pow2, q=q, scales=s, workspace=ws)
        t_pre = time.perf_counter()
        while (time.perf_counter() - t_pre) * 1e3 < PREWARM_MS:
            call(x2)
        torch.cuda.synchronize()

        def launch(i):
            call(x if i % 2 == 0 else x2)

        def time_b2b():
            """Per-launch time of three launches back to back, from stamp
            kernels right after the first launch (which takes the wake-up of
            an idle queue) and after the fourth; the first stamp adds its own
            short run to the three. Stamp kernels run in stream order, while
            an event queued behind short launches can be stamped before the
            launch ahead of it ends."""
            launch(1)
            stamp(0)
            for i in range(3):
                launch(i)
            stamp(1)
            torch.cuda.synchronize()
            sv = stamps.cpu().numpy().astype(np.int64)
            return (sv[1] - sv[0]) * TICK_US / 3

        def time_cold():
            sweep.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch(0)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3

        def recorded(mode):
            """The launch whose tiles are summarised: the last of four back
            to back, or one after a read sweep, between stamp kernels."""
            if L.mgs_tile_trace_clear() != 0:
                raise RuntimeError("mgs_tile_trace_clear failed")
            if mode == "b2b":
                for i in range(3):
                    launch(i + 1)
            else:
                sweep.max()
            stamp(0)
            launch(0)
            stamp(1)
            torch.cuda.synchronize()

        for mode in ("b2b", "cold"):
            kernel_us = float(np.median([time_b2b() if mode == "b2b" else time_cold() for _ in range(5)]))
            recorded(mode)
            raw = np.zeros(cap * 8, np.uint64)
            if L.mgs_tile_trace_read(raw.ctypes.data_as(ctypes.c_void_p), raw.nbytes) != 0:
                raise RuntimeError("mgs_tile_trace_read failed")
            sv = stamps.cpu().numpy().astype(np.int64)
            d = decode(raw)
            edges = ((d["first_tick"] - sv[0]) * TICK_US, (sv[1] - d["last_tick"]) * TICK_US)
            lines += ["## %s%s: %s, %s" % (name, " (dim0_t)" if transposed else "", desc,
                                            "the last of four launches back to back" if mode == "b2b"
                                            else "one launch after a 1 GiB read sweep"), ""]
            lines += summarise(d, kernel_us, edges) + [""]
            print("traced %s %s" % (name, mode), file=sys.stderr, flush=True)
        del x, x2, q, s, ws
        torch.cuda.empty_cache()
    text = "\n".join(lines)
    if out_path:
        with open(out_path, "w") as f:
            f.write(text + "\n")
    return text


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", action="append", choices=("g64", "g1", "g256", "g1024", "c2", "c3"))
    ap.add_argument("--transposed", action="store_true",
                    help="the transposed kernel (mgs_quant_groups_dim0_t); offsets must be multiples of 16")
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    print(run(args.workload or ["g64", "c2"], args.out, args.transposed))


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the 25-point (R = 4) star stencil on a 512^3 fp32 interior
(520^3 allocated with a 4-point halo) on one MI355X, plus the acoustic wave
step on a 1024^3 interior (and the PML kernel's step on the same fields),
the R = 1 Jacobi sweeps on 512^3 and the fp64 ragged grid as secondary
figures.

    python bench.py [--steps K] [--warmup W] [--no-wave] [--no-others]
                    [--no-cpu]

Prints ONE JSON line.  A step is one stencil3d_apply over the whole grid
(input already resident in HBM).  `value` = interior points * K / wall time
of the K timed steps (GPoints/s).  `roofline.achieved` = algorithmic bytes
of one launch / its mean duration from HIP events recorded on the launch
stream.  `cpu_baseline` times the CPU oracle on the host cores over a
bounded number of whole-grid applications.

--calib adds a plain device copy of known size (for the counter runs that
turn FETCH_SIZE / WRITE_SIZE into bytes); --ceilings times copy kernels that
walk memory like the apply (libwalkcopy.so) beside it; --only-headline skips everything
but the timed stencil launches, --only-others runs only the Jacobi and fp64
workloads, --only-wave {wave,pml,regions,pml_regions,blocked,blocked_regions,
pml_blocked,both,all} only
the 1032^3 leapfrog with those step kinds (both: wave and pml; all: every
kind; for profiler runs).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
METRIC = ("GPoints/s and achieved HBM GB/s (% of peak), "
          "R=4 25-pt stencil at 512³ fp32")
PROF = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROF, "star2p5d_r4_512cube_traffic.md")
WAVE_TRAFFIC = {v: os.path.join(PROF, "%s_r4_1024cube_traffic.md" % v)
                for v in ("wave", "pml", "blocked", "blocked_regions", "pml_blocked")}
COUNTERS = {"headline": os.path.join(PROF, "star2p5d_r4_512cube_counters.md"),
            "blocked": os.path.join(PROF, "blocked_r4_1024cube_counters.md"),
            "pml_blocked": os.path.join(PROF, "pml_blocked_r4_1024cube_counters.md"),
            "jacobi": os.path.join(PROF, "jacobi_r1_512cube_counters.md")}
JACOBI_TRAFFIC = os.path.join(PROF, "jacobi_r1_512cube_traffic.md")
F64_TRAFFIC = os.path.join(PROF, "apply_r4_f64_ragged_traffic.md")
# VALU issue rate: a wave64 fp32 VALU instruction holds a 16-lane SIMD for 4
# cycles (packed FP32 is off); MI355X has 256 CUs x 4 SIMDs at 2.4 GHz
VALU_CYCLES, SIMDS, CLOCK_HZ = 4, 1024, 2.4e9


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _current(text: str) -> bool:
    """Whether a profile summary was taken on the current kernel sources (its
    source set's hash still matches)."""
    from acoustic_wave_propagation_amd.profiling import SOURCE_SETS, kernel_hash
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    srcs = re.search(r"kernel_sources:\s*(\w+)", text)
    name = srcs.group(1) if srcs else "stream"
    return bool(m) and name in SOURCE_SETS and m.group(1) == kernel_hash(name)


def recorded_traffic(kernel: str, path: str = TRAFFIC_FILE, what="traffic"):
    """Bytes per launch measured by the committed counter runs (what:
    "traffic", "read" or "write"), if they were taken on the current kernel
    source; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    t = re.search(r"%s_bytes_per_launch\[%s\]:\s*([0-9.eE+]+)" %
                  (what, re.escape(kernel)), text)
    if not t or not _current(text):
        return None
    return float(t.group(1))


def recorded_counter(path: str, counter: str):
    """Mean per dispatch of a counter in a committed counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    t = re.search(r"counter_mean\[%s\]:\s*([0-9.eE+]+)" % re.escape(counter), text)
    if not t or not _current(text):
        return None
    return float(t.group(1))


def valu_roofline(counters_path: str, kernel_s: float, launches: float = 1.0):
    """VALU bound of a kernel from its committed SQ_INSTS_VALU: the issue time
    of its VALU instructions spread over every SIMD, against the measured
    time of `launches` dispatches (None if the counters are stale)."""
    insts = recorded_counter(counters_path, "SQ_INSTS_VALU")
    if insts is None:
        return None
    t = insts * launches * VALU_CYCLES / (SIMDS * CLOCK_HZ)
    return dict(bound="alu", insts_per_dispatch=insts, issue_ms=round(t * 1e3, 5),
                measured_ms=round(kernel_s * 1e3, 5), frac=round(t / kernel_s, 4),
                derivation="SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x 2.4 GHz)")


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def reported_hbm_peak(torch):
    """Peak HBM GB/s from the device's reported memory clock and bus width
    (double data rate), where the runtime reports them; else None."""
    p = torch.cuda.get_device_properties(0)
    clk = getattr(p, "memory_clock_rate", None)   # kHz
    bus = getattr(p, "memory_bus_width", None)    # bits
    if not clk or not bus:
        return None
    return round(2.0 * clk * 1e3 * bus / 8 / 1e9, 1)


WARM_S = 0.25  # least device time of untimed calls before a timed region


def timed_launches(torch, fn, steps, warmup):
    """Untimed calls, at least W + 1 of them and at least WARM_S seconds of them
    (the GPU's clocks ramp up under load: after 10 launches of the 520^3
    apply a step takes ~0.223 ms, after 200 ~0.210 ms, and half a second idle
    undoes it), then K timed ones back to back: their wall time (synchronised
    on both sides).  Then K more calls, each bracketed by HIP events on the
    launch stream, for per-launch durations; the events stay out of the
    wall-timed region, where they would add a stream packet and a gap between
    consecutive kernels."""
    stream = torch.cuda.current_stream()
    fn()  # the first call also loads code objects: not a timing sample
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    for _ in range(max(warmup, 1)):
        fn()
    torch.cuda.synchronize()
    spent = time.perf_counter() - t_warm
    # the rest of the warm-up time in one back-to-back batch
    per_call = spent / max(warmup, 1)
    for _ in range(int(np.ceil(max(WARM_S - spent, 0.0) / per_call))):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3  # s
    return wall, durs


def flushed_launches(torch, fn, steps, flush_bytes=1 << 30):
    """Launch durations with 1 GiB of scratch read before each launch, so
    that no part of the inputs can still sit in the 256 MB Infinity Cache (or
    L2) from the previous launch.  Reading (not writing) leaves clean lines,
    so evicting them costs the launch nothing."""
    stream = torch.cuda.current_stream()
    scratch = torch.ones(flush_bytes // 4, dtype=torch.float32,
                         device="cuda:0")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        sink += scratch.sum()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in ev])
    del scratch, sink
    torch.cuda.empty_cache()
    return dict(mean=float(durs.mean()), median=float(np.median(durs)),
                min=float(durs.min()), launches=steps,
                flush="1 GiB scratch read before each launch")


def cpu_rate(fn, points, budget_s):
    """Run fn (one oracle evaluation over `points` outputs) until the budget
    is spent (at least once); GPoints/s from the median duration."""
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    med = float(np.median(times))
    return points / med / 1e9, len(times), med


# algorithmic bytes: one read of the interior plus its 2R-deep face slabs,
# one write of the interior (edges and corners of the halo are never read);
# the wave step adds u_prev, vel2 and eta
from acoustic_wave_propagation_amd.traffic import apply_bytes as star_bytes  # noqa: E402
from acoustic_wave_propagation_amd.traffic import wave_bytes  # noqa: E402


def walk_lib():
    """libwalkcopy.so: copy kernels with the apply's memory walk."""
    import ctypes
    path = os.path.join(ROOT, "acoustic_wave_propagation_amd", "libwalkcopy.so")
    if not os.path.exists(path):
        raise RuntimeError("libwalkcopy.so is not built (%s); run "
                           "python -m acoustic_wave_propagation_amd.build" % path)
    L = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.walk_copy_zmarch.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp]
    L.walk_copy_rows.argtypes = [vp, vp, i32, i32, i32, vp]
    return L


def bench_ceilings(torch, inp, out, steps, warmup, full=True):
    """Copies of the 512^3 interior of the 520^3 grid (inp -> out): with
    the apply kernel's memory walk but without its arithmetic, and one-shot
    row copies.  zmarch: 512-thread workgroups streaming 256 x 16 (or
    512 x 8) tiles through 4 chunks of 128 planes, one barrier per step;
    rows: one-shot row copies.  Stores at the rows' own place (16 bytes into
    each row, so each row's end sectors are written in part), shifted to
    the row start (whole 32-byte sectors), or with the rows' halo rewritten
    from out (whole sectors).  ms are mean HIP-event launch durations;
    stencil_frac is the apply's algorithmic bytes over that time over 8 TB/s,
    the fraction the stencil would report at the copy's speed."""
    L = walk_lib()
    n, R = inp.shape[0], 4
    stream = torch.cuda.current_stream().cuda_stream
    ip, op = inp.data_ptr(), out.data_ptr()
    variants = [("zmarch_256x16", lambda: L.walk_copy_zmarch(ip, op, n, R, 256, 4, 0, stream)),
                ("zmarch_256x16_aligned",
                 lambda: L.walk_copy_zmarch(ip, op, n, R, 256, 4, 1, stream))]
    if full:
        variants += [
            ("zmarch_512x8", lambda: L.walk_copy_zmarch(ip, op, n, R, 512, 4, 0, stream)),
            ("zmarch_512x8_aligned",
             lambda: L.walk_copy_zmarch(ip, op, n, R, 512, 4, 1, stream)),
            ("rows", lambda: L.walk_copy_rows(ip, op, n, R, 0, stream)),
            ("rows_halo_rewritten", lambda: L.walk_copy_rows(ip, op, n, R, 2, stream)),
            ("rows_aligned", lambda: L.walk_copy_rows(ip, op, n, R, 1, stream))]
    ni = n - 2 * R
    copy_b = 2 * 4 * ni ** 3
    stencil_b = star_bytes((ni, ni, ni), R, 4)
    res = {}
    for name, fn in variants:
        if fn() != 0:
            raise RuntimeError("walk_copy %s refused the grid" % name)
        _, durs = timed_launches(torch, fn, steps, warmup)
        ms = float(durs.mean()) * 1e3
        res[name] = dict(ms=round(ms, 4), copy_gbs=round(copy_b / ms / 1e6, 1),
                         stencil_frac=round(stencil_b / ms / 1e6 / PEAK_HBM_GBS, 4))
    return res


def bench_headline(torch, B, wl, args):
    w = wl.R4_512
    dev = torch.device("cuda:0")
    log("generating %s %s" % (w.name, w.shape))
    host = wl.input_planes(w)
    inp = torch.from_numpy(host).to(dev)
    out = torch.zeros_like(inp)
    d = B.desc_init("f32", w.shape, w.radius)
    fn = lambda: B.stencil3d_apply(d, inp, out)
    wall, durs = timed_launches(torch, fn, args.steps, args.warmup)
    pts = w.interior_points
    nbytes = star_bytes(w.interior, w.radius, 4)
    mean = float(durs.mean())
    achieved = nbytes / mean / 1e9
    flushed = None if args.only_headline else flushed_launches(
        torch, fn, min(args.steps, 20))
    res = dict(
        value=pts * args.steps / wall / 1e9,
        ms_per_step=wall / args.steps * 1e3,
        kernel_ms=dict(mean=mean * 1e3, median=float(np.median(durs)) * 1e3,
                       min=float(durs.min()) * 1e3,
                       p90=float(np.percentile(durs, 90)) * 1e3),
        kernel_ms_cache_flushed=flushed,
        roofline=dict(bound="hbm", achieved=round(achieved, 1),
                      peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(achieved / PEAK_HBM_GBS, 4),
                      traffic=recorded_traffic("star2p5d_r4_f32"),
                      algorithmic_bytes=nbytes,
                      # counter reads and writes against their floors
                      traffic_read=recorded_traffic("star2p5d_r4_f32",
                                                    what="read"),
                      traffic_write=recorded_traffic("star2p5d_r4_f32",
                                                     what="write"),
                      read_floor=nbytes - 4 * pts, write_floor=4 * pts,
                      kernel="star2p5d_kernel<float,4,false>",
                      valu=valu_roofline(COUNTERS["headline"], mean)),
        gbs_wall=round(nbytes * args.steps / wall / 1e9, 1),
    )
    # plain copies of the same interior (context): with the apply's walk,
    # and one-shot row copies, the fastest way found to move those bytes
    # (not in profiling runs, which time the apply alone)
    if args.only_headline:
        return res, host
    res["roofline"]["walk_copies"] = dict(
        bench_ceilings(torch, inp, out, min(args.steps, 100), args.warmup),
        note="copies of the 512^3 interior: zmarch_* with the apply's walk "
             "(tiles streaming 4 chunks of 128 planes, a barrier per step), "
             "rows_* one-shot; *_aligned: rows stored from the row start "
             "(whole 32-byte sectors); stencil_frac: the apply's algorithmic "
             "bytes over the copy's time over 8 TB/s")
    return res, host


def bench_wave(torch, B, wl, args,
               variants=("wave", "pml", "regions", "pml_regions", "blocked",
                         "blocked_regions", "pml_blocked")):
    """20-step leapfrog on 1032^3 (1024^3 interior), native time loop, with
    the pointwise step ("wave"), the PML kernel's step ("pml"), both
    launched as data regions ("regions", "pml_regions": pml_width = the
    sponge width, so eta is read only near the faces) and the
    time-blocked runs ("blocked", "pml_blocked": two steps per pass over four
    buffers; "blocked_regions": the plain one with the sponge width)."""
    w = wl.WAVE_1024
    e = w.extra
    dev = torch.device("cuda:0")
    log("generating %s %s" % (w.name, w.shape))
    shp = w.shape

    def up(gen):
        t = torch.empty(shp, dtype=torch.float32, device=dev)
        for z0 in range(0, shp[0], 64):
            z1 = min(shp[0], z0 + 64)
            t[z0:z1].copy_(torch.from_numpy(gen(z0, z1)))
        return t

    vel2 = up(lambda a, b: wl.vel2_planes(w, a, b))
    eta = up(lambda a, b: wl.eta_planes(w, a, b))
    u_prev = torch.zeros_like(vel2)
    u = torch.zeros_like(vel2)
    work = ([torch.zeros_like(vel2) for _ in range(2)]
            if any("blocked" in v for v in variants) else None)
    # pml_width 0: one launch reading eta everywhere (the "wave" line);
    # the "regions" line states the sponge width (data regions)
    d = B.desc_init("f32", shp, w.radius)
    src = wl.source_point(w)
    trace = wl.source_trace(w)
    runs = max(1, min(args.steps, 5))
    pts = w.interior_points * w.sweeps
    # one read and one write per field: u (with its face slabs), u_prev,
    # vel2, eta read, u_next written.  The PML kernel's step (eta-gradient
    # coupling, eta's 7-point stencil) moves the same bytes: eta's
    # neighbours come from LDS and registers.
    nbytes = wave_bytes(w.interior, w.radius, 4)
    # data regions: eta is zero from depth `sponge` on, so the wave step
    # reads it only on the points eta_read_points counts; the true bytes
    # lack the other eta reads
    dr = B.desc_init("f32", shp, w.radius)
    dr.pml_width = e["sponge"]
    # (the PML step's data regions run on its own 128-wide tiles, the
    # two-step pass on 56-wide output tiles)
    eta_pts = {"regions": eta_read_points(w.interior, e["sponge"]),
               "pml_regions": eta_read_points(w.interior, e["sponge"],
                                              tile_x=128),
               "blocked_regions": eta_read_points(w.interior, e["sponge"],
                                                  tile_x=56)}
    res = {}
    for v in variants:
        dv = dr if v in ("regions", "pml_regions", "blocked_regions") else d
        if v in ("blocked", "pml_blocked", "blocked_regions"):
            # 20 steps = 10 passes; the fields end in (u_prev, u) again
            fn = lambda: B.wave_run_blocked(dv, u_prev, u, work[0], work[1],
                                            vel2, eta, e["dt"], e["h"],
                                            w.sweeps, src, trace,
                                            pml=(v == "pml_blocked"))
        else:
            fn = lambda: B.wave_run(dv, u_prev, u, vel2, eta, e["dt"], e["h"],
                                    w.sweeps, src, trace,
                                    pml=(v in ("pml", "pml_regions")))
        wall, durs = timed_launches(torch, fn, runs, 1)
        per = float(durs.mean()) / w.sweeps
        ach = nbytes / per / 1e9
        res[v] = dict(value=pts * runs / wall / 1e9, unit="GPoints/s",
                      ms_per_step=per * 1e3, steps_per_run=w.sweeps,
                      runs=runs,
                      roofline=dict(bound="hbm", achieved=round(ach, 1),
                                    peak=PEAK_HBM_GBS, unit="GB/s",
                                    frac=round(ach / PEAK_HBM_GBS, 4),
                                    traffic=recorded_traffic(
                                        "%s_r4_f32" % v, WAVE_TRAFFIC[v])
                                    if v in WAVE_TRAFFIC else None,
                                    algorithmic_bytes_per_step=nbytes))
        if v in ("blocked", "pml_blocked", "blocked_regions"):
            # what a pass of two steps moves: the single step's reads plus
            # a second written field.  achieved / frac are the pass kernel's
            # own bytes over its own time; the per-step equivalent (20.09
            # B/point per step, the single step's convention) is named apart.
            pass_b = nbytes + 4 * w.interior_points
            rl = res[v]["roofline"]
            rl["achieved_step_equivalent"] = rl["achieved"]
            rl["frac_step_equivalent"] = rl["frac"]
            rl["achieved"] = round(pass_b / (2 * per) / 1e9, 1)
            rl["frac"] = round(pass_b / (2 * per) / 1e9 / PEAK_HBM_GBS, 4)
            rl["pass_bytes"] = pass_b
            rl["traffic_per"] = "pass (one launch, two steps)"
            rl["kernel"] = {"pml_blocked": "wave2_kernel<float,4,PML>",
                            "blocked_regions": "wave2_kernel<float,4,data regions>"
                            }.get(v, "wave2_kernel<float,4>")
            rl["valu"] = (valu_roofline(COUNTERS[v], 2 * per)
                          if v in COUNTERS else None)
            rl["note"] = ("achieved/frac: pass bytes over pass time (one "
                          "pass = two steps); *_step_equivalent: 20.09 "
                          "B/point per step over the per-step time")
        if v in ("regions", "pml_regions"):
            true_b = nbytes - 4 * (w.interior_points - eta_pts[v])
            res[v]["roofline"]["true_bytes_per_step"] = true_b
            res[v]["roofline"]["achieved_true_bytes"] = round(
                true_b / per / 1e9, 1)
            res[v]["pml_width"] = e["sponge"]
        if v == "blocked_regions":
            # the pass reads eta once per point of its tiles (stage 1), on
            # the points eta_read_points counts for 56-wide output tiles
            # (the tiles' overlap columns aside)
            true_b = res[v]["roofline"]["pass_bytes"] - 4 * (
                w.interior_points - eta_pts[v])
            res[v]["roofline"]["true_pass_bytes"] = true_b
            res[v]["roofline"]["achieved_true_bytes"] = round(
                true_b / (2 * per) / 1e9, 1)
            res[v]["pml_width"] = e["sponge"]
        log("%s: %.1f GPoints/s, %.3f ms/step, %.1f GB/s"
            % ({"wave": "wave", "pml": "wave, PML step",
                "regions": "wave, data regions",
                "pml_regions": "wave, PML step, data regions",
                "blocked": "wave, time-blocked",
                "blocked_regions": "wave, time-blocked, data regions",
                "pml_blocked": "wave, PML step, time-blocked"}[v],
               res[v]["value"],
               res[v]["ms_per_step"], ach))
    del vel2, eta, u_prev, u, work
    torch.cuda.empty_cache()
    for v in variants:
        if v in ("regions", "pml_regions", "blocked", "blocked_regions",
                 "pml_blocked"):  # updates timed above
            continue
        res[v]["cpu_baseline"] = None if args.no_cpu else cpu_wave_slab(
            wl, w, args.cpu_budget / 4, pml=(v == "pml"))
    for v in ("regions", "blocked", "blocked_regions"):
        if v in res:
            res[v]["cpu_baseline"] = res.get("wave", {}).get("cpu_baseline")
    for v in ("pml_regions", "pml_blocked"):
        if v in res:
            res[v]["cpu_baseline"] = res.get("pml", {}).get("cpu_baseline")
    if "wave" not in res:
        return res
    out = dict(workload=w.name, **res["wave"])
    out["roofline"]["note"] = ("per-step mean incl. the 1-thread source "
                               "kernel; bytes in the one-read-one-write "
                               "convention for all five fields (20.09 "
                               "B/point)")
    if "pml" in res:
        out["pml_step"] = res["pml"]
        if "pml_regions" in res:
            out["pml_step"]["data_regions"] = res["pml_regions"]
        if "pml_blocked" in res:
            out["pml_step"]["time_blocked"] = res["pml_blocked"]
    if "regions" in res:
        out["data_regions"] = res["regions"]
    if "blocked" in res:
        out["time_blocked"] = res["blocked"]
        if "blocked_regions" in res:
            out["time_blocked"]["data_regions"] = res["blocked_regions"]
    return out


def eta_read_points(interior, pw, tile_x=256, group=4):
    """Interior points whose eta the data-region wave step loads (fp32,
    sponge width pw): every point of the rows within pw of a y face (their
    own launches); in the other rows every point of the planes within pw of
    a z face, and elsewhere the 4-column groups within pw of an x face or of
    a multiple of two tile widths (tile_x: 256 for the wave step, 128 for
    the PML step; each tile reads pw of its columns)."""
    iz, iy, ix = interior
    ox = np.arange(0, ix, group)              # group starts, interior coords
    m = ox % (2 * tile_x)                     # position in the two-tile band period
    cols = ((ox < pw) | (ox + group > ix - pw) | (m < pw) |
            (m + group > 2 * tile_x - pw))
    ncols = int(np.minimum(group, ix - ox)[cols].sum())
    slabs = 2 * pw * ix * iz
    rows = iy - 2 * pw
    return slabs + rows * (2 * pw * ix + (iz - 2 * pw) * ncols)


def cpu_wave_slab(wl, w, budget_s, planes=64, pml=False):
    """The oracle's wave step (pml: the PML step) on a slab of the 1032^3
    workload: `planes` interior z planes (plus the R halo planes on each
    side) of the real fields, mid-simulation values for u and u_prev (seeded
    uniform), the real vel2 and eta."""
    import oracle
    e = w.extra
    R = w.radius
    z0 = w.shape[0] // 2 - planes // 2 - R
    z1 = z0 + planes + 2 * R
    v2 = wl.vel2_planes(w, z0, z1)
    et = wl.eta_planes(w, z0, z1)
    shp = (z1 - z0,) + tuple(w.shape[1:])
    u = wl.uniform_planes(shp, w.seed + 17, -1, 1)
    up = wl.uniform_planes(shp, w.seed + 18, -1, 1)
    c = oracle.laplacian_weights(R)
    out = np.zeros(shp, np.float64)
    npts = planes * (w.shape[1] - 2 * R) * (w.shape[2] - 2 * R)
    step = oracle.wave_step_pml if pml else oracle.wave_step
    rate, nrun, med = cpu_rate(
        lambda: step(up, u, v2, et, R, c, e["dt"], e["h"], out=out),
        npts, budget_s)
    return dict(value=round(rate, 4), unit="GPoints/s",
                cores=oracle.num_threads(), kind="oracle",
                sample="%d %s steps on a %d-plane z slab of the 1032^3 "
                       "grid (fp64 oracle), median %.2f s each"
                       % (nrun, "PML" if pml else "wave", planes, med))


def bench_others(torch, B, wl, args):
    """The remaining workloads, each timed the same way as the headline:
    10-sweep Jacobi with the R = 1 7-point stencil on 512^3, and one R = 4
    fp64 application on the ragged 1001 x 603 x 297 grid."""
    dev = torch.device("cuda:0")
    res = {}
    runs = max(1, min(args.steps, 10))

    w = wl.R1_JACOBI_512
    log("generating %s %s" % (w.name, w.shape))
    host_j = wl.input_planes(w)
    a = torch.from_numpy(host_j).to(dev)
    b = torch.empty_like(a)
    d = B.desc_init("f32", w.shape, w.radius, B.DIRICHLET_COPY)
    wall, durs = timed_launches(
        torch, lambda: B.stencil3d_jacobi(d, a, b, w.sweeps), runs, 1)
    call = float(durs.mean())
    per = call / w.sweeps
    nbytes = star_bytes(w.interior, w.radius, 4)
    # the call's own bytes: each pass reads and writes the field once (the
    # sweep's algorithmic bytes); the passes are the library's own plan
    passes, plan_ns = B.stencil3d_jacobi_plan(d, w.sweeps)
    call_b = nbytes * passes if passes else None
    res[w.name] = dict(
        value=round(w.interior_points * w.sweeps * runs / wall / 1e9, 2),
        unit="GPoints/s", ms_per_sweep=round(per * 1e3, 5),
        ms_per_call=round(call * 1e3, 5),
        sweeps_per_run=w.sweeps, runs=runs,
        roofline=dict(bound="hbm",
                      achieved=round(call_b / call / 1e9, 1) if call_b else None,
                      peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(call_b / call / 1e9 / PEAK_HBM_GBS, 4)
                      if call_b else None,
                      passes_per_call=passes, sweeps_per_pass=plan_ns,
                      bytes_per_call=call_b,
                      achieved_sweep_equivalent=round(nbytes / per / 1e9, 1),
                      frac_sweep_equivalent=round(nbytes / per / 1e9 / PEAK_HBM_GBS, 4),
                      algorithmic_bytes_per_sweep=nbytes,
                      kernel="sweeps_fused_kernel<float,1,%d>" % max(plan_ns),
                      traffic=recorded_traffic("jacobi_r1_f32", JACOBI_TRAFFIC),
                      valu=valu_roofline(COUNTERS["jacobi"], call / passes)
                      if passes else None,
                      note="achieved/frac: the call's own bytes (one read and "
                           "one write of the field per fused pass) over the "
                           "call time, boundary copy included; "
                           "*_sweep_equivalent: one sweep's algorithmic bytes "
                           "over the per-sweep time, which temporal blocking "
                           "lets exceed the floor"))
    del a, b
    if not args.no_cpu:
        import oracle
        c = list(d.cx[:2])
        out = np.zeros(host_j.shape, np.float64)
        rate, nrun, med = cpu_rate(
            lambda: oracle.star_apply(host_j, 1, c, boundary=1, out=out),
            w.interior_points, args.cpu_budget / 4)
        res[w.name]["cpu_baseline"] = dict(
            value=round(rate, 4), unit="GPoints/s", cores=oracle.num_threads(),
            kind="oracle", sample="%d single sweeps of the 512^3 grid "
            "(fp64 oracle), median %.2f s each" % (nrun, med))
    del host_j

    w = wl.R4_RAGGED_F64
    log("generating %s %s" % (w.name, w.shape))
    host_f = wl.input_planes(w)
    inp = torch.from_numpy(host_f).to(dev)
    out = torch.zeros_like(inp)
    d = B.desc_init("f64", w.shape, w.radius)
    wall, durs = timed_launches(
        torch, lambda: B.stencil3d_apply(d, inp, out), args.steps,
        args.warmup)
    per = float(durs.mean())
    nbytes = star_bytes(w.interior, w.radius, 8)
    res[w.name] = dict(
        value=round(w.interior_points * args.steps / wall / 1e9, 2),
        unit="GPoints/s", kernel_ms=round(per * 1e3, 5),
        roofline=dict(bound="hbm", achieved=round(nbytes / per / 1e9, 1),
                      peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(nbytes / per / 1e9 / PEAK_HBM_GBS, 4),
                      algorithmic_bytes=nbytes,
                      kernel="star2p5d_kernel<double,4,false>",
                      traffic=recorded_traffic("apply_r4_f64", F64_TRAFFIC)))
    del inp, out
    torch.cuda.empty_cache()
    if not args.no_cpu:
        import oracle
        c = oracle.laplacian_weights(w.radius)
        out = np.zeros(host_f.shape, np.float64)
        rate, nrun, med = cpu_rate(
            lambda: oracle.star_apply(host_f, w.radius, c, out=out),
            w.interior_points, args.cpu_budget / 4)
        res[w.name]["cpu_baseline"] = dict(
            value=round(rate, 4), unit="GPoints/s", cores=oracle.num_threads(),
            kind="oracle", sample="%d applications of the whole ragged fp64 "
            "grid (fp64 oracle), median %.2f s each" % (nrun, med))
    return res


def cpu_baseline(wl, host, budget_s):
    """The oracle as it stands, on the host cores: whole 520^3 applications
    repeated until the time budget is spent (at least one)."""
    import oracle
    w = wl.R4_512
    c = oracle.laplacian_weights(w.radius)
    out = np.zeros(host.shape, dtype=np.float64)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.star_apply(host, w.radius, c, out=out)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    med = float(np.median(times))
    # context: the same application on one thread (one run)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    t0 = time.perf_counter()
    oracle.star_apply(host, w.radius, c, out=out)
    single = time.perf_counter() - t0
    oracle.set_num_threads(threads)
    return dict(value=round(w.interior_points / med / 1e9, 4),
                unit="GPoints/s", cores=threads, kind="oracle",
                host=host_cpu_model(),
                single_thread_value=round(w.interior_points / single / 1e9, 4),
                sample="%d whole-grid applications of the 520^3 R=4 fp32 "
                       "workload (fp64 oracle, long-double accumulation); "
                       "median %.2f s each" % (len(times), med))


def calib_copy(torch, nbytes=1 << 30):
    """A plain device copy of known size, for scaling the counters."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("calibration copy: %d bytes read, %d bytes written per launch"
        % (nbytes, nbytes))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-wave", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calib", action="store_true")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--only-others", action="store_true",
                    help="run only the Jacobi and fp64 workloads (profiling)")
    ap.add_argument("--ceilings", action="store_true",
                    help="time only the copy kernels with the apply's memory "
                         "walk (libwalkcopy.so) beside the apply, one JSON line")
    ap.add_argument("--only-wave",
                    choices=("wave", "pml", "regions", "pml_regions",
                             "blocked", "blocked_regions", "pml_blocked",
                             "both", "all"),
                    help="run only the 1032^3 leapfrog with that step "
                         "(profiling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from acoustic_wave_propagation_amd import binding as B
    from acoustic_wave_propagation_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fail loudly if the library is missing

    if args.ceilings:
        w = wl.R4_512
        inp = torch.from_numpy(wl.input_planes(w)).to("cuda:0")
        out = torch.zeros_like(inp)
        d = B.desc_init("f32", w.shape, w.radius)
        _, durs = timed_launches(torch, lambda: B.stencil3d_apply(d, inp, out),
                                 args.steps, args.warmup)
        ms = float(durs.mean()) * 1e3
        nb = star_bytes(w.interior, w.radius, 4)
        res = dict(apply=dict(ms=round(ms, 4),
                              stencil_frac=round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)))
        res.update(bench_ceilings(torch, inp, out, args.steps, args.warmup))
        print(json.dumps(dict(workload=w.name, ceilings=res)), flush=True)
        return
    if args.only_wave:
        bench_wave(torch, B, wl, args,
                   variants={"both": ("wave", "pml"),
                             "all": ("wave", "pml", "regions", "pml_regions",
                                     "blocked", "blocked_regions",
                                     "pml_blocked")}.get(
                                 args.only_wave, (args.only_wave,)))
        if args.calib:
            calib_copy(torch)
        return
    if args.only_others:
        for k, v in bench_others(torch, B, wl, args).items():
            log("%s: %.1f GPoints/s, %s GB/s"
                % (k, v["value"], v["roofline"]["achieved"]))
        if args.calib:
            calib_copy(torch)
        return
    head, host = bench_headline(torch, B, wl, args)
    log("headline: %.1f GPoints/s, kernel %.4f ms, %.1f GB/s"
        % (head["value"], head["kernel_ms"]["mean"],
           head["roofline"]["achieved"]))
    if args.calib:
        calib_copy(torch)
    if args.only_headline:
        return
    wave = None if args.no_wave else bench_wave(torch, B, wl, args)
    others = None if args.no_others else bench_others(torch, B, wl, args)
    if others:
        for k, v in others.items():
            log("%s: %.1f GPoints/s, %s GB/s"
                % (k, v["value"], v["roofline"]["achieved"]))
    cpu = None if args.no_cpu else cpu_baseline(wl, host, args.cpu_budget)

    w = wl.R4_512
    line = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": "GPoints/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded uniform [-1,1])",
        "config": {"workload": w.name, "grid": list(w.shape[::-1]),
                   "interior": list(w.interior[::-1]), "radius": w.radius,
                   "boundary": "halo_untouched",
                   "device": torch.cuda.get_device_name(0),
                   "hbm_peak_reported_gbs": reported_hbm_peak(torch)},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "kernel_ms": head["kernel_ms"],
        "kernel_ms_cache_flushed": head["kernel_ms_cache_flushed"],
        "hbm_gbs_wall": head["gbs_wall"],
        "wave_step": wave,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

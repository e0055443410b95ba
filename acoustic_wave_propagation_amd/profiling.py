"""Summaries of rocprofv3 output (rocpd SQLite databases or CSV directories).

    python -m acoustic_wave_propagation_amd.profiling trace DB --cmd "..."
    python -m acoustic_wave_propagation_amd.profiling traffic FETCH_DB WRITE_DB \
        --kernel star2p5d_kernel --name star2p5d_r4_f32 --calib-bytes 1073741824 \
        --cmd-fetch "..." --cmd-write "..."
    python -m acoustic_wave_propagation_amd.profiling counters DB [DB ...] \
        --kernel star2p5d_kernel --cmd "..." [--cmd "..."]

`trace` prints the per-kernel call count and duration statistics of a
`--kernel-trace --stats` run.  `traffic` turns two `--pmc FETCH_SIZE` /
`--pmc WRITE_SIZE` runs into bytes per launch: each counter (KiB per
dispatch) is scaled by the bytes a plain device copy of known size moved,
divided by what the same counter read for that copy (the copy is the
runtime's copyBuffer kernel that the benchmark's --calib flag launches).
`counters` tabulates the mean per dispatch of every counter of any number of
`--pmc` runs for one kernel, with L2 hit rate and LDS ratios derived.
The output also records a hash of the kernel sources (comments and
whitespace ignored), so a consumer can tell whether the figures still
describe the current kernel.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
_STREAM = ["star2p5d_kernel.h", "work_plan.h", "star2p5d.hip"]
# The sources each summary's figures depend on: a summary is stale once any
# of them changes (comments and whitespace aside).
SOURCE_SETS = {
    "stream": _STREAM,                                     # apply, wave, PML step
    "blocked": _STREAM + ["wave2_kernel.h", "wave2.hip"],  # two-step pass
    "fused": _STREAM + ["sweeps_fused_kernel.h", "sweeps_fused.hip",
                        "pass_plan.h"],                    # fused Jacobi passes
    "walk": _STREAM + ["walk_copy.hip"],                   # the apply beside its copies
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: what
    the compiler sees, so that editing a comment leaves the hash alone.
    (String literals in these sources contain no comment markers.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(sources: str = "stream") -> str:
    """Hash of the code (comments and whitespace ignored) of one source set."""
    h = hashlib.sha256()
    for name in SOURCE_SETS[sources]:
        with open(os.path.join(PKG, "csrc", name), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _stamp(sources: str) -> list:
    return ["kernel_sources: " + sources + " (" + ", ".join(SOURCE_SETS[sources]) + ")",
            "kernel_source_sha256_16: " + kernel_hash(sources), ""]


def _db(path):
    if os.path.isdir(path):
        found = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
        if not found:
            raise FileNotFoundError("no rocpd database under " + path)
        path = found[0]
    return sqlite3.connect(path)


def kernel_stats(path):
    """[(name, calls, total_us, avg_us, min_us, max_us)] by total time.
    Instantiations that share a (truncated) name are told apart by their
    kernel id and labelled with workgroups x threads, LDS bytes and the
    trace's vgpr_count field (for these wave64 kernels half the compiler's
    VGPR figure, rounded up to 8 VGPRs first: 96 for 192, 116 for 229)."""
    db = _db(path)
    rows = db.execute(
        "select name, count(*), sum(duration), avg(duration), min(duration), "
        "max(duration), max(grid_x / workgroup_x), max(workgroup_x), "
        "max(lds_size), max(vgpr_count), count(distinct kernel_id) from "
        "kernels group by name, kernel_id order by sum(duration) desc"
    ).fetchall()
    names = {}
    for r in rows:
        names[r[0]] = names.get(r[0], 0) + 1
    out = []
    # durations are in ns
    for n, c, t, a, mn, mx, wgs, thr, lds, vg, _ in rows:
        label = n if names[n] == 1 else "%s [%d x %d, LDS %d, vgpr_count %d]" % (
            n, wgs, thr, lds, vg)
        out.append((label, c, t / 1e3, a / 1e3, mn / 1e3, mx / 1e3))
    return out


def counter_means(path, counter):
    """{kernel name: (dispatches, mean counter value)}."""
    db = _db(path)
    rows = db.execute(
        "select name, count(*), avg(counter_value) from pmc_events where "
        "counter_name = ? group by name", (counter,)).fetchall()
    return {n: (c, v) for n, c, v in rows}


def trace_md(path, cmd, sources="stream") -> str:
    out = ["# Kernel trace summary", "",
           "Command (run from /tmp, repository at $REPO, raw output under $RAW):", "",
           "    " + cmd, "",
           "| kernel | calls | total (us) | mean (us) | min (us) | max (us) |",
           "|---|---|---|---|---|---|"]
    for n, c, t, a, mn, mx in kernel_stats(path):
        out.append("| %s | %d | %.1f | %.3f | %.3f | %.3f |" %
                   (n, c, t, a, mn, mx))
    out += [""] + _stamp(sources)
    return "\n".join(out)


def traffic_md(fetch, write, kernel, name, calib_bytes, cmd_fetch,
               cmd_write, algorithmic=None, sources="stream") -> str:
    f = counter_means(fetch, "FETCH_SIZE")
    w = counter_means(write, "WRITE_SIZE")
    if COPY_KERNEL not in f or COPY_KERNEL not in w:
        raise RuntimeError("calibration copy kernel not found in the runs")
    ff = calib_bytes / (f[COPY_KERNEL][1] * 1024.0)
    fw = calib_bytes / (w[COPY_KERNEL][1] * 1024.0)
    kf = [v for k, v in f.items() if k.startswith(kernel)]
    kw = [v for k, v in w.items() if k.startswith(kernel)]
    if not kf or not kw:
        raise RuntimeError("kernel %s not found in the runs" % kernel)
    rd = kf[0][1] * 1024.0 * ff
    wr = kw[0][1] * 1024.0 * fw
    out = ["# HBM traffic of %s (%s)" % (kernel, name), "",
           "FETCH_SIZE run:", "", "    " + cmd_fetch, "",
           "WRITE_SIZE run:", "", "    " + cmd_write, "",
           "| counter | copy calibration (KiB/dispatch) | scale | %s "
           "(KiB/dispatch) | dispatches | bytes/launch |" % kernel,
           "|---|---|---|---|---|---|",
           "| FETCH_SIZE | %.1f | %.4f | %.1f | %d | %.0f |" %
           (f[COPY_KERNEL][1], ff, kf[0][1], kf[0][0], rd),
           "| WRITE_SIZE | %.1f | %.4f | %.1f | %d | %.0f |" %
           (w[COPY_KERNEL][1], fw, kw[0][1], kw[0][0], wr), "",
           "The calibration copy moves %d bytes each way per launch; scale = "
           "known bytes / counter bytes." % calib_bytes, ""]
    if algorithmic:
        out.append("Algorithmic bytes per launch: %d (traffic / algorithmic = "
                   "%.3f)" % (algorithmic, (rd + wr) / algorithmic))
        out.append("")
    out += ["traffic_bytes_per_launch[%s]: %.0f" % (name, rd + wr),
            "read_bytes_per_launch[%s]: %.0f" % (name, rd),
            "write_bytes_per_launch[%s]: %.0f" % (name, wr)] + _stamp(sources)
    return "\n".join(out)


# derived ratios shown under the counter table, when their inputs are there
RATIOS = [
    ("L2 hit rate", "TCC_HIT_sum", ("TCC_HIT_sum", "TCC_MISS_sum")),
    ("LDS bank-conflict cycles per LDS-active cycle", "SQ_LDS_BANK_CONFLICT",
     ("SQ_LDS_IDX_ACTIVE",)),
    ("VALU instructions per wave", "SQ_INSTS_VALU", ("SQ_WAVES",)),
    ("LDS instructions per wave", "SQ_INSTS_LDS", ("SQ_WAVES",)),
]


def counters_md(dbs, kernel, cmds, sources="stream") -> str:
    """Mean value per dispatch of every counter recorded for `kernel` in the
    given --pmc runs, plus a few derived ratios."""
    vals = {}
    for db in dbs:
        # a counter may be reported per hardware instance (SE, XCD): sum the
        # instances of each dispatch, then average over dispatches
        rows = _db(db).execute(
            "select counter_name, count(*), avg(total) from (select "
            "dispatch_id, counter_name, sum(counter_value) as total from "
            "pmc_events where name like ? group by dispatch_id, counter_name) "
            "group by counter_name", (kernel + "%",)).fetchall()
        for c, cnt, v in rows:
            vals[c] = (cnt, v)
    if not vals:
        raise RuntimeError("kernel %s not found in the runs" % kernel)
    out = ["# Counters of %s" % kernel, "", "Runs:", ""]
    out += ["    " + c for c in cmds]
    out += ["", "| counter | dispatches | mean per dispatch |", "|---|---|---|"]
    for c in sorted(vals):
        out.append("| %s | %d | %.0f |" % (c, vals[c][0], vals[c][1]))
    out.append("")
    for label, num, den in RATIOS:
        if num in vals and all(d in vals for d in den):
            d = sum(vals[x][1] for x in den)
            if d > 0:
                out.append("* %s: %.3f" % (label, vals[num][1] / d))
    if "SQ_INSTS_VALU" in vals:
        # VALU issue bound: a wave64 fp32 VALU instruction (packed FP32 off)
        # holds a 16-lane SIMD for 4 cycles; 1024 SIMDs at 2.4 GHz
        t = vals["SQ_INSTS_VALU"][1] * 4 / (1024 * 2.4e9)
        out.append("* VALU issue time at 4 cycles per instruction on 1024 SIMDs "
                   "at 2.4 GHz: %.4f ms per dispatch" % (t * 1e3))
    out += [""]
    for c in sorted(vals):
        out.append("counter_mean[%s]: %.0f" % (c, vals[c][1]))
    out += [""] + _stamp(sources)
    return "\n".join(out)


def _dispatch_means(db, like):
    """{counter: mean over dispatches of the per-dispatch sum over hardware
    instances} for the kernels whose full name matches `like`."""
    rows = _db(db).execute(
        "select counter_name, avg(total) from (select dispatch_id, "
        "counter_name, sum(counter_value) as total from pmc_events where "
        "name like ? group by dispatch_id, counter_name) group by counter_name",
        (like,)).fetchall()
    return {c: v for c, v in rows}


def latency_md(dbs, kernels, cmds, cus=256, xccs=8, sources="walk") -> str:
    """Request latencies and requests in flight of several kernels from --pmc
    runs of TCP_TCC_{READ,WRITE}_REQ{,_LATENCY}_sum, TCC_EA0_{RD,WR}REQ{,
    _LEVEL}_sum and GRBM_GUI_ACTIVE.  kernels: (label, SQL LIKE pattern on
    the full kernel name).  Latency per request = latency (or level) sum /
    requests, in cycles; requests in flight = the same sums / elapsed cycles
    (GRBM_GUI_ACTIVE summed over the XCCs / xccs), by Little's law: per
    compute unit for the vector L1 -> L2 requests, chip-wide for the L2 ->
    memory (EA) requests."""
    out = ["# Memory request latency and concurrency", "", "Runs:", ""]
    out += ["    " + c for c in cmds]
    out += ["",
            "| kernel | cycles | L1->L2 read latency | L1->L2 write latency | "
            "L1->L2 reads in flight per CU | writes in flight per CU | "
            "L2->memory read latency | reads in flight (chip) | "
            "L2->memory write latency | writes in flight (chip) |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    keys = []
    for label, like in kernels:
        v = {}
        for db in dbs:
            v.update(_dispatch_means(db, like))
        need = ("GRBM_GUI_ACTIVE", "TCP_TCC_READ_REQ_sum", "TCP_TCC_WRITE_REQ_sum",
                "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_WRITE_REQ_LATENCY_sum",
                "TCC_EA0_RDREQ_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_RDREQ_LEVEL_sum",
                "TCC_EA0_WRREQ_LEVEL_sum")
        if not all(k in v and v[k] for k in need):
            raise RuntimeError("counters of %s missing from the runs" % label)
        cyc = v["GRBM_GUI_ACTIVE"] / xccs
        r = dict(
            cycles=cyc,
            rd_lat=v["TCP_TCC_READ_REQ_LATENCY_sum"] / v["TCP_TCC_READ_REQ_sum"],
            wr_lat=v["TCP_TCC_WRITE_REQ_LATENCY_sum"] / v["TCP_TCC_WRITE_REQ_sum"],
            rd_fl=v["TCP_TCC_READ_REQ_LATENCY_sum"] / cyc / cus,
            wr_fl=v["TCP_TCC_WRITE_REQ_LATENCY_sum"] / cyc / cus,
            ea_rd_lat=v["TCC_EA0_RDREQ_LEVEL_sum"] / v["TCC_EA0_RDREQ_sum"],
            ea_rd_fl=v["TCC_EA0_RDREQ_LEVEL_sum"] / cyc,
            ea_wr_lat=v["TCC_EA0_WRREQ_LEVEL_sum"] / v["TCC_EA0_WRREQ_sum"],
            ea_wr_fl=v["TCC_EA0_WRREQ_LEVEL_sum"] / cyc)
        out.append("| %s | %.0f | %.0f | %.0f | %.1f | %.1f | %.0f | %.0f | %.0f | %.0f |" % (
            label, r["cycles"], r["rd_lat"], r["wr_lat"], r["rd_fl"], r["wr_fl"],
            r["ea_rd_lat"], r["ea_rd_fl"], r["ea_wr_lat"], r["ea_wr_fl"]))
        keys.append((label, r))
    out += ["", "Latencies in cycles per request; cycles: GRBM_GUI_ACTIVE per XCC "
            "per dispatch.", ""]
    for label, r in keys:
        for k in ("rd_lat", "wr_lat", "rd_fl", "wr_fl", "ea_rd_lat", "ea_rd_fl",
                  "ea_wr_lat", "ea_wr_fl"):
            out.append("%s[%s]: %.2f" % (k, label, r[k]))
    out += [""] + _stamp(sources)
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("fetch_db")
    r.add_argument("write_db")
    r.add_argument("--kernel", required=True)
    r.add_argument("--name", required=True)
    r.add_argument("--calib-bytes", type=int, required=True)
    r.add_argument("--algorithmic", type=int, default=None)
    r.add_argument("--cmd-fetch", required=True)
    r.add_argument("--cmd-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", action="append", default=[])
    for sp in (t, r, c):
        sp.add_argument("--sources", default="stream", choices=sorted(SOURCE_SETS))
    a = ap.parse_args(argv)
    if a.mode == "trace":
        sys.stdout.write(trace_md(a.db, a.cmd, a.sources))
    elif a.mode == "counters":
        sys.stdout.write(counters_md(a.dbs, a.kernel, a.cmd, a.sources))
    else:
        sys.stdout.write(traffic_md(a.fetch_db, a.write_db, a.kernel, a.name,
                                    a.calib_bytes, a.cmd_fetch, a.cmd_write,
                                    a.algorithmic, a.sources))


if __name__ == "__main__":
    main()

"""Summaries of rocprofv3 output (rocpd SQLite databases or CSV directories).

    python -m acoustic_wave_propagation_amd.profiling trace DB --cmd "..."
    python -m acoustic_wave_propagation_amd.profiling traffic FETCH_DB WRITE_DB \
        --kernel star2p5d_kernel --name star2p5d_r4_f32 --calib-bytes 1073741824 \
        --cmd-fetch "..." --cmd-write "..."

`trace` prints the per-kernel call count and duration statistics of a
`--kernel-trace --stats` run.  `traffic` turns two `--pmc FETCH_SIZE` /
`--pmc WRITE_SIZE` runs into bytes per launch: each counter (KiB per
dispatch) is scaled by the bytes a plain device copy of known size moved,
divided by what the same counter read for that copy (the copy is the
runtime's copyBuffer kernel that the benchmark's --calib flag launches).
The output also records a hash of the kernel sources, so a consumer can tell
whether the figures still describe the current kernel.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import os
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = [os.path.join(PKG, "csrc", "star2p5d_kernel.h"),
                  os.path.join(PKG, "csrc", "star2p5d.hip")]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _db(path):
    if os.path.isdir(path):
        found = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
        if not found:
            raise FileNotFoundError("no rocpd database under " + path)
        path = found[0]
    return sqlite3.connect(path)


def kernel_stats(path):
    """[(name, calls, total_us, avg_us, min_us, max_us)] by total time."""
    db = _db(path)
    rows = db.execute(
        "select name, count(*), sum(duration), avg(duration), min(duration), "
        "max(duration) from kernels group by name order by sum(duration) desc"
    ).fetchall()
    # durations are in ns
    return [(n, c, t / 1e3, a / 1e3, mn / 1e3, mx / 1e3)
            for n, c, t, a, mn, mx in rows]


def counter_means(path, counter):
    """{kernel name: (dispatches, mean counter value)}."""
    db = _db(path)
    rows = db.execute(
        "select name, count(*), avg(counter_value) from pmc_events where "
        "counter_name = ? group by name", (counter,)).fetchall()
    return {n: (c, v) for n, c, v in rows}


def trace_md(path, cmd) -> str:
    out = ["# Kernel trace summary", "",
           "Command (run from /tmp, repository at $REPO):", "",
           "    " + cmd, "",
           "| kernel | calls | total (us) | mean (us) | min (us) | max (us) |",
           "|---|---|---|---|---|---|"]
    for n, c, t, a, mn, mx in kernel_stats(path):
        out.append("| %s | %d | %.1f | %.3f | %.3f | %.3f |" %
                   (n, c, t, a, mn, mx))
    out += ["", "kernel_source_sha256_16: " + kernel_hash(), ""]
    return "\n".join(out)


def traffic_md(fetch, write, kernel, name, calib_bytes, cmd_fetch,
               cmd_write, algorithmic=None) -> str:
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
    out = ["# HBM traffic of %s" % kernel, "",
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
            "write_bytes_per_launch[%s]: %.0f" % (name, wr),
            "kernel_source_sha256_16: " + kernel_hash(), ""]
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
    a = ap.parse_args(argv)
    if a.mode == "trace":
        sys.stdout.write(trace_md(a.db, a.cmd))
    else:
        sys.stdout.write(traffic_md(a.fetch_db, a.write_db, a.kernel, a.name,
                                    a.calib_bytes, a.cmd_fetch, a.cmd_write,
                                    a.algorithmic))


if __name__ == "__main__":
    main()

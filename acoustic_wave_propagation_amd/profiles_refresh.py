"""Rewrite the rocprofv3 summaries under profiles/ from the raw output of
one profiling session: the databases the commands below write under $RAW.

    python -m acoustic_wave_propagation_amd.profiles_refresh RAW_DIR [OUT_DIR]
    python -m acoustic_wave_propagation_amd.profiles_refresh --commands KEY...

Each summary records the exact command that produced its database; the
commands are run from /tmp with TMPDIR=/tmp, the repository at $REPO and the
raw output directory at $RAW.  Summaries whose databases are missing from
RAW_DIR are skipped (a session may run only some of the commands); they are
written to OUT_DIR (default: profiles/).  --commands prints the commands of
the given keys (or of all), one per line, for a shell to run.
"""
from __future__ import annotations

import os
import sys

from . import profiling as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PRE = "cd /tmp && TMPDIR=/tmp rocprofv3 "
BENCH = " -- python3 $REPO/bench.py "
SQ = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
      "SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES SQ_WAIT_INST_LDS")
CMDS = {
    "trace": PRE + "--kernel-trace --stats -T -d $RAW/prof_trace -o trace"
    + BENCH + "--only-headline --steps 50 --warmup 10",
    "fetch": PRE + "--pmc FETCH_SIZE -T -d $RAW/pmc_fetch -o fetch"
    + BENCH + "--only-headline --calib --steps 5 --warmup 2",
    "write": PRE + "--pmc WRITE_SIZE -T -d $RAW/pmc_write -o write"
    + BENCH + "--only-headline --calib --steps 5 --warmup 2",
    "others": PRE + "--kernel-trace --stats -T -d $RAW/prof_others -o others"
    + BENCH + "--only-others --no-cpu --steps 20 --warmup 5",
    "sq": PRE + "--pmc " + SQ + " -T -d $RAW/pmc_sq -o sq"
    + BENCH + "--only-headline --steps 5 --warmup 2",
    "tcc": PRE + "--pmc TCC_HIT_sum TCC_MISS_sum -T -d $RAW/pmc_tcc -o tcc"
    + BENCH + "--only-headline --steps 5 --warmup 2",
    # full kernel names: the two-step passes with and without data regions
    # differ only in a template argument
    "wave_trace": PRE + "--kernel-trace --stats -d $RAW/prof_wave -o wave"
    + BENCH + "--only-wave all --no-cpu --steps 2",
}
# request latency and concurrency of the apply beside copies that walk
# memory the same way (bench.py --ceilings); full kernel names (no -T), so
# the copies' store variants stay apart
LAT_TCP = ("TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_WRITE_REQ_LATENCY_sum "
           "TCP_TCC_READ_REQ_sum TCP_TCC_WRITE_REQ_sum GRBM_GUI_ACTIVE")
LAT_EA = ("TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_LEVEL_sum "
          "TCC_EA0_WRREQ_sum GRBM_GUI_ACTIVE")
CMDS["lat_tcp"] = (PRE + "--pmc " + LAT_TCP + " -d $RAW/pmc_lat_tcp -o lat"
                   + BENCH + "--ceilings --steps 20 --warmup 2")
CMDS["lat_ea"] = (PRE + "--pmc " + LAT_EA + " -d $RAW/pmc_lat_ea -o lat"
                  + BENCH + "--ceilings --steps 20 --warmup 2")
# the same counters on the single wave step (one launch, eta everywhere)
CMDS["lat_wave_tcp"] = (PRE + "--pmc " + LAT_TCP + " -d $RAW/pmc_lat_wave_tcp -o lat"
                        + BENCH + "--only-wave wave --no-cpu --steps 1")
CMDS["lat_wave_ea"] = (PRE + "--pmc " + LAT_EA + " -d $RAW/pmc_lat_wave_ea -o lat"
                       + BENCH + "--only-wave wave --no-cpu --steps 1")
# the same counters on the two-step passes (plain, with data regions, PML)
CMDS["lat_passes_tcp"] = (PRE + "--pmc " + LAT_TCP + " -d $RAW/pmc_lat_passes_tcp -o lat"
                          + BENCH + "--only-wave all --no-cpu --steps 1")
CMDS["lat_passes_ea"] = (PRE + "--pmc " + LAT_EA + " -d $RAW/pmc_lat_passes_ea -o lat"
                         + BENCH + "--only-wave all --no-cpu --steps 1")
PASS_KERNELS = [
    ("two-step pass (wave2_kernel, 64 x 40 extended tiles)",
     "%wave2_kernel<float, 4, st::Wave2Cfg<4, 1, 16, 40, 3, true, true, 2, true>, false, false>%"),
    ("two-step pass with data regions",
     "%wave2_kernel<float, 4, st::Wave2Cfg<4, 1, 16, 40, 3, true, true, 2, true>, false, true>%"),
    ("two-step PML pass (64 x 32 extended tiles)",
     "%wave2_kernel<float, 4, st::Wave2Cfg<4, 1, 16, 32, 2, true, true, 2, true>, true, false>%"),
]
LAT_KERNELS = [
    ("R=4 apply (star2p5d_kernel, 256 x 16 tiles)", "%star2p5d_kernel<float, 4, false%"),
    ("z-march copy, 256 x 16 tiles", "%zmarch_kernel<64, 8, 0>%"),
    ("z-march copy, 256 x 16 tiles, row-aligned stores", "%zmarch_kernel<64, 8, 1>%"),
    ("z-march copy, 512 x 8 tiles", "%zmarch_kernel<128, 4, 0>%"),
    ("one-shot row copy", "%rows_kernel<0>%"),
    ("one-shot row copy, row-aligned stores", "%rows_kernel<1>%"),
]
for _v in ("wave", "pml", "blocked", "blocked_regions", "pml_blocked"):
    for _c, _n in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        CMDS["%s_%s" % (_v, _n)] = (
            PRE + "--pmc %s -T -d $RAW/pmc_%s_%s -o %s" % (_c, _v, _n, _n)
            + BENCH + "--only-wave %s --calib --no-cpu --steps 1" % _v)
# the two-step pass and the fused Jacobi passes: SQ and L2 counters
CMDS["blocked_sq"] = (PRE + "--pmc " + SQ + " -T -d $RAW/pmc_blocked_sq -o sq"
                      + BENCH + "--only-wave blocked --no-cpu --steps 1")
CMDS["blocked_tcc"] = (PRE + "--pmc TCC_HIT_sum TCC_MISS_sum -T -d $RAW/pmc_blocked_tcc -o tcc"
                       + BENCH + "--only-wave blocked --no-cpu --steps 1")
CMDS["pml_blocked_sq"] = (PRE + "--pmc " + SQ + " -T -d $RAW/pmc_pml_blocked_sq -o sq"
                          + BENCH + "--only-wave pml_blocked --no-cpu --steps 1")
CMDS["pml_blocked_tcc"] = (PRE + "--pmc TCC_HIT_sum TCC_MISS_sum -T -d "
                           "$RAW/pmc_pml_blocked_tcc -o tcc"
                           + BENCH + "--only-wave pml_blocked --no-cpu --steps 1")
CMDS["others_sq"] = (PRE + "--pmc " + SQ + " -T -d $RAW/pmc_others_sq -o sq"
                     + BENCH + "--only-others --no-cpu --steps 2 --warmup 1")
CMDS["others_tcc"] = (PRE + "--pmc TCC_HIT_sum TCC_MISS_sum -T -d $RAW/pmc_others_tcc -o tcc"
                      + BENCH + "--only-others --no-cpu --steps 2 --warmup 1")
# HBM traffic of the fused Jacobi pass and the fp64 ragged apply
for _c, _n in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
    CMDS["others_%s" % _n] = (
        PRE + "--pmc %s -T -d $RAW/pmc_others_%s -o %s" % (_c, _n, _n)
        + BENCH + "--only-others --calib --no-cpu --steps 2 --warmup 1")
HEADLINE_BYTES = 1098907648  # algorithmic bytes of one 512^3 R=4 fp32 apply
WAVE_BYTES = 21575499776     # one 1024^3 R=4 fp32 wave (or PML) step
PASS_BYTES = WAVE_BYTES + 4 * 1024 ** 3  # a two-step pass: one more field written
JACOBI_PASS_BYTES = 1067450400  # a fused R=1 pass over 512^3: one read, one write
F64_BYTES = 2799206128          # one R=4 fp64 apply on 1001 x 603 x 297


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "--commands":
        for k in (argv[1:] or sorted(CMDS)):
            print(CMDS[k])
        return 0
    if len(argv) not in (1, 2):
        print(__doc__, file=sys.stderr)
        return 2
    raw = argv[0]
    prof = argv[1] if len(argv) == 2 else os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)

    class Missing(Exception):
        pass

    def db(d, n):
        path = os.path.join(raw, d, n + "_results.db")
        if not os.path.exists(path):
            raise Missing(path)
        return path

    makers = {
        "star2p5d_r4_512cube_trace.md":
            lambda: P.trace_md(db("prof_trace", "trace"), CMDS["trace"]),
        "star2p5d_r4_512cube_traffic.md":
            lambda: P.traffic_md(db("pmc_fetch", "fetch"), db("pmc_write", "write"),
                         "star2p5d_kernel", "star2p5d_r4_f32", 1 << 30,
                         CMDS["fetch"], CMDS["write"], HEADLINE_BYTES),
        "jacobi_r1_512cube_and_f64_ragged_trace.md":
            lambda: P.trace_md(db("prof_others", "others"), CMDS["others"], "fused"),
        "blocked_r4_1024cube_counters.md":
            lambda: P.counters_md([db("pmc_blocked_sq", "sq"), db("pmc_blocked_tcc", "tcc")],
                          "wave2_kernel", [CMDS["blocked_sq"], CMDS["blocked_tcc"]],
                          "blocked"),
        "pml_blocked_r4_1024cube_counters.md":
            lambda: P.counters_md([db("pmc_pml_blocked_sq", "sq"),
                                   db("pmc_pml_blocked_tcc", "tcc")],
                                  "wave2_kernel", [CMDS["pml_blocked_sq"],
                                                   CMDS["pml_blocked_tcc"]], "blocked"),
        "jacobi_r1_512cube_counters.md":
            lambda: P.counters_md([db("pmc_others_sq", "sq"), db("pmc_others_tcc", "tcc")],
                          "sweeps_fused_kernel", [CMDS["others_sq"], CMDS["others_tcc"]],
                          "fused"),
        "jacobi_r1_512cube_traffic.md":
            lambda: P.traffic_md(db("pmc_others_fetch", "fetch"), db("pmc_others_write", "write"),
                         "sweeps_fused_kernel", "jacobi_r1_f32", 1 << 30,
                         CMDS["others_fetch"], CMDS["others_write"], JACOBI_PASS_BYTES,
                         "fused"),
        "apply_r4_f64_ragged_traffic.md":
            lambda: P.traffic_md(db("pmc_others_fetch", "fetch"), db("pmc_others_write", "write"),
                         "star2p5d_kernel", "apply_r4_f64", 1 << 30,
                         CMDS["others_fetch"], CMDS["others_write"], F64_BYTES),
        "star2p5d_r4_512cube_counters.md":
            lambda: P.counters_md([db("pmc_sq", "sq"), db("pmc_tcc", "tcc")],
                          "star2p5d_kernel", [CMDS["sq"], CMDS["tcc"]]),
        "wave_pml_blocked_r4_1024cube_trace.md":
            lambda: P.trace_md(db("prof_wave", "wave"), CMDS["wave_trace"], "blocked"),
        "wave_r4_1024cube_latency.md":
            lambda: P.latency_md([db("pmc_lat_wave_tcp", "lat"), db("pmc_lat_wave_ea", "lat")],
                                 [("R=4 wave step (star2p5d_kernel, 128 x 32 tiles)",
                                   "%star2p5d_kernel<float, 4, true%")],
                                 [CMDS["lat_wave_tcp"], CMDS["lat_wave_ea"]], sources="stream"),
        "two_step_passes_r4_1024cube_latency.md":
            lambda: P.latency_md([db("pmc_lat_passes_tcp", "lat"),
                                  db("pmc_lat_passes_ea", "lat")],
                                 PASS_KERNELS,
                                 [CMDS["lat_passes_tcp"], CMDS["lat_passes_ea"]],
                                 sources="blocked"),
        "apply_and_walk_copies_r4_512cube_latency.md":
            lambda: P.latency_md([db("pmc_lat_tcp", "lat"), db("pmc_lat_ea", "lat")],
                                 LAT_KERNELS, [CMDS["lat_tcp"], CMDS["lat_ea"]]),
    }
    for v in ("wave", "pml", "blocked", "blocked_regions", "pml_blocked"):
        two = v in ("blocked", "blocked_regions", "pml_blocked")
        makers["%s_r4_1024cube_traffic.md" % v] = (lambda v=v, two=two: P.traffic_md(
            db("pmc_%s_fetch" % v, "fetch"), db("pmc_%s_write" % v, "write"),
            "wave2_kernel" if two else "star2p5d_kernel",
            "%s_r4_f32" % v, 1 << 30, CMDS["%s_fetch" % v],
            CMDS["%s_write" % v], PASS_BYTES if two else WAVE_BYTES,
            "blocked" if two else "stream"))
    for name, make in makers.items():
        try:
            text = make()
        except Missing as e:
            print("skipped %s (no %s)" % (name, e))
            continue
        with open(os.path.join(prof, name), "w") as f:
            f.write(text)
        print("wrote " + os.path.join(prof, name))
    return 0


if __name__ == "__main__":
    sys.exit(main())

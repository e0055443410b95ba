"""Host logic of the measurement (CPU only): the one-GPU guard of bench.py,
the algorithmic-byte formulas the roofline divides by, the staleness check of
recorded HBM traffic, and the counter-to-bytes scaling of the profile
summaries (on a synthetic rocpd database)."""
import importlib.util
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    b = _bench()
    # 512^3 interior, R = 4, fp32: interior + 8-deep face slabs read once,
    # interior written once
    n = 512 ** 3
    faces = 2 * 4 * 3 * 512 * 512
    assert b.star_bytes((512, 512, 512), 4, 4) == 4 * (2 * n + faces) \
        == 1098907648
    # the wave step adds u_prev, vel2, eta reads on the 1024^3 interior
    m = 1024 ** 3
    wave = b.star_bytes((1024,) * 3, 4, 4) + 3 * 4 * m
    assert wave == 21575499776
    # non-cubic: faces are per pair of axes
    assert b.star_bytes((3, 5, 7), 1, 8) == 8 * (2 * 105 + 2 * (35 + 21 + 15))


def test_recorded_traffic_tracks_the_kernel_source(tmp_path):
    b = _bench()
    from acoustic_wave_propagation_amd.profiling import kernel_hash
    good = tmp_path / "t.md"
    good.write_text("traffic_bytes_per_launch[k_r4]: 1234567\n"
                    "read_bytes_per_launch[k_r4]: 1000000\n"
                    "write_bytes_per_launch[k_r4]: 234567\n"
                    "kernel_sources: stream\n"
                    "kernel_source_sha256_16: %s\n" % kernel_hash("stream"))
    assert b.recorded_traffic("k_r4", str(good)) == 1234567.0
    assert b.recorded_traffic("k_r4", str(good), what="read") == 1000000.0
    assert b.recorded_traffic("k_r4", str(good), what="write") == 234567.0
    assert b.recorded_traffic("other", str(good)) is None
    stale = tmp_path / "s.md"
    stale.write_text("traffic_bytes_per_launch[k_r4]: 1234567\n"
                     "kernel_source_sha256_16: 0000000000000000\n")
    assert b.recorded_traffic("k_r4", str(stale)) is None
    assert b.recorded_traffic("k_r4", str(tmp_path / "missing.md")) is None
    # a summary stamped with another source set checks that set's hash
    other = tmp_path / "o.md"
    other.write_text("traffic_bytes_per_launch[k_r4]: 5\n"
                     "kernel_sources: blocked\n"
                     "kernel_source_sha256_16: %s\n" % kernel_hash("blocked"))
    assert b.recorded_traffic("k_r4", str(other)) == 5.0
    assert kernel_hash("blocked") != kernel_hash("stream")


def test_recorded_counters_and_valu_bound(tmp_path):
    """Counter means and the VALU issue bound from a counter summary; stale
    summaries give None."""
    b = _bench()
    from acoustic_wave_propagation_amd.profiling import kernel_hash
    c = tmp_path / "c.md"
    c.write_text("counter_mean[SQ_INSTS_VALU]: 614400000\n"
                 "kernel_sources: stream\n"
                 "kernel_source_sha256_16: %s\n" % kernel_hash("stream"))
    assert b.recorded_counter(str(c), "SQ_INSTS_VALU") == 614400000.0
    assert b.recorded_counter(str(c), "SQ_WAVES") is None
    v = b.valu_roofline(str(c), 2e-3)
    # 614.4e6 instructions x 4 cycles / (1024 SIMDs x 2.4e9 Hz) = 1 ms
    assert abs(v["issue_ms"] - 1.0) < 1e-9 and abs(v["frac"] - 0.5) < 1e-9
    c.write_text("counter_mean[SQ_INSTS_VALU]: 1\n"
                 "kernel_source_sha256_16: 0000000000000000\n")
    assert b.valu_roofline(str(c), 1.0) is None


def test_kernel_hash_ignores_comments():
    from acoustic_wave_propagation_amd.profiling import code_only
    a = "int f(int x) {  // the value\n  return x + 1; /* one\n more */ }\n"
    b = "int f(int x) { return x + 1; }  // other words\n"
    assert code_only(a) == code_only(b) == "int f(int x) { return x + 1; }"
    assert code_only("return x + 2;") != code_only("return x + 1;")


def _pmc_db(path, counter, rows):
    db = sqlite3.connect(path)
    db.execute("create table pmc_events (dispatch_id integer, name text, "
               "counter_name text, counter_value real)")
    db.executemany("insert into pmc_events values (?, ?, ?, ?)",
                   [(i, n, counter, v) for i, (n, v) in enumerate(rows)])
    db.commit()
    db.close()


def test_traffic_scaling(tmp_path):
    """FETCH_SIZE reads half the bytes of the 1 GiB calibration copy, so the
    kernel's fetch counter is scaled by 2; WRITE_SIZE reads them all."""
    from acoustic_wave_propagation_amd import profiling as P
    gib = 1 << 30
    f, w = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _pmc_db(f, "FETCH_SIZE", [(P.COPY_KERNEL, gib / 2 / 1024),
                              ("star2p5d_kernel", 1000.0),
                              ("star2p5d_kernel", 1200.0)])
    _pmc_db(w, "WRITE_SIZE", [(P.COPY_KERNEL, gib / 1024),
                              ("star2p5d_kernel", 500.0)])
    text = P.traffic_md(f, w, "star2p5d_kernel", "k_r4", gib, "cmd f",
                        "cmd w", algorithmic=4000 * 1024)
    lines = dict(l.split(": ", 1) for l in text.splitlines()
                 if l.startswith(("read_", "write_", "traffic_")))
    assert float(lines["read_bytes_per_launch[k_r4]"]) == 2 * 1100 * 1024
    assert float(lines["write_bytes_per_launch[k_r4]"]) == 500 * 1024
    assert float(lines["traffic_bytes_per_launch[k_r4]"]) == 2700 * 1024
    assert "traffic / algorithmic = 0.675" in text
    with pytest.raises(RuntimeError):
        _pmc_db(str(tmp_path / "n.db"), "FETCH_SIZE",
                [("star2p5d_kernel", 1.0)])
        P.traffic_md(str(tmp_path / "n.db"), w, "star2p5d_kernel", "k", gib,
                     "", "")


def test_latency_summary(tmp_path):
    """Request latency = latency (or level) sum / requests; in flight = the
    same sum / elapsed cycles (GRBM_GUI_ACTIVE summed over the XCCs, divided
    by their number), per CU for L1 -> L2.  Counters of one dispatch are
    summed over hardware instances, then averaged over dispatches."""
    from acoustic_wave_propagation_amd import profiling as P
    db = str(tmp_path / "lat.db")
    con = sqlite3.connect(db)
    con.execute("create table pmc_events (dispatch_id integer, name text, "
                "counter_name text, counter_value real)")
    k = "void st::star2p5d_kernel<float, 4, false, X>(st::StarArgs<float>)"
    rows = []
    for disp, scale in ((0, 1.0), (1, 3.0)):   # dispatch means: 2x dispatch 0
        rows += [(disp, k, "GRBM_GUI_ACTIVE", 500.0 * scale),   # two XCCs
                 (disp, k, "GRBM_GUI_ACTIVE", 500.0 * scale),
                 (disp, k, "TCP_TCC_READ_REQ_sum", 100.0 * scale),
                 (disp, k, "TCP_TCC_READ_REQ_LATENCY_sum", 40000.0 * scale),
                 (disp, k, "TCP_TCC_READ_REQ_LATENCY_sum", 10000.0 * scale),
                 (disp, k, "TCP_TCC_WRITE_REQ_sum", 50.0 * scale),
                 (disp, k, "TCP_TCC_WRITE_REQ_LATENCY_sum", 20000.0 * scale),
                 (disp, k, "TCC_EA0_RDREQ_sum", 80.0 * scale),
                 (disp, k, "TCC_EA0_RDREQ_LEVEL_sum", 160000.0 * scale),
                 (disp, k, "TCC_EA0_WRREQ_sum", 40.0 * scale),
                 (disp, k, "TCC_EA0_WRREQ_LEVEL_sum", 20000.0 * scale)]
    rows.append((2, "other_kernel", "GRBM_GUI_ACTIVE", 1e9))
    con.executemany("insert into pmc_events values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    text = P.latency_md([db], [("apply", "%star2p5d_kernel<float, 4, false%")],
                        ["cmd"], cus=2, xccs=2)
    v = dict(l.split(": ", 1) for l in text.splitlines() if "[apply]: " in l)
    # dispatch means: cycles 2000 / 2 XCCs = 1000; reads 200 with latency
    # sum 100000 -> 500 cycles each, 100000 / 1000 / 2 CUs = 50 in flight
    assert float(v["rd_lat[apply]"]) == 500.0
    assert float(v["rd_fl[apply]"]) == 50.0
    assert float(v["wr_lat[apply]"]) == 400.0
    assert float(v["wr_fl[apply]"]) == 20.0
    assert float(v["ea_rd_lat[apply]"]) == 2000.0
    assert float(v["ea_rd_fl[apply]"]) == 320.0
    assert float(v["ea_wr_lat[apply]"]) == 500.0
    assert float(v["ea_wr_fl[apply]"]) == 40.0
    with pytest.raises(RuntimeError):
        P.latency_md([db], [("none", "%nothing%")], ["cmd"])


def test_walk_copy_library_exports():
    """The measurement copies (bench.py --ceilings) are built beside the
    stencil library and export their two entry points."""
    path = os.path.join(ROOT, "acoustic_wave_propagation_amd", "libwalkcopy.so")
    if not os.path.exists(path):
        pytest.skip("libwalkcopy.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert {"walk_copy_zmarch", "walk_copy_rows"} <= names


def test_eta_read_points_model():
    """The data-region byte model: pw = 32 on a 1024^3 interior reads eta on
    the two 32-row y slabs, the 64 z-sponge planes of the other rows, and
    elsewhere 32 columns of each tile (the left 32 of even tiles, the right
    32 of odd ones, which include the x sponges): an eighth of the columns
    on 256-wide tiles, a quarter on the PML step's 128-wide ones."""
    b = _bench()
    n, pw = 1024, 32
    want = 2 * pw * n * n + (n - 2 * pw) * (2 * pw * n + (n - 2 * pw) * (n // 8))
    assert b.eta_read_points((n, n, n), pw) == want
    want = 2 * pw * n * n + (n - 2 * pw) * (2 * pw * n + (n - 2 * pw) * (n // 4))
    assert b.eta_read_points((n, n, n), pw, tile_x=128) == want
    # the two-step pass's 56-wide output tiles: 64 of every 112 columns
    # (nine periods), the last 16 columns (band) and the x faces inside
    # those: 592 columns
    want = 2 * pw * n * n + (n - 2 * pw) * (2 * pw * n + (n - 2 * pw) * 592)
    assert b.eta_read_points((n, n, n), pw, tile_x=56) == want
    # a ragged row of 1000 columns: bands [0, 32) and [480, 544), and the x
    # face rule reads [968, 1000), where the last tile's band would lie past
    # the row: 128 columns
    iz, iy, ix = 100, 100, 1000
    want = 2 * pw * ix * iz + (iy - 2 * pw) * (2 * pw * ix + (iz - 2 * pw) * 128)
    assert b.eta_read_points((iz, iy, ix), pw) == want

"""The time-blocked leapfrog (wave_run_blocked: two wave steps per pass over
HBM) on an MI355X.

Its two-step kernel does, per point and step, the operations of the single
wave step in the same order, so the first bar is bit-identity: every pass
must equal two single steps (wave_step into fresh buffers, then
wave_add_source) bit for bit, and a whole run must equal wave_run's.  The
single step is checked against the CPU oracle elsewhere; the oracle is also
applied here directly (teacher-forced, fp32 max|err| <= 1e-5 max|ref| per
step) on small grids.  u_prev and u share their halo (zero, or a constant),
as the entry point requires; the work buffers start as a sentinel or NaN,
and the call must set their non-interior points from u.
"""
import numpy as np
import pytest

from acoustic_wave_propagation_amd import binding as B
from acoustic_wave_propagation_amd import workloads as wl

from gpu_common import (F32_TOL, SENTINEL, check_close, check_halo_untouched,
                        device, interior, log, upload, upload_planes)

pytestmark = pytest.mark.gpu

R = 4
DT, H = 1e-3, 10.0


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    d = device()
    B.lib()
    return torch, d


def _zero_halo(a, r=R):
    b = np.zeros_like(a)
    b[r:-r, r:-r, r:-r] = a[r:-r, r:-r, r:-r]
    return b


def _fields(shape, seed, eta_hi=0.1, r=R):
    up = _zero_halo(wl.uniform_planes(shape, seed, -1, 1), r)
    uc = _zero_halo(wl.uniform_planes(shape, seed + 1, -1, 1), r)
    v2 = wl.uniform_planes(shape, seed + 2, 1.5e3 ** 2, 4.5e3 ** 2)
    et = wl.uniform_planes(shape, seed + 3, 0.0, eta_hi)
    return up, uc, v2, et


def _sentinel(torch, shape):
    return torch.full(shape, SENTINEL, dtype=torch.float32, device=device())


def _single_steps(torch, d, up, uc, v2, et, nsteps, src, trace):
    """nsteps single steps into fresh zero-halo buffers, each followed by
    its source; returns the list of levels 0..nsteps+1 (device tensors)."""
    lv = [up.clone(), uc.clone()]
    for n in range(nsteps):
        nxt = torch.zeros_like(uc)
        B.wave_step(d, lv[-2], lv[-1], nxt, v2, et, DT, H)
        if trace is not None:
            B.wave_add_source(d, nxt, *src, float(trace[n]))  # rounded to d's type
        lv.append(nxt)
    return lv


def _same_interior(got, want, what, r=R):
    g, w = interior(got, r), interior(want, r)
    bad = int((g != w).sum())
    if bad:
        diff = float((g - w).abs().max())
        raise AssertionError("%s: %d interior points differ (max |diff| %.3e)"
                             % (what, bad, diff))


@pytest.mark.parametrize("r", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [
    (20, 40, 70),      # one tile in x and y (R = 4)
    (45, 61, 139),     # ragged tiles in x and y, one z chunk
    (130, 77, 121),    # several z chunks
    (17, 33, 9 + 56),  # one output column of tiles, thin z
])
def test_one_pass_bit_identical_to_two_steps(torch_dev, shape, r):
    torch, _ = torch_dev
    log("case blocked pass R=%d %s" % (r, shape))
    up, uc, v2, et = (upload(a) for a in _fields(shape, 1100 + shape[0], r=r))
    d = B.desc_init("f32", shape, r)
    nz, ny, nx = shape
    src = (nx // 2, ny // 3, nz // 2)
    trace = [0.25, -0.5]
    w0, w1 = _sentinel(torch, shape), _sentinel(torch, shape)
    old, new = B.wave_run_blocked(d, up.clone(), uc.clone(), w0, w1, v2, et,
                                  DT, H, 2, src, trace)
    assert old.data_ptr() == w0.data_ptr() and new.data_ptr() == w1.data_ptr()
    lv = _single_steps(torch, d, up, uc, v2, et, 2, src, trace)
    torch.cuda.synchronize()
    _same_interior(w0, lv[2], "step 1 of the pass", r)
    _same_interior(w1, lv[3], "step 2 of the pass", r)
    for t, name in ((w0, "work0"), (w1, "work1")):
        check_halo_untouched(t.cpu().numpy(), r, name, value=0.0)


@pytest.mark.parametrize("r", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [(45, 61, 139), (130, 77, 71)])
def test_one_pass_bit_identical_f64(torch_dev, shape, r):
    """The fp64 two-step pass (2 x 1 points per thread, 32 x 40 extended
    tiles) against two fp64 single steps, bit for bit."""
    torch, _ = torch_dev
    log("case blocked pass f64 R=%d %s" % (r, shape))
    up, uc, v2, et = (upload(a.astype(np.float64))
                      for a in _fields(shape, 1700 + shape[0], r=r))
    d = B.desc_init("f64", shape, r)
    nz, ny, nx = shape
    src = (nx // 3, ny // 2, nz // 2)
    trace = [0.25, -0.5]
    w0 = torch.full(shape, SENTINEL, dtype=torch.float64, device=device())
    w1 = torch.full(shape, SENTINEL, dtype=torch.float64, device=device())
    B.wave_run_blocked(d, up.clone(), uc.clone(), w0, w1, v2, et, DT, H, 2,
                       src, trace)
    lv = _single_steps(torch, d, up, uc, v2, et, 2, src, trace)
    torch.cuda.synchronize()
    _same_interior(w0, lv[2], "f64 step 1 of the pass", r)
    _same_interior(w1, lv[3], "f64 step 2 of the pass", r)
    for t, name in ((w0, "work0"), (w1, "work1")):
        check_halo_untouched(t.cpu().numpy(), r, name, value=0.0)


def test_one_pass_matches_the_oracle(oracle_mod, torch_dev):
    """Both steps of a pass against the oracle's wave step, teacher-forced,
    with the sponge-like eta of the real workload replaced by random eta
    (every point differs)."""
    torch, _ = torch_dev
    shape = (37, 53, 131)
    up, uc, v2, et = _fields(shape, 1200)
    d = B.desc_init("f32", shape, R)
    c = list(d.cx[:R + 1])
    nz, ny, nx = shape
    src = (60, 30, 20)
    trace = [0.75, -1.25]
    w0, w1 = _sentinel(torch, shape), _sentinel(torch, shape)
    B.wave_run_blocked(d, upload(up), upload(uc), w0, w1, upload(v2),
                       upload(et), DT, H, 2, src, trace)
    a = w0.cpu().numpy()
    ref1 = oracle_mod.wave_step(up, uc, v2, et, R, c, DT, H)
    ref1[src[2], src[1], src[0]] += np.float32(trace[0])
    check_close(interior(a, R), interior(ref1, R), F32_TOL, "blocked step 1")
    a0 = _zero_halo(a)  # the pass takes level 2's halo to be zero, as u's
    ref2 = oracle_mod.wave_step(uc, a0, v2, et, R, c, DT, H)
    ref2[src[2], src[1], src[0]] += np.float32(trace[1])
    check_close(interior(w1.cpu().numpy(), R), interior(ref2, R), F32_TOL,
                "blocked step 2")
    assert abs(float(interior(a, R)[src[2] - R, src[1] - R, src[0] - R]) -
               float(interior(ref1, R)[src[2] - R, src[1] - R, src[0] - R])) \
        < 1e-4, "source missing in step 1"


@pytest.mark.parametrize("dtype,r,nsteps", [
    ("f32", 4, 0), ("f32", 4, 1), ("f32", 4, 2), ("f32", 4, 3), ("f32", 4, 4),
    ("f32", 4, 5), ("f32", 4, 7), ("f32", 1, 6), ("f32", 3, 5),
    ("f64", 4, 5), ("f64", 2, 4), ("f64", 1, 3), ("f64", 3, 6)])
def test_run_equals_wave_run(torch_dev, dtype, r, nsteps):
    """A whole run, passes plus an odd last single step, against wave_run
    (two buffers, in place): same bits for both returned levels, and the
    levels sit in the buffers the rotation rule names."""
    torch, _ = torch_dev
    shape = (41, 50, 97)
    np_t = np.float32 if dtype == "f32" else np.float64
    up, uc, v2, et = (upload(a.astype(np_t))
                      for a in _fields(shape, 1300 + nsteps, r=r))
    d = B.desc_init(dtype, shape, r)
    src = (40, 20, 17)
    trace = [0.1 * (k + 1) * (-1) ** k for k in range(max(nsteps, 1))]
    bufs = [up.clone(), uc.clone(), torch.zeros_like(uc), torch.zeros_like(uc)]
    old, new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, nsteps, src, trace)
    assert old.data_ptr() == bufs[nsteps % 4].data_ptr()
    assert new.data_ptr() == bufs[(nsteps + 1) % 4].data_ptr()
    a, b = B.wave_run(d, up.clone(), uc.clone(), v2, et, DT, H, nsteps, src,
                      trace)
    torch.cuda.synchronize()
    _same_interior(old, a, "run of %d steps, older level" % nsteps, r)
    _same_interior(new, b, "run of %d steps, newest level" % nsteps, r)


def test_mixed_chunking_and_source_in_the_overlap(torch_dev):
    """More tiles than compute units (groups A and B of the launch), with the
    source on a point that several extended tiles compute (next to a tile
    corner), over two passes."""
    torch, _ = torch_dev
    # 56 x 32 output tiles (R = 4): 10 x 30 = 300 tiles; 200 planes make
    # the mixed plan (256 whole columns, 44 in chunks) the cheaper one
    shape = (208, 8 + 32 * 30, 8 + 56 * 10)
    log("case blocked mixed chunking %s" % (shape,))
    up, uc, v2, et = (upload(a) for a in _fields(shape, 1400))
    d = B.desc_init("f32", shape, R)
    src = (R + 56 * 3, R + 32 * 7 - 1, 13)  # last row of a tile, first column of the next
    trace = [0.5, -0.25, 0.125, 1.0]
    bufs = [up.clone(), uc.clone(), torch.zeros_like(uc), torch.zeros_like(uc)]
    old, new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, 4, src, trace)
    lv = _single_steps(torch, d, up, uc, v2, et, 4, src, trace)
    torch.cuda.synchronize()
    _same_interior(old, lv[4], "mixed chunking, level 4")
    _same_interior(new, lv[5], "mixed chunking, level 5")


def test_no_source_and_pml_width(torch_dev):
    """Without a source trace; with pml_width set, the single steps of
    wave_run and the passes of wave_run_blocked both launch data regions
    (eta read only near the faces): equal."""
    torch, _ = torch_dev
    shape = (60, 70, 90)
    up, uc, v2, _ = _fields(shape, 1500)
    w = np.zeros(shape, np.float32)
    w[R:-R, R:-R, R:-R] = 0.1  # eta zero inside a 10-point shell
    w[R + 10:-R - 10, R + 10:-R - 10, R + 10:-R - 10] = 0.0
    up, uc, v2, et = upload(up), upload(uc), upload(v2), upload(w)
    d = B.desc_init("f32", shape, R)
    d.pml_width = 10
    bufs = [up.clone(), uc.clone(), torch.zeros_like(uc), torch.zeros_like(uc)]
    old, new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, 6)
    a, b = B.wave_run(d, up.clone(), uc.clone(), v2, et, DT, H, 6)
    torch.cuda.synchronize()
    assert torch.equal(interior(old, R), interior(a, R))
    assert torch.equal(interior(new, R), interior(b, R))


def test_blocked_1024_two_steps(torch_dev):
    """The full 1032^3 workload fields (vel2, 32-point sponge, Ricker source
    at the centre) in the launch configuration the benchmark times: one pass
    against two single steps, bit for bit, over the whole interior."""
    torch, _ = torch_dev
    w = wl.WAVE_1024
    e = w.extra
    log("case blocked 1024 %s" % (w.shape,))
    vel2 = upload_planes(lambda a, b: wl.vel2_planes(w, a, b), w.shape,
                         w.np_dtype)
    eta = upload_planes(lambda a, b: wl.eta_planes(w, a, b), w.shape,
                        w.np_dtype)
    # nonzero levels so that every term of the update matters
    up = upload_planes(lambda a, b: _zero_halo_slab(w.shape, 881, a, b),
                       w.shape, w.np_dtype)
    uc = upload_planes(lambda a, b: _zero_halo_slab(w.shape, 882, a, b),
                       w.shape, w.np_dtype)
    d = B.desc_init("f32", w.shape, R)
    src = wl.source_point(w)
    trace = [float(v) for v in wl.source_trace(w)[:2]]
    w0 = torch.zeros_like(uc)
    w1 = torch.zeros_like(uc)
    B.wave_run_blocked(d, up, uc, w0, w1, vel2, eta, e["dt"], e["h"], 2, src,
                       trace)
    # the same pass with data regions (pml_width = the sponge width): the
    # same bits over the whole array
    log("  blocked 1024, pml_width %d" % e["sponge"])
    dp = B.desc_init("f32", w.shape, R)
    dp.pml_width = e["sponge"]
    v0 = torch.zeros_like(uc)
    v1 = torch.zeros_like(uc)
    B.wave_run_blocked(dp, up, uc, v0, v1, vel2, eta, e["dt"], e["h"], 2, src,
                       trace)
    torch.cuda.synchronize()
    assert torch.equal(v0, w0) and torch.equal(v1, w1), "data regions differ"
    del v0, v1
    ref = torch.zeros_like(uc)
    B.wave_step(d, up, uc, ref, vel2, eta, e["dt"], e["h"])
    B.wave_add_source(d, ref, *src, float(np.float32(trace[0])))
    torch.cuda.synchronize()
    _same_interior(w0, ref, "1024 step 1")
    B.wave_step(d, uc, ref, up, vel2, eta, e["dt"], e["h"])  # level 3 over level 0
    B.wave_add_source(d, up, *src, float(np.float32(trace[1])))
    torch.cuda.synchronize()
    _same_interior(w1, up, "1024 step 2")
    del vel2, eta, up, uc, w0, w1, ref
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["f32", "f64"])
@pytest.mark.parametrize("shape,s,widths,false_claim", [
    # ragged in every direction
    ((82, 75, 141), 12, (12, 30), 1),
    # 1000 interior columns: tiles away from the x sponge and their own x
    # edges, whose lanes skip eta away from the z faces
    ((40, 44, 1008), 12, (12, 13), 6),
    # six rows away from the y faces (8); none (11)
    ((46, 30, 90), 8, (8, 11), 3),
])
def test_blocked_data_regions(oracle_mod, torch_dev, dt, shape, s, widths,
                              false_claim):
    """Two-step passes with data regions (R = 4: eta read only where it may
    be nonzero): with eta = 0 at every interior point at least s from all
    interior faces (and random in [0, 0.1] nearer), pml_width s (exact) and
    larger (conservative) give the same bits as 0 over two passes; a false
    claim changes the result, so the skipped loads are really skipped.  The
    result also matches the oracle (four free steps)."""
    torch, _ = torch_dev
    npt = np.float32 if dt == "f32" else np.float64
    up, uc, v2, et = _fields(shape, 1700 + s)
    inner = np.zeros(shape, bool)
    inner[R + s:-R - s, R + s:-R - s, R + s:-R - s] = True
    et[inner] = 0.0
    et = _zero_halo(et)
    host = [a.astype(npt) for a in (up, uc, v2, et)]
    up, uc, v2, et = (upload(a) for a in host)
    runs = {}
    for pw in (0,) + tuple(widths) + (false_claim,):
        log("case blocked data regions %s %s sponge %d pml_width %d"
            % (dt, shape, s, pw))
        d = B.desc_init(dt, shape, R)
        d.pml_width = pw
        bufs = [up.clone(), uc.clone(), torch.zeros_like(uc),
                torch.zeros_like(uc)]
        old, new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, 4)
        runs[pw] = (old.cpu().numpy(), new.cpu().numpy())
    for pw in widths:
        for a, b in zip(runs[pw], runs[0]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), pw
    assert not np.array_equal(runs[false_claim][1], runs[0][1])
    c = oracle_mod.laplacian_weights(R)
    _, ref = oracle_mod.wave_run(*host, R, c, DT, H, 4)
    tol = 1e-4 if dt == "f32" else 1e-11
    check_close(interior(runs[widths[0]][1], R), interior(ref, R), tol,
                "4 free steps, blocked data regions")


def _zero_halo_slab(shape, seed, z0, z1):
    a = wl.uniform_planes(shape, seed, -1, 1, z0, z1)
    nz = shape[0]
    for k in range(z1 - z0):
        if z0 + k < R or z0 + k >= nz - R:
            a[k] = 0
    a[:, :R] = 0
    a[:, -R:] = 0
    a[:, :, :R] = 0
    a[:, :, -R:] = 0
    return a


def test_blocked_run_graph_capture(torch_dev):
    """wave_run_blocked only enqueues kernels (passes, a single step for the
    odd last one, source kernels), so a whole run can be captured into a HIP
    graph: five steps captured once and replayed three times, with eager
    work in between, give the eager result bit for bit every time."""
    torch, _ = torch_dev
    shape = (40, 47, 131)
    up, uc, v2, et = (upload(a) for a in _fields(shape, 1600))
    d = B.desc_init("f32", shape, R)
    src = (50, 20, 19)
    trace = [0.5, -0.25, 0.75, 0.125, -1.0]
    bufs = [torch.zeros_like(uc) for _ in range(4)]

    def work():
        for b in bufs:
            b.zero_()  # a fill kernel, not a memset node
        bufs[0].copy_(up)
        bufs[1].copy_(uc)
        B.wave_run_blocked(d, *bufs, v2, et, DT, H, 5, src, trace)

    work()
    torch.cuda.synchronize()
    eager = [b.cpu().numpy() for b in bufs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for b in bufs:
            b.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [b.cpu().numpy() for b in bufs]
        for a, e in zip(got, eager):
            assert np.array_equal(a.view(np.uint8), e.view(np.uint8)), rep
        # eager work between replays
        B.wave_step(d, up, uc, bufs[2], v2, et, DT, H)
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("r", [1, 2, 3, 4])
def test_smallest_grids(torch_dev, dtype, r):
    """Every extent 2R+1 (one interior point) and a one-plane interior on a
    wider face: runs of 4 steps against wave_run, bit for bit."""
    torch, _ = torch_dev
    np_t = np.float32 if dtype == "f32" else np.float64
    for shape in ((2 * r + 1,) * 3, (2 * r + 1, 2 * r + 9, 2 * r + 70)):
        up, uc, v2, et = (upload(a.astype(np_t))
                          for a in _fields(shape, 1800 + r, r=r))
        d = B.desc_init(dtype, shape, r)
        src = (r, r, r)
        trace = [0.5, -0.25, 0.125, 1.0]
        bufs = [up.clone(), uc.clone(), torch.zeros_like(uc),
                torch.zeros_like(uc)]
        old, new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, 4, src, trace)
        a, b = B.wave_run(d, up.clone(), uc.clone(), v2, et, DT, H, 4, src,
                          trace)
        torch.cuda.synchronize()
        _same_interior(old, a, "%s R=%d %s older" % (dtype, r, shape), r)
        _same_interior(new, b, "%s R=%d %s newest" % (dtype, r, shape), r)


def test_blocked_deterministic_and_side_stream(torch_dev):
    """No atomics: five repeated blocked runs (mixed chunking: more tiles
    than compute units) are bitwise identical, also on a non-default stream."""
    torch, _ = torch_dev
    shape = (120, 8 + 32 * 30, 8 + 56 * 10)
    up, uc, v2, et = (upload(a) for a in _fields(shape, 1900))
    d = B.desc_init("f32", shape, R)
    src, trace = (100, 200, 60), [0.5, -0.25, 0.125, 1.0]
    runs = []
    for k in range(6):
        bufs = [up.clone(), uc.clone(), torch.zeros_like(uc),
                torch.zeros_like(uc)]
        if k < 5:
            B.wave_run_blocked(d, *bufs, v2, et, DT, H, 4, src, trace)
        else:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                B.wave_run_blocked(d, *bufs, v2, et, DT, H, 4, src, trace)
            s.synchronize()
        torch.cuda.synchronize()
        runs.append([b.cpu().numpy() for b in bufs[:2]])
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("nsteps", [3, 4, 5])
def test_uninitialised_work_buffers(torch_dev, dtype, nsteps):
    """work0 and work1 filled with NaN everywhere, as an uninitialised
    workspace may be, and u_prev and u sharing a nonzero halo: the call sets
    the work buffers' non-interior points from u before any pass reads them,
    so from the second pass on (and in the odd last single step) every level
    equals wave_run's bit for bit, no NaN appears, and all four buffers end
    with u's halo."""
    torch, _ = torch_dev
    shape = (43, 52, 101)
    r = R
    np_t = np.float32 if dtype == "f32" else np.float64
    log("case blocked NaN workspace %s %d steps" % (dtype, nsteps))
    halo = 0.25
    fields = _fields(shape, 2000 + nsteps, r=r)
    up, uc = (a.astype(np_t) for a in fields[:2])
    for a in (up, uc):
        m = np.ones(shape, bool)
        m[r:-r, r:-r, r:-r] = False
        a[m] = halo
    up, uc = upload(up), upload(uc)
    v2, et = (upload(a.astype(np_t)) for a in fields[2:])
    d = B.desc_init(dtype, shape, r)
    src = (50, 25, 20)
    trace = [0.2 * (k + 1) * (-1) ** k for k in range(nsteps)]
    nan = float("nan")
    bufs = [up.clone(), uc.clone(), torch.full_like(uc, nan),
            torch.full_like(uc, nan)]
    old, new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, nsteps, src, trace)
    a, b = B.wave_run(d, up.clone(), uc.clone(), v2, et, DT, H, nsteps, src,
                      trace)
    torch.cuda.synchronize()
    _same_interior(old, a, "NaN workspace, %d steps, older level" % nsteps, r)
    _same_interior(new, b, "NaN workspace, %d steps, newest level" % nsteps, r)
    for k, t in enumerate(bufs):
        h = t.cpu().numpy()
        assert not np.isnan(h).any(), "buffer %d holds NaN" % k
        check_halo_untouched(h, r, "buffer %d" % k, value=halo)

"""The time-blocked run of the PML kernel's step (wave_run_pml_blocked: two
wave_step_pml steps per pass over HBM, eta's 7-point coupling in both) on an
MI355X.

The pass does, per point and step, the operations of the single PML step in
the same order, so the first bar is bit-identity with wave_step_pml steps
(into fresh buffers, then wave_add_source), for every radius and both
element types, on ragged grids and on the full 1032^3 fields; the oracle's
PML step is also applied directly, teacher-forced, at the per-step bar
(fp32 max|err| <= 1e-5 max|ref|).  eta is random everywhere, so the coupling
term is nonzero at every point.
"""
import numpy as np
import pytest

from acoustic_wave_propagation_amd import binding as B
from acoustic_wave_propagation_amd import workloads as wl

from gpu_common import (F32_TOL, check_close, check_halo_untouched, device,
                        interior, log, upload, upload_planes)

pytestmark = pytest.mark.gpu

DT, H = 1e-3, 10.0


def _zero_halo(a, r):
    b = np.zeros_like(a)
    b[r:-r, r:-r, r:-r] = a[r:-r, r:-r, r:-r]
    return b


def _fields(shape, seed, r, np_t=np.float32):
    up = _zero_halo(wl.uniform_planes(shape, seed, -1, 1), r).astype(np_t)
    uc = _zero_halo(wl.uniform_planes(shape, seed + 1, -1, 1), r).astype(np_t)
    v2 = wl.uniform_planes(shape, seed + 2, 1.5e3 ** 2, 4.5e3 ** 2).astype(np_t)
    # eta nonzero in the halo too: the coupling reads it there
    et = wl.uniform_planes(shape, seed + 3, 0.0, 0.1).astype(np_t)
    return up, uc, v2, et


def _single_pml_steps(torch, d, up, uc, v2, et, nsteps, src, trace):
    lv = [up.clone(), uc.clone()]
    for n in range(nsteps):
        nxt = torch.zeros_like(uc)
        B.wave_step_pml(d, lv[-2], lv[-1], nxt, v2, et, DT, H)
        if trace is not None:
            B.wave_add_source(d, nxt, *src, float(trace[n]))
        lv.append(nxt)
    return lv


def _same_interior(got, want, what, r):
    g, w = interior(got, r), interior(want, r)
    bad = int((g != w).sum())
    if bad:
        diff = float((g - w).abs().max())
        raise AssertionError("%s: %d interior points differ (max |diff| %.3e)"
                             % (what, bad, diff))


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    d = device()
    B.lib()
    return torch, d


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("r", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", [
    (20, 40, 70),      # one tile in x and y
    (45, 61, 139),     # ragged tiles in x and y
    (130, 77, 121),    # several z chunks
])
def test_pml_pass_bit_identical_to_two_pml_steps(torch_dev, shape, r, dtype):
    torch, _ = torch_dev
    np_t = np.float32 if dtype == "f32" else np.float64
    log("case pml blocked pass %s R=%d %s" % (dtype, r, shape))
    up, uc, v2, et = (upload(a) for a in _fields(shape, 3100 + shape[0], r,
                                                  np_t))
    d = B.desc_init(dtype, shape, r)
    nz, ny, nx = shape
    src = (nx // 2, ny // 3, nz // 2)
    trace = [0.25, -0.5]
    nan = float("nan")
    w0, w1 = torch.full_like(uc, nan), torch.full_like(uc, nan)
    old, new = B.wave_run_pml_blocked(d, up.clone(), uc.clone(), w0, w1, v2,
                                      et, DT, H, 2, src, trace)
    assert old.data_ptr() == w0.data_ptr() and new.data_ptr() == w1.data_ptr()
    lv = _single_pml_steps(torch, d, up, uc, v2, et, 2, src, trace)
    torch.cuda.synchronize()
    _same_interior(w0, lv[2], "step 1 of the PML pass", r)
    _same_interior(w1, lv[3], "step 2 of the PML pass", r)
    for t, name in ((w0, "work0"), (w1, "work1")):
        check_halo_untouched(t.cpu().numpy(), r, name, value=0.0)


def test_pml_pass_matches_the_oracle(oracle_mod, torch_dev):
    """Both steps of a PML pass against the oracle's PML step, teacher-forced,
    at the per-step bar."""
    torch, _ = torch_dev
    r = 4
    shape = (37, 53, 131)
    up, uc, v2, et = _fields(shape, 3200, r)
    d = B.desc_init("f32", shape, r)
    c = list(d.cx[:r + 1])
    src = (60, 30, 20)
    trace = [0.75, -1.25]
    w0 = torch.zeros(shape, dtype=torch.float32, device=device())
    w1 = torch.zeros_like(w0)
    B.wave_run_pml_blocked(d, upload(up), upload(uc), w0, w1, upload(v2),
                           upload(et), DT, H, 2, src, trace)
    a = w0.cpu().numpy()
    ref1 = oracle_mod.wave_step_pml(up, uc, v2, et, r, c, DT, H)
    ref1[src[2], src[1], src[0]] += np.float32(trace[0])
    check_close(interior(a, r), interior(ref1, r), F32_TOL, "PML pass step 1")
    ref2 = oracle_mod.wave_step_pml(uc, _zero_halo(a, r), v2, et, r, c, DT, H)
    ref2[src[2], src[1], src[0]] += np.float32(trace[1])
    check_close(interior(w1.cpu().numpy(), r), interior(ref2, r), F32_TOL,
                "PML pass step 2")


@pytest.mark.parametrize("dtype,r,nsteps", [
    ("f32", 4, 0), ("f32", 4, 1), ("f32", 4, 3), ("f32", 4, 4), ("f32", 4, 5),
    ("f32", 4, 7), ("f32", 1, 6), ("f32", 2, 5), ("f64", 4, 5), ("f64", 3, 4)])
def test_pml_run_equals_wave_run_pml(torch_dev, dtype, r, nsteps):
    """A whole run (passes plus an odd last single PML step) against
    wave_run_pml: same bits for both returned levels, in the buffers the
    rotation rule names; the work buffers start as NaN."""
    torch, _ = torch_dev
    shape = (41, 50, 97)
    np_t = np.float32 if dtype == "f32" else np.float64
    up, uc, v2, et = (upload(a) for a in _fields(shape, 3300 + nsteps, r, np_t))
    d = B.desc_init(dtype, shape, r)
    src = (40, 20, 17)
    trace = [0.1 * (k + 1) * (-1) ** k for k in range(max(nsteps, 1))]
    nan = float("nan")
    bufs = [up.clone(), uc.clone(), torch.full_like(uc, nan),
            torch.full_like(uc, nan)]
    old, new = B.wave_run_pml_blocked(d, *bufs, v2, et, DT, H, nsteps, src,
                                      trace)
    assert old.data_ptr() == bufs[nsteps % 4].data_ptr()
    assert new.data_ptr() == bufs[(nsteps + 1) % 4].data_ptr()
    a, b = B.wave_run_pml(d, up.clone(), uc.clone(), v2, et, DT, H, nsteps,
                          src, trace)
    torch.cuda.synchronize()
    _same_interior(old, a, "PML run of %d steps, older level" % nsteps, r)
    _same_interior(new, b, "PML run of %d steps, newest level" % nsteps, r)


def test_pml_pass_mixed_chunking(torch_dev):
    """More output tiles than compute units (56 x 24 tiles: 10 x 40 = 400),
    over two passes, with the source next to a tile corner."""
    torch, _ = torch_dev
    r = 4
    shape = (208, 8 + 24 * 40, 8 + 56 * 10)
    log("case pml blocked mixed chunking %s" % (shape,))
    up, uc, v2, et = (upload(a) for a in _fields(shape, 3400, r))
    d = B.desc_init("f32", shape, r)
    src = (r + 56 * 3, r + 24 * 7 - 1, 13)
    trace = [0.5, -0.25, 0.125, 1.0]
    bufs = [up.clone(), uc.clone(), torch.zeros_like(uc), torch.zeros_like(uc)]
    old, new = B.wave_run_pml_blocked(d, *bufs, v2, et, DT, H, 4, src, trace)
    lv = _single_pml_steps(torch, d, up, uc, v2, et, 4, src, trace)
    torch.cuda.synchronize()
    _same_interior(old, lv[4], "PML mixed chunking, level 4", r)
    _same_interior(new, lv[5], "PML mixed chunking, level 5", r)


def test_pml_blocked_1024_two_steps(torch_dev):
    """The full 1032^3 workload fields (vel2, the 32-point sponge as eta,
    Ricker source at the centre) with nonzero levels: one PML pass against
    two single PML steps, bit for bit, over the whole interior."""
    torch, _ = torch_dev
    w = wl.WAVE_1024
    e = w.extra
    r = w.radius
    log("case pml blocked 1024 %s" % (w.shape,))
    vel2 = upload_planes(lambda a, b: wl.vel2_planes(w, a, b), w.shape,
                         w.np_dtype)
    eta = upload_planes(lambda a, b: wl.eta_planes(w, a, b), w.shape,
                        w.np_dtype)

    def zh(seed, z0, z1):
        a = wl.uniform_planes(w.shape, seed, -1, 1, z0, z1)
        nz = w.shape[0]
        for k in range(z1 - z0):
            if z0 + k < r or z0 + k >= nz - r:
                a[k] = 0
        a[:, :r] = 0
        a[:, -r:] = 0
        a[:, :, :r] = 0
        a[:, :, -r:] = 0
        return a

    up = upload_planes(lambda a, b: zh(981, a, b), w.shape, w.np_dtype)
    uc = upload_planes(lambda a, b: zh(982, a, b), w.shape, w.np_dtype)
    d = B.desc_init("f32", w.shape, r)
    src = wl.source_point(w)
    trace = [float(v) for v in wl.source_trace(w)[:2]]
    w0 = torch.empty_like(uc)
    w1 = torch.empty_like(uc)
    B.wave_run_pml_blocked(d, up, uc, w0, w1, vel2, eta, e["dt"], e["h"], 2,
                           src, trace)
    ref = torch.zeros_like(uc)
    B.wave_step_pml(d, up, uc, ref, vel2, eta, e["dt"], e["h"])
    B.wave_add_source(d, ref, *src, float(np.float32(trace[0])))
    torch.cuda.synchronize()
    _same_interior(w0, ref, "PML 1024 step 1", r)
    B.wave_step_pml(d, uc, ref, up, vel2, eta, e["dt"], e["h"])
    B.wave_add_source(d, up, *src, float(np.float32(trace[1])))
    torch.cuda.synchronize()
    _same_interior(w1, up, "PML 1024 step 2", r)
    del vel2, eta, up, uc, w0, w1, ref
    torch.cuda.empty_cache()

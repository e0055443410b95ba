"""Parity of the PML step (wave_step_pml / wave_run_pml: the wave update
with the eta-gradient coupling, eta's 7-point stencil of halo 1) with the
CPU oracle on an MI355X.

Same bar as the other parity tests: fp32 max|err| <= 1e-5 max|ref| per step
(teacher-forced), fp64 <= 1e-12 max|ref|; non-interior points keep their
sentinel bits.  Eta is drawn at random per point in most cases, so its
gradient is large everywhere and every neighbour index of the coupling
matters; each case also checks that the coupling moves the result far
beyond the tolerance (a kernel without it would fail).
"""
import dataclasses

import numpy as np
import pytest

from acoustic_wave_propagation_amd import binding as B
from acoustic_wave_propagation_amd import workloads as wl

from gpu_common import (F32_TOL, F64_TOL, SENTINEL, check_close,
                        check_halo_untouched, device, interior, log, rel_err,
                        sentinel_like, upload, upload_planes)

pytestmark = pytest.mark.gpu

DT, H = 1e-3, 10.0


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    d = device()
    B.lib()
    return torch, d


def _tol(dtype):
    return F32_TOL if np.dtype(dtype) == np.float32 else F64_TOL


def _name(dtype):
    return "f32" if np.dtype(dtype) == np.float32 else "f64"


def _fields(shape, seed, dtype):
    up = wl.uniform_planes(shape, seed, -1, 1, dtype=dtype)
    uc = wl.uniform_planes(shape, seed + 1, -1, 1, dtype=dtype)
    v2 = wl.uniform_planes(shape, seed + 2, 1.5e3 ** 2, 4.5e3 ** 2,
                           dtype=dtype)
    et = wl.uniform_planes(shape, seed + 3, 0.0, 0.1, dtype=dtype)
    return up, uc, v2, et


def _step_case(oracle_mod, R, dtype, shape, seed, what):
    up, uc, v2, et = _fields(shape, seed, dtype)
    d = B.desc_init(_name(dtype), shape, R)
    c = list(d.cx[:R + 1])
    out = sentinel_like(shape, dtype)
    B.wave_step_pml(d, upload(up), upload(uc), out, upload(v2), upload(et),
                    DT, H)
    got = out.cpu().numpy()
    ref = oracle_mod.wave_step_pml(up, uc, v2, et, R, c, DT, H)
    check_close(interior(got, R), interior(ref, R), _tol(dtype), what)
    check_halo_untouched(got, R, what)
    plain = oracle_mod.wave_step(up, uc, v2, et, R, c, DT, H)
    share = rel_err(interior(plain, R), interior(ref, R))
    assert share > 100 * _tol(dtype), "%s: coupling share %.1e" % (what, share)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_pml_step_radii(oracle_mod, torch_dev, R, dtype):
    """Ragged tiles in x and y (139 and 41 interior points), every radius."""
    shape = (23 + 2 * R, 41 + 2 * R, 139 + 2 * R)
    log("case pml step R=%d %s %s" % (R, _name(dtype), shape))
    _step_case(oracle_mod, R, dtype, shape, 700 + R, "pml R=%d %s" %
               (R, _name(dtype)))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_pml_step_many_chunks(oracle_mod, torch_dev, dtype):
    """Few tiles and a tall grid: the z axis is cut into several chunks, so
    eta's z neighbours at chunk ends come from the next chunk's planes."""
    R = 4
    shape = (233, 40, 70)
    log("case pml chunks %s %s" % (_name(dtype), shape))
    _step_case(oracle_mod, R, dtype, shape, 720, "pml chunks %s" %
               _name(dtype))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_pml_step_smallest_and_narrow(oracle_mod, torch_dev, dtype):
    """One interior point; one interior plane; an interior 30 points wide
    (narrow tiles at R = 4) and one 33 wide (primary tiles, ragged)."""
    for R, shape in [(1, (3, 3, 3)), (4, (9, 9, 9)), (4, (9, 14, 40)),
                     (2, (13, 11, 5)), (4, (30, 50, 38)), (4, (30, 50, 41))]:
        log("case pml small R=%d %s %s" % (R, _name(dtype), shape))
        up, uc, v2, et = _fields(shape, 730, dtype)
        d = B.desc_init(_name(dtype), shape, R)
        out = sentinel_like(shape, dtype)
        B.wave_step_pml(d, upload(up), upload(uc), out, upload(v2),
                        upload(et), DT, H)
        got = out.cpu().numpy()
        ref = oracle_mod.wave_step_pml(up, uc, v2, et, R, list(d.cx[:R + 1]),
                                       DT, H)
        check_close(interior(got, R), interior(ref, R), _tol(dtype),
                    "pml small %s" % (shape,))
        check_halo_untouched(got, R, "pml small")


def test_pml_step_in_place_and_side_stream(oracle_mod, torch_dev):
    """u_next may be u_prev (each point reads u_prev only at itself); the
    result is the same bits as into a separate buffer, also on a
    non-default stream."""
    torch, _ = torch_dev
    R, dtype = 4, np.float32
    shape = (40, 60, 150)
    up, uc, v2, et = _fields(shape, 740, dtype)
    d = B.desc_init("f32", shape, R)
    t_u, t_v, t_e = upload(uc), upload(v2), upload(et)
    sep = sentinel_like(shape, dtype)
    B.wave_step_pml(d, upload(up), t_u, sep, t_v, t_e, DT, H)
    inplace = upload(up)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        B.wave_step_pml(d, inplace, t_u, inplace, t_v, t_e, DT, H)
    s.synchronize()
    a, b = sep.cpu().numpy(), inplace.cpu().numpy()
    assert np.array_equal(interior(a, R).view(np.uint8),
                          interior(b, R).view(np.uint8))
    # the in-place buffer's halo keeps u_prev's values
    mask = np.ones(shape, bool)
    mask[R:-R, R:-R, R:-R] = False
    assert np.array_equal(b[mask], up[mask])


def _wave_fields(w):
    vel2 = upload_planes(lambda a, b: wl.vel2_planes(w, a, b), w.shape,
                         w.np_dtype)
    eta = upload_planes(lambda a, b: wl.eta_planes(w, a, b), w.shape,
                        w.np_dtype)
    u_prev = upload_planes(lambda a, b: wl.initial_u_planes(w, "u_prev", a, b),
                           w.shape, w.np_dtype)
    u = upload_planes(lambda a, b: wl.initial_u_planes(w, "u", a, b),
                      w.shape, w.np_dtype)
    return u_prev, u, vel2, eta


def test_pml_sponge_steps_teacher_forced(oracle_mod, torch_dev):
    """The 128^3 random-field case with the 32-point sponge: 4 steps, each
    checked against the oracle's step from the GPU's previous state."""
    w = wl.WAVE_128_RANDOM
    e, R = w.extra, w.radius
    u_prev, u, vel2, eta = _wave_fields(w)
    v2n, etn = vel2.cpu().numpy(), eta.cpu().numpy()
    d = B.desc_init("f32", w.shape, R)
    c = list(d.cx[:R + 1])
    a, b = u_prev, u
    for n in range(4):
        an, bn = a.cpu().numpy(), b.cpu().numpy()
        B.wave_step_pml(d, a, b, a, vel2, eta, e["dt"], e["h"])
        ref = oracle_mod.wave_step_pml(an, bn, v2n, etn, R, c, e["dt"], e["h"])
        check_close(interior(a.cpu().numpy(), R), interior(ref, R), F32_TOL,
                    "pml sponge step %d" % n)
        a, b = b, a


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_pml_data_regions_and_run(oracle_mod, torch_dev, dtype):
    """wave_run_pml on a ragged grid with a 12-point sponge: pml_width 12
    (exact) and 30 (conservative) read eta only near the faces and give the
    same bits as 0; at 40 the y slabs would overlap (one launch, eta still
    read only near the faces); 1 is a false claim and changes the result.
    Three free steps against the oracle's loop."""
    dt = _name(dtype)
    base = wl.WAVE_128_RANDOM
    w = dataclasses.replace(base, shape=(82, 75, 141), dtype=dt,
                            extra=dict(base.extra, sponge=12))
    e, R = w.extra, w.radius
    u_prev, u, vel2, eta = _wave_fields(w)
    runs = {}
    for pml in (0, 12, 30, 40, 1):
        log("case pml data regions %s pml_width=%d" % (dt, pml))
        d = B.desc_init(dt, w.shape, R)
        d.pml_width = pml
        older, newest = B.wave_run(d, u_prev.clone(), u.clone(), vel2, eta,
                                   e["dt"], e["h"], 3, pml=True)
        runs[pml] = newest.cpu().numpy()
    for pml in (12, 30, 40):
        assert np.array_equal(runs[pml].view(np.uint8),
                              runs[0].view(np.uint8)), pml
    assert not np.array_equal(runs[1], runs[0])
    c = oracle_mod.laplacian_weights(R)
    args = (u_prev.cpu().numpy(), u.cpu().numpy(), vel2.cpu().numpy(),
            eta.cpu().numpy(), R, c, e["dt"], e["h"], 3)
    _, ref = oracle_mod.wave_run(*args, pml=True)
    tol = 1e-4 if dtype == np.float32 else 1e-11
    check_close(interior(runs[12], R), interior(ref, R), tol,
                "3 free PML steps, data regions")
    # the sponge's coupling is visible after three steps
    _, plain = oracle_mod.wave_run(*args)
    assert rel_err(interior(plain, R), interior(ref, R)) > 5 * tol


def test_pml_run_source_and_roles(oracle_mod, torch_dev):
    """wave_run_pml with a point source: the newest field is in u for an
    even step count, else in u_prev, and matches the oracle's loop."""
    R = 4
    shape = (40, 44, 48)
    up, uc, v2, et = _fields(shape, 750, np.float64)
    d = B.desc_init("f64", shape, R)
    trace = [0.5, -0.25, 0.125]
    src = (20, 22, 24)
    c = list(d.cx[:R + 1])
    for n in (0, 1, 3):
        a, b = upload(up), upload(uc)
        older, newest = B.wave_run(d, a, b, upload(v2), upload(et), DT, H, n,
                                   src=src, src_trace=trace, pml=True)
        assert newest is (b if n % 2 == 0 else a)
        ro, rn = oracle_mod.wave_run(up, uc, v2, et, R, c, DT, H, n,
                                     src=src, src_trace=trace, pml=True)
        check_close(newest.cpu().numpy(), rn, 1e-11, "pml run n=%d" % n)
        check_close(older.cpu().numpy(), ro, 1e-11, "pml run older n=%d" % n)


def test_huge_pml_width_is_one_launch(oracle_mod, torch_dev):
    """A sponge width beyond every extent (up to INT64_MAX) cannot split the
    interior: the single launch, same bits as pml_width = 0, both steps."""
    R, dtype = 4, np.float32
    shape = (30, 31, 70)
    up, uc, v2, et = _fields(shape, 760, dtype)
    t = [upload(a) for a in (up, uc, v2, et)]
    for step in (B.wave_step, B.wave_step_pml):
        outs = []
        for pw in (0, 1 << 30, 1 << 62, (1 << 63) - 1):
            d = B.desc_init("f32", shape, R)
            d.pml_width = pw
            out = sentinel_like(shape, dtype)
            step(d, t[0], t[1], out, t[2], t[3], DT, H)
            outs.append(out.cpu().numpy())
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8))


def test_pml_1024_sampled_slabs(oracle_mod, torch_dev):
    """One PML step on the full 1032^3 fields in the launch configuration the
    benchmark times (random u_prev, u; the workload's vel2 and 32-point
    sponge), checked against the oracle on three 12-plane slabs: the bottom
    of the sponge, the middle and the top."""
    torch, _ = torch_dev
    w = wl.WAVE_1024
    e, R = w.extra, w.radius
    nz = w.shape[0]
    log("case pml 1024 slabs %s" % (w.shape,))
    vel2 = upload_planes(lambda a, b: wl.vel2_planes(w, a, b), w.shape,
                         w.np_dtype)
    eta = upload_planes(lambda a, b: wl.eta_planes(w, a, b), w.shape,
                        w.np_dtype)
    up = upload_planes(lambda a, b: wl.uniform_planes(w.shape, 771, -1, 1, a, b),
                       w.shape, w.np_dtype)
    uc = upload_planes(lambda a, b: wl.uniform_planes(w.shape, 772, -1, 1, a, b),
                       w.shape, w.np_dtype)
    out = sentinel_like(w.shape, w.np_dtype)
    d = B.desc_init("f32", w.shape, R)
    c = list(d.cx[:R + 1])
    B.wave_step_pml(d, up, uc, out, vel2, eta, e["dt"], e["h"])
    torch.cuda.synchronize()
    for z0 in (R, nz // 2 - 6, nz - R - 12):
        z1 = z0 + 12
        sl = slice(z0 - R, z1 + R)
        sub = [t[sl].cpu().numpy() for t in (up, uc, vel2, eta)]
        ref = oracle_mod.wave_step_pml(*sub, R, c, e["dt"], e["h"])
        got = out[z0:z1].cpu().numpy()
        check_close(got[:, R:-R, R:-R], ref[R:-R, R:-R, R:-R], F32_TOL,
                    "pml 1024 slab z %d..%d" % (z0, z1))
        s = np.float32(SENTINEL)
        assert (np.all(got[:, :R] == s) and np.all(got[:, -R:] == s) and
                np.all(got[:, :, :R] == s) and np.all(got[:, :, -R:] == s)), \
            "pml 1024 slab: y or x halo written"
    del vel2, eta, up, uc, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_anisotropic_weights_wave_and_pml(oracle_mod, torch_dev, dtype):
    """Per-axis weights from the descriptor in the wave and PML steps (each
    axis scaled by dt^2/h^2 on its own), against the oracle's anisotropic
    stencil."""
    R = 4
    shape = (30, 41, 77)
    up, uc, v2, et = _fields(shape, 780, dtype)
    d = B.desc_init(_name(dtype), shape, R)
    w = np.random.default_rng(781).uniform(-1, 1, (3, R + 1))
    for k in range(R + 1):
        d.cx[k], d.cy[k], d.cz[k] = w[0, k], w[1, k], w[2, k]
    t = [upload(a) for a in (up, uc, v2, et)]
    for step, ref_fn in ((B.wave_step, oracle_mod.wave_step),
                         (B.wave_step_pml, oracle_mod.wave_step_pml)):
        out = sentinel_like(shape, dtype)
        step(d, t[0], t[1], out, t[2], t[3], DT, H)
        got = out.cpu().numpy()
        ref = ref_fn(up, uc, v2, et, R, w[0], DT, H, cy=w[1], cz=w[2])
        check_close(interior(got, R), interior(ref, R), _tol(dtype),
                    "anisotropic %s %s" % (step.__name__, _name(dtype)))
        check_halo_untouched(got, R, "anisotropic")

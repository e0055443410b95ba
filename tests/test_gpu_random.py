"""Seeded random sweep of small cases through the C ABI, each checked
against the CPU oracle: shapes drawn around the tile sizes (so ragged tiles,
single-tile and sub-tile grids all occur), every radius, both element types,
both boundary modes, random anisotropic weights; wave steps on random fields;
Jacobi runs of random length compared bit for bit with one apply per sweep.
The case list is fixed by the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest

from acoustic_wave_propagation_amd import binding as B
from acoustic_wave_propagation_amd import workloads as wl

from gpu_common import (F32_TOL, F64_TOL, check_close, check_halo_untouched,
                        device, interior, log, sentinel_like, upload)

pytestmark = pytest.mark.gpu

# x extents near multiples of the x tile widths (32, 64, 128, 256, 512)
_X_NEAR = [1, 3, 31, 33, 63, 65, 127, 129, 255, 257, 300, 449, 511, 513]


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        R = int(rng.integers(1, 5))
        dtype = np.float32 if rng.random() < 0.6 else np.float64
        ix = int(rng.choice(_X_NEAR)) if rng.random() < 0.5 else \
            int(rng.integers(1, 200))
        iy = int(rng.integers(1, 70))
        iz = int(rng.integers(1, 40))
        # keep the oracle's work small
        while ix * iy * iz > 600_000:
            iz = max(1, iz // 2)
            iy = max(1, iy - 10)
        shape = (iz + 2 * R, iy + 2 * R, ix + 2 * R)
        boundary = B.DIRICHLET_COPY if rng.random() < 0.3 else \
            B.HALO_UNTOUCHED
        aniso = rng.random() < 0.4
        wseed = int(rng.integers(1 << 30))
        cases.append((i, R, dtype, shape, boundary, aniso, wseed))
    return cases


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    d = device()
    B.lib()
    return torch, d


def _tol(dtype):
    return F32_TOL if np.dtype(dtype) == np.float32 else F64_TOL


@pytest.mark.parametrize("case", _draw_cases(40, 20261202),
                         ids=lambda c: "case%d" % c[0])
def test_random_apply(oracle_mod, torch_dev, case):
    i, R, dtype, shape, boundary, aniso, wseed = case
    name = np.dtype(dtype).name
    log("case %d: apply R=%d %s shape %s boundary %d aniso %s" %
        (i, R, name, shape, boundary, aniso))
    u = wl.uniform_planes(shape, 3000 + i, -1, 1, dtype=dtype)
    d = B.desc_init("f32" if dtype == np.float32 else "f64", shape, R,
                    boundary)
    if aniso:
        w = np.random.default_rng(wseed).uniform(-1, 1, (3, R + 1))
        for k in range(R + 1):
            d.cx[k], d.cy[k], d.cz[k] = w[0, k], w[1, k], w[2, k]
    cx, cy, cz = (list(v[:R + 1]) for v in (d.cx, d.cy, d.cz))
    inp = upload(u)
    out = sentinel_like(shape, dtype)
    B.stencil3d_apply(d, inp, out)
    got = out.cpu().numpy()
    ref = oracle_mod.star_apply(u, R, cx, cy, cz, boundary)
    check_close(interior(got, R), interior(ref, R), _tol(dtype),
                "random apply case %d" % i)
    if boundary == B.HALO_UNTOUCHED:
        check_halo_untouched(got, R, "random apply case %d" % i)
    else:
        mask = np.ones(shape, bool)
        mask[R:-R, R:-R, R:-R] = False
        assert np.array_equal(got[mask], u[mask]), "boundary copy, case %d" % i


@pytest.mark.parametrize("case", _draw_cases(12, 777),
                         ids=lambda c: "case%d" % c[0])
def test_random_wave_step(oracle_mod, torch_dev, case):
    i, R, dtype, shape, _, _, wseed = case
    torch, _ = torch_dev
    name = np.dtype(dtype).name
    log("case %d: wave step R=%d %s shape %s" % (i, R, name, shape))
    g = np.random.default_rng(wseed)
    up = g.uniform(-1, 1, shape).astype(dtype)
    uu = g.uniform(-1, 1, shape).astype(dtype)
    v2 = g.uniform(1.5e3 ** 2, 4.5e3 ** 2, shape).astype(dtype)
    et = g.uniform(0.0, 0.1, shape).astype(dtype)
    dt_, h = 1e-3, 10.0
    d = B.desc_init("f32" if dtype == np.float32 else "f64", shape, R)
    c = list(d.cx[:R + 1])
    nxt = sentinel_like(shape, dtype)
    B.wave_step(d, upload(up), upload(uu), nxt, upload(v2), upload(et), dt_, h)
    got = nxt.cpu().numpy()
    ref = oracle_mod.wave_step(up, uu, v2, et, R, c, dt_, h)
    check_close(interior(got, R), interior(ref, R), _tol(dtype),
                "random wave case %d" % i)
    check_halo_untouched(got, R, "random wave case %d" % i)


@pytest.mark.parametrize("case", _draw_cases(10, 4242),
                         ids=lambda c: "case%d" % c[0])
def test_random_jacobi(torch_dev, case):
    i, R, dtype, shape, _, _, wseed = case
    sweeps = int(np.random.default_rng(wseed).integers(0, 14))
    name = np.dtype(dtype).name
    log("case %d: jacobi R=%d %s shape %s sweeps %d" %
        (i, R, name, shape, sweeps))
    u = wl.uniform_planes(shape, 5000 + i, -1, 1, dtype=dtype)
    d = B.desc_init("f32" if dtype == np.float32 else "f64", shape, R,
                    B.DIRICHLET_COPY)
    state = upload(u)
    for _ in range(sweeps):
        nxt = sentinel_like(shape, dtype)
        B.stencil3d_apply(d, state, nxt)
        state = nxt
    b0, b1 = upload(u), sentinel_like(shape, dtype)
    res = B.stencil3d_jacobi(d, b0, b1, sweeps)
    assert res is (b0 if sweeps % 2 == 0 else b1)
    got, want = res.cpu().numpy(), state.cpu().numpy()
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), \
        "case %d: %d points differ" % (i, int((got != want).sum()))


def _sponge(shape, R, width, emax=0.1):
    """eta ramping from emax on the outermost interior layer to 0 at depth
    `width` (zero from there inward); the halo gets the outer value."""
    def dist(n):
        i = np.arange(n) - R
        return np.clip(np.minimum(i, n - 2 * R - 1 - i), 0, None)
    dz, dy, dx = (dist(n) for n in shape)
    d = np.minimum(np.minimum(dz[:, None, None], dy[None, :, None]),
                   dx[None, None, :])
    return np.where(d < width, emax * (width - d) / max(width, 1), 0.0)


@pytest.mark.parametrize("seed", range(8))
def test_random_wave_data_regions(oracle_mod, torch_dev, seed):
    """R = 4 wave steps with pml_width on random ragged shapes: the
    data-region launches (two y slabs and the rows between them, eta read
    only near the faces) give the same bits as one launch and match the
    oracle."""
    g = np.random.default_rng(900 + seed)
    R = 4
    dtype = np.float32 if seed % 2 == 0 else np.float64
    iz, iy, ix = (int(g.integers(9, 60)), int(g.integers(9, 80)),
                  int(g.integers(9, 300)))
    shape = (iz + 2 * R, iy + 2 * R, ix + 2 * R)
    width = int(g.integers(1, max(2, min(iz, iy, ix) // 2)))
    pml = width + int(g.integers(0, 3))
    log("case %d: data regions %s shape %s sponge %d pml_width %d" %
        (seed, np.dtype(dtype).name, shape, width, pml))
    up = g.uniform(-1, 1, shape).astype(dtype)
    uu = g.uniform(-1, 1, shape).astype(dtype)
    v2 = g.uniform(1.5e3 ** 2, 4.5e3 ** 2, shape).astype(dtype)
    et = _sponge(shape, R, width).astype(dtype)
    dt_, h = 1e-3, 10.0
    name = "f32" if dtype == np.float32 else "f64"
    outs = []
    for p in (0, pml):
        d = B.desc_init(name, shape, R)
        d.pml_width = p
        nxt = sentinel_like(shape, dtype)
        B.wave_step(d, upload(up), upload(uu), nxt, upload(v2), upload(et),
                    dt_, h)
        outs.append(nxt.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8)), \
        "case %d: %d points differ" % (seed, int((outs[0] != outs[1]).sum()))
    check_halo_untouched(outs[1], R, "data regions case %d" % seed)
    d = B.desc_init(name, shape, R)
    ref = oracle_mod.wave_step(up, uu, v2, et, R, list(d.cx[:R + 1]), dt_, h)
    check_close(interior(outs[1], R), interior(ref, R), _tol(dtype),
                "data regions case %d" % seed)



@pytest.mark.parametrize("case", _draw_cases(12, 5151),
                         ids=lambda c: "case%d" % c[0])
def test_random_pml_step(oracle_mod, torch_dev, case):
    """The PML step (eta-gradient coupling) on random shapes, radii and
    types, with eta drawn per point."""
    i, R, dtype, shape, _, _, wseed = case
    log("case %d: pml step R=%d %s shape %s" %
        (i, R, np.dtype(dtype).name, shape))
    g = np.random.default_rng(wseed)
    up = g.uniform(-1, 1, shape).astype(dtype)
    uu = g.uniform(-1, 1, shape).astype(dtype)
    v2 = g.uniform(1.5e3 ** 2, 4.5e3 ** 2, shape).astype(dtype)
    et = g.uniform(0.0, 0.1, shape).astype(dtype)
    dt_, h = 1e-3, 10.0
    d = B.desc_init("f32" if dtype == np.float32 else "f64", shape, R)
    nxt = sentinel_like(shape, dtype)
    B.wave_step_pml(d, upload(up), upload(uu), nxt, upload(v2), upload(et),
                    dt_, h)
    got = nxt.cpu().numpy()
    ref = oracle_mod.wave_step_pml(up, uu, v2, et, R, list(d.cx[:R + 1]),
                                   dt_, h)
    check_close(interior(got, R), interior(ref, R), _tol(dtype),
                "random pml case %d" % i)
    check_halo_untouched(got, R, "random pml case %d" % i)

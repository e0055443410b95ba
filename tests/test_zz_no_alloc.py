"""wave_run_blocked_noalloc on an MI355X: the time-blocked leapfrog with the
library's static workspace, against the entry point it varies
(wave_run_blocked with caller-owned work buffers) and against wave_run.

Both paths are bit-identical to single steps, so the bar is bit-identity.
Calls run back to back with different grids, the later ones smaller, so a
call finds the workspace holding the previous call's levels in another
layout: anything it read before writing would show."""
import numpy as np
import pytest

from acoustic_wave_propagation_amd import binding as B
from acoustic_wave_propagation_amd import workloads as wl

from gpu_common import device, interior, log, upload

pytestmark = pytest.mark.gpu

DT, H = 1e-3, 10.0


def _fields(shape, seed, r, np_t, halo):
    up = wl.uniform_planes(shape, seed, -1, 1).astype(np_t)
    uc = wl.uniform_planes(shape, seed + 1, -1, 1).astype(np_t)
    m = np.ones(shape, bool)
    m[r:-r, r:-r, r:-r] = False
    up[m] = halo
    uc[m] = halo
    v2 = wl.uniform_planes(shape, seed + 2, 1.5e3 ** 2, 4.5e3 ** 2).astype(np_t)
    et = wl.uniform_planes(shape, seed + 3, 0.0, 0.1).astype(np_t)
    return [upload(a) for a in (up, uc, v2, et)]


def _same(got, want, what, r):
    g, w = interior(got, r), interior(want, r)
    bad = int((g != w).sum())
    assert bad == 0, "%s: %d interior points differ" % (what, bad)


def _case(torch, dtype, shape, r, nsteps, seed, halo=0.0):
    np_t = np.float32 if dtype == "f32" else np.float64
    log("case noalloc %s R=%d %s %d steps" % (dtype, r, shape, nsteps))
    up, uc, v2, et = _fields(shape, seed, r, np_t, halo)
    d = B.desc_init(dtype, shape, r)
    nz, ny, nx = shape
    src = (nx // 2, ny // 3, nz // 2)
    trace = [0.3 * (k + 1) * (-1) ** k for k in range(max(nsteps, 1))]
    a = [up.clone(), uc.clone()]
    old, new = B.wave_run_blocked_noalloc(d, a[0], a[1], v2, et, DT, H,
                                          nsteps, src, trace)
    # the existing entry point, with caller-owned (NaN) work buffers
    bufs = [up.clone(), uc.clone(), torch.full_like(uc, float("nan")),
            torch.full_like(uc, float("nan"))]
    ref_old, ref_new = B.wave_run_blocked(d, *bufs, v2, et, DT, H, nsteps,
                                          src, trace)
    w_old, w_new = B.wave_run(d, up.clone(), uc.clone(), v2, et, DT, H, nsteps,
                              src, trace)
    torch.cuda.synchronize()
    # result placement is wave_run's
    want = (a[0], a[1]) if nsteps % 2 == 0 else (a[1], a[0])
    assert old.data_ptr() == want[0].data_ptr()
    assert new.data_ptr() == want[1].data_ptr()
    _same(new, ref_new, "newest level vs wave_run_blocked", r)
    _same(old, ref_old, "older level vs wave_run_blocked", r)
    _same(new, w_new, "newest level vs wave_run", r)
    _same(old, w_old, "older level vs wave_run", r)
    for t in (old, new):
        h = t.cpu().numpy()
        assert not np.isnan(h).any()
        m = np.ones(shape, bool)
        m[r:-r, r:-r, r:-r] = False
        assert np.all(h[m] == np.array(halo, dtype=np_t)), "halo written"


def test_noalloc_matches_blocked_two_calls():
    """Three calls in a row on one GPU: the largest fp32 field the workspace
    takes (32 MiB), then a smaller grid with a nonzero halo, then a smaller
    fp64 grid; step counts cover passes only, passes plus one to three
    single steps, and a single step alone."""
    import torch
    device()
    B.lib()
    _case(torch, "f32", (512, 128, 128), 4, 6, 2100)
    _case(torch, "f32", (45, 61, 139), 4, 5, 2200, halo=0.25)
    _case(torch, "f64", (37, 40, 71), 4, 7, 2300)
    _case(torch, "f32", (29, 30, 47), 2, 4, 2400)
    _case(torch, "f32", (29, 30, 47), 4, 1, 2500)
    _case(torch, "f32", (29, 30, 47), 4, 0, 2600)


def test_noalloc_rejects_oversized_field():
    """One plane over the limit: ST_ERR_WORKSPACE, nothing enqueued, the
    buffers unchanged."""
    import torch
    device()
    shape = (513, 128, 128)
    d = B.desc_init("f32", shape, 4)
    bufs = [torch.full(shape, 1.5, device=device()) for _ in range(4)]
    with pytest.raises(B.Stencil3DError) as e:
        B.wave_run_blocked_noalloc(d, *bufs, DT, H, 2)
    assert e.value.code == -14
    torch.cuda.synchronize()
    for t in bufs:
        assert bool((t == 1.5).all())

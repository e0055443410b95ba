"""Pins for the oracle's wave step and time loop (CPU only).

The update is u_next = (2u - (1-eta) u_prev + vel2 dt^2 star(u)/h^2)/(1+eta).
Each pin isolates one factor: constant fields isolate where eta enters, a
discrete plane wave (undamped and damped) fixes the factor 2, the sign of
u_prev, dt^2, h^2 and the placement of vel2, and the light cone fixes the
stencil's reach per step.
"""
import cmath
import math

import numpy as np
import pytest

from acoustic_wave_propagation_amd import workloads as wl

EPS = np.finfo(np.float64).eps


def _fields(shape, seed, eta_const=None):
    rng = np.random.default_rng(seed)
    vel2 = rng.uniform(1.5e3 ** 2, 4.5e3 ** 2, shape)
    eta = rng.uniform(0, 0.1, shape) if eta_const is None else \
        np.full(shape, eta_const)
    return vel2, eta


def _inner(a, R=4):
    return a[R:-R, R:-R, R:-R]


def test_only_u_prev(oracle_mod):
    shape = (11, 12, 13)
    vel2, eta = _fields(shape, 1)
    w = oracle_mod.laplacian_weights(4)
    out = oracle_mod.wave_step(np.ones(shape), np.zeros(shape), vel2, eta, 4,
                               w, 1e-3, 10.0)
    want = -(1 - eta) / (1 + eta)
    assert np.abs(_inner(out - want)).max() <= 4 * EPS


def test_only_constant_u(oracle_mod):
    shape = (11, 12, 13)
    vel2, eta = _fields(shape, 2)
    w = oracle_mod.laplacian_weights(4)
    out = oracle_mod.wave_step(np.zeros(shape), np.ones(shape), vel2, eta, 4,
                               w, 1e-3, 10.0)
    want = 2 / (1 + eta)
    # star(const) is zero up to the rounding of the weights
    assert np.abs(_inner(out - want)).max() <= 1e-12


def _symbol(w, th):
    R = len(w) - 1
    return sum(w[0] + 2 * sum(w[k] * math.cos(k * t) for k in range(1, R + 1))
               for t in th)


@pytest.mark.parametrize("eta0", [0.0, 0.07])
def test_discrete_plane_wave(oracle_mod, eta0):
    """With constant vel2 and eta, u^n = Re(A^n) cos(theta.x) solves the
    update exactly when A is a root of (1+eta)A^2 - (2 + r lam)A + (1-eta),
    r = vel2 dt^2/h^2 and lam the rule's symbol.  One step from the exact
    (u^{n-1}, u^n) must give u^{n+1}."""
    R = 4
    shape = (15, 13, 17)
    nz, ny, nx = shape
    Z, Y, X = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx),
                          indexing="ij")
    th = (0.41, 0.83, 1.37)
    space = np.cos(th[0] * X + th[1] * Y + th[2] * Z + 0.2)
    w = oracle_mod.laplacian_weights(R)
    v2, dt, h = 3.1e3 ** 2, 1e-3, 10.0
    r = v2 * dt * dt / (h * h)
    lam = _symbol(w, th)
    a, b, c = 1 + eta0, -(2 + r * lam), 1 - eta0
    A = (-b + cmath.sqrt(b * b - 4 * a * c)) / (2 * a)
    n = 5
    t = [(A ** k).real for k in (n - 1, n, n + 1)]
    out = oracle_mod.wave_step(t[0] * space, t[1] * space,
                               np.full(shape, v2), np.full(shape, eta0), R, w,
                               dt, h)
    err = np.abs(_inner(out - t[2] * space)).max()
    assert err <= 1e-13, err
    # and a wrong reading (u_prev with + sign) is far off
    bad = oracle_mod.wave_step(-t[0] * space, t[1] * space,
                               np.full(shape, v2), np.full(shape, eta0), R, w,
                               dt, h)
    assert np.abs(_inner(bad - t[2] * space)).max() > 1e-2


def test_light_cone_and_axis_tip(oracle_mod):
    """Zero initial state, a point source: after step n (0-based) the field
    vanishes exactly outside the L1 ball of radius R*n about the source, and
    the axis tips at distance R*n are non-zero."""
    R = 4
    n_steps = 3
    N = 2 * R * n_steps + 5
    shape = (N + 2 * R,) * 3
    src = (shape[2] // 2, shape[1] // 2, shape[0] // 2)
    vel2 = np.full(shape, 2.0e3 ** 2)
    eta = np.zeros(shape)
    w = oracle_mod.laplacian_weights(R)
    trace = wl.ricker(np.arange(n_steps) * 1e-3, 15.0)
    Z, Y, X = np.meshgrid(*(np.arange(s) for s in shape), indexing="ij")
    l1 = np.abs(X - src[0]) + np.abs(Y - src[1]) + np.abs(Z - src[2])
    seen = []

    def cb(n, up, u):
        seen.append(n)
        assert np.all(u[l1 > R * n] == 0.0)
        if n > 0:
            ix, iy, iz = src
            for d in (-R * n, R * n):
                assert u[iz, iy, ix + d] != 0.0
                assert u[iz, iy + d, ix] != 0.0
                assert u[iz + d, iy, ix] != 0.0
        # isotropic medium: symmetric under axis permutations about the source
        sub = u[src[2] - R * n:src[2] + R * n + 1,
                src[1] - R * n:src[1] + R * n + 1,
                src[0] - R * n:src[0] + R * n + 1]
        for perm in ((0, 2, 1), (1, 0, 2), (2, 1, 0)):
            assert np.allclose(sub, sub.transpose(perm), rtol=0,
                               atol=1e-12 * np.abs(sub).max())

    oracle_mod.wave_run(np.zeros(shape), np.zeros(shape), vel2, eta, R, w,
                        1e-3, 10.0, n_steps, src=src, src_trace=trace,
                        callback=cb)
    assert seen == list(range(n_steps))


def test_wave_workload_is_stable():
    """The leapfrog is stable when (v dt/h)^2 * max|lambda| <= 4; for the
    order-8 rule in 3D max|lambda| = 3 * 2048/315.  The 1024^3 run's fastest
    medium (4.5 km/s, dt 1 ms, h 10 m) sits just inside."""
    from fractions import Fraction
    import oracle
    c = oracle.second_diff_fractions(4)
    lam_max = 3 * abs(c[0] + 2 * sum(c[k] * (-1) ** k for k in range(1, 5)))
    assert lam_max == 3 * Fraction(2048, 315)
    e = wl.WAVE_1024.extra
    courant = e["vmax"] * e["dt"] / e["h"]
    assert courant ** 2 * float(lam_max) <= 4.0
    assert courant ** 2 * float(lam_max) > 3.9


# ---- the PML kernel's step: eta-gradient coupling --------------------------
# u_next = (2u - (1-eta) u_prev + vel2 dt^2 (star(u) + G)/h^2) / (1+eta),
# G = sum_a (eta(p+e_a) - eta(p-e_a)) (u(p+e_a) - u(p-e_a)) / 4.

def _cubic(rng, scale):
    """Random polynomial of total degree <= 3 as {(i, j, k): coef} for the
    monomial x^i y^j z^k."""
    return {(i, j, k): scale * rng.uniform(-1, 1)
            for i in range(4) for j in range(4) for k in range(4)
            if i + j + k <= 3}


def _poly_eval(p, X, Y, Z, d=(0, 0, 0)):
    """Value of the partial derivative d/dx^d0 d/dy^d1 d/dz^d2 of p."""
    def fall(n, m):  # n (n-1) ... (n-m+1)
        r = 1
        for t in range(m):
            r *= n - t
        return r
    out = np.zeros(X.shape)
    for (i, j, k), c in p.items():
        if i < d[0] or j < d[1] or k < d[2]:
            continue
        f = c * fall(i, d[0]) * fall(j, d[1]) * fall(k, d[2])
        out += f * X ** (i - d[0]) * Y ** (j - d[1]) * Z ** (k - d[2])
    return out


def test_pml_constant_eta_is_the_pointwise_step(oracle_mod):
    """Where eta is the same on a point's six face neighbours the coupling
    vanishes exactly, so with a constant eta field the PML step is the
    pinned pointwise step, bit for bit."""
    shape = (13, 12, 14)
    g = np.random.default_rng(11)
    up, u = g.uniform(-1, 1, shape), g.uniform(-1, 1, shape)
    vel2, _ = _fields(shape, 12)
    eta = np.full(shape, 0.0625)
    for R in (1, 4):
        w = oracle_mod.laplacian_weights(R)
        a = oracle_mod.wave_step(up, u, vel2, eta, R, w, 1e-3, 10.0)
        b = oracle_mod.wave_step_pml(up, u, vel2, eta, R, w, 1e-3, 10.0)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("R", [1, 4])
def test_pml_cubic_fields_closed_form(oracle_mod, R):
    """u and eta cubic polynomials in centred grid coordinates.  The order-2R
    rule is exact on cubics, so star(u) = lap(u); a central difference over
    +-1 of a cubic is exact up to its third derivative: (f(p+e) - f(p-e))/2
    = f' + f'''/6.  Hence G = sum_a (eta'_a + eta'''_a/6)(u'_a + u'''_a/6).
    A dropped term, a wrong sign, a factor 1/2 for 1/4, a difference over
    +-2 (weight 4/6 on the third derivative) or crossed axes each move the
    result far past the bound."""
    shape = (2 * R + 9, 2 * R + 8, 2 * R + 10)
    nz, ny, nx = shape
    g = np.random.default_rng(40 + R)
    Z, Y, X = np.meshgrid(np.arange(nz) - (nz - 1) / 2,
                          np.arange(ny) - (ny - 1) / 2,
                          np.arange(nx) - (nx - 1) / 2, indexing="ij")
    pu = _cubic(g, 1.0)
    pe = _cubic(g, 0.004)
    pe[(0, 0, 0)] = 0.05
    u = _poly_eval(pu, X, Y, Z)
    eta = _poly_eval(pe, X, Y, Z)
    up = g.uniform(-1, 1, shape)
    vel2, _ = _fields(shape, 41)
    dt, h = 1e-3, 10.0
    lap = sum(_poly_eval(pu, X, Y, Z, d) for d in ((2, 0, 0), (0, 2, 0),
                                                   (0, 0, 2)))
    G = 0.0
    for a in range(3):
        d1 = tuple(1 if b == a else 0 for b in range(3))
        d3 = tuple(3 if b == a else 0 for b in range(3))
        G = G + (_poly_eval(pe, X, Y, Z, d1) + _poly_eval(pe, X, Y, Z, d3) / 6) \
            * (_poly_eval(pu, X, Y, Z, d1) + _poly_eval(pu, X, Y, Z, d3) / 6)
    want = (2 * u - (1 - eta) * up + vel2 * dt * dt * (lap + G) / (h * h)) / \
        (1 + eta)
    w = oracle_mod.laplacian_weights(R)
    got = oracle_mod.wave_step_pml(up, u, vel2, eta, R, w, dt, h)
    I = (slice(R, -R),) * 3
    scale = np.abs(u[I]).max() + np.abs(up[I]).max()
    err = np.abs(got[I] - want[I]).max()
    assert err <= 1e-11 * scale, err
    # the coupling is well above that bound: its share of the update
    gshare = np.abs((vel2 * dt * dt * G / (h * h) / (1 + eta))[I]).max()
    assert gshare > 1e-5 * scale
    # and the pointwise step misses it by about that share
    plain = oracle_mod.wave_step(up, u, vel2, eta, R, w, dt, h)
    assert np.abs(plain[I] - want[I]).max() > 0.5 * gshare


def test_pml_run_matches_steps(oracle_mod):
    """wave_run(pml=True) is the PML step in the leapfrog loop."""
    R = 4
    shape = (2 * R + 6,) * 3
    g = np.random.default_rng(5)
    up, u = g.uniform(-1, 1, shape), g.uniform(-1, 1, shape)
    vel2, eta = _fields(shape, 6)
    w = oracle_mod.laplacian_weights(R)
    a, b = np.array(up), np.array(u)
    for _ in range(3):
        n = np.array(a)
        oracle_mod.wave_step_pml(a, b, vel2, eta, R, w, 1e-3, 10.0, out=n)
        a, b = b, n
    rp, ru = oracle_mod.wave_run(up, u, vel2, eta, R, w, 1e-3, 10.0, 3,
                                 pml=True)
    assert np.array_equal(rp, a) and np.array_equal(ru, b)


def test_anisotropic_wave_weights_follow_the_apply(oracle_mod):
    """With per-axis weights the wave step's Laplacian term is the oracle's
    anisotropic stencil: u_next - (2u - (1-eta)u_prev)/(1+eta) equals
    vel2 dt^2 star(u) / (h^2 (1+eta)) with star from star_apply, and the
    axis permutation x <-> z of the fields and weights permutes the result."""
    R = 2
    shape = (11, 12, 13)
    g = np.random.default_rng(91)
    up, u = g.uniform(-1, 1, shape), g.uniform(-1, 1, shape)
    vel2, eta = _fields(shape, 92)
    cx, cy, cz = (g.uniform(-1, 1, R + 1) for _ in range(3))
    dt, h = 1e-3, 10.0
    got = oracle_mod.wave_step(up, u, vel2, eta, R, cx, dt, h, cy=cy, cz=cz)
    st = oracle_mod.star_apply(u, R, cx, cy, cz)
    want = (2 * u - (1 - eta) * up + vel2 * dt * dt * st / (h * h)) / (1 + eta)
    assert np.abs(_inner(got - want, R)).max() <= 1e-12
    perm = (2, 1, 0)
    got_t = oracle_mod.wave_step(up.transpose(perm).copy(),
                                 u.transpose(perm).copy(),
                                 vel2.transpose(perm).copy(),
                                 eta.transpose(perm).copy(), R, cz, dt, h,
                                 cy=cy, cz=cx)
    assert np.abs(_inner(got_t - got.transpose(perm), R)).max() <= 1e-12
    # the PML step with constant eta is the same
    pml = oracle_mod.wave_step_pml(up, u, vel2, np.full(shape, 0.04), R, cx,
                                   dt, h, cy=cy, cz=cz)
    plain = oracle_mod.wave_step(up, u, vel2, np.full(shape, 0.04), R, cx, dt,
                                 h, cy=cy, cz=cz)
    assert np.array_equal(pml, plain)

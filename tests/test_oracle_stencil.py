"""Pins for the oracle's star stencil (CPU only).

Each test checks the oracle against something other than itself: the Taylor
conditions of the weights in exact arithmetic, the exact Laplacian of
polynomials, the known error term one degree above exactness, the closed-form
symbol on plane waves, an exact rational brute force over a dense correlation
box, and an independent library correlation.  Anisotropic weights and
non-cubic grids are used throughout so that a transposed axis or a swapped
extent cannot pass.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.ndimage

EPS = np.finfo(np.float64).eps


def _grid(shape):
    nz, ny, nx = shape
    Z, Y, X = np.meshgrid(np.arange(nz) - nz // 2, np.arange(ny) - ny // 2,
                          np.arange(nx) - nx // 2, indexing="ij")
    return X, Y, Z


def _interior(a, R):
    return a[R:-R, R:-R, R:-R]


# --------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------
@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_weights_taylor_conditions(oracle_mod, R):
    """Order-2R second difference: c0 + 2 sum c_k = 0, sum c_k k^2 = 1,
    sum c_k k^(2m) = 0 for m = 2..R, and the next moment is non-zero."""
    c = oracle_mod.second_diff_fractions(R)
    assert len(c) == R + 1
    assert c[0] + 2 * sum(c[1:]) == 0
    assert sum(c[k] * k ** 2 for k in range(1, R + 1)) == 1
    for m in range(2, R + 1):
        assert sum(c[k] * k ** (2 * m) for k in range(1, R + 1)) == 0
    assert sum(c[k] * k ** (2 * R + 2) for k in range(1, R + 1)) != 0


def test_weights_r4_values_and_tenth_moment(oracle_mod):
    c = oracle_mod.second_diff_fractions(4)
    assert c == (Fraction(-205, 72), Fraction(8, 5), Fraction(-1, 5),
                 Fraction(8, 315), Fraction(-1, 560))
    assert sum(c[k] * k ** 10 for k in range(1, 5)) == -576
    w = oracle_mod.laplacian_weights(4)
    assert w[0] == -205.0 / 72.0 and w[3] == 8.0 / 315.0


# --------------------------------------------------------------------------
# Polynomials: exact up to degree 2R+1 per axis
# --------------------------------------------------------------------------
def _random_poly(rng, deg):
    terms = {}
    for a in range(deg + 1):
        for b in range(deg + 1 - a):
            for c in range(deg + 1 - a - b):
                k = int(rng.integers(-3, 4))
                if k:
                    terms[(a, b, c)] = k
    return terms


def _eval_poly(terms, X, Y, Z):
    out = np.zeros(X.shape, dtype=object)
    for (a, b, c), k in terms.items():
        out = out + k * (X.astype(object) ** a) * (Y.astype(object) ** b) * \
            (Z.astype(object) ** c)
    return out


def _d2(terms, axis):
    out = {}
    for e, k in terms.items():
        if e[axis] >= 2:
            ne = list(e)
            ne[axis] -= 2
            ne = tuple(ne)
            out[ne] = out.get(ne, 0) + k * e[axis] * (e[axis] - 1)
    return out


@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_polynomial_exact(oracle_mod, R):
    rng = np.random.default_rng(10 + R)
    shape = (2 * R + 4, 2 * R + 5, 2 * R + 7)
    X, Y, Z = _grid(shape)
    p = _random_poly(rng, 2 * R + 1)
    u_exact = _eval_poly(p, X, Y, Z)
    u = u_exact.astype(np.float64)
    assert np.all(u.astype(object) == u_exact)  # exactly representable
    w = oracle_mod.laplacian_weights(R)
    sx, sy, sz = 1.0, 2.0, 3.0
    out = oracle_mod.star_apply(u, R, sx * w, sy * w, sz * w)
    want = (sx * _eval_poly(_d2(p, 0), X, Y, Z)
            + sy * _eval_poly(_d2(p, 1), X, Y, Z)
            + sz * _eval_poly(_d2(p, 2), X, Y, Z)).astype(np.float64)
    tol = 64 * EPS * 6 * np.abs(w).sum() * np.abs(u).max()
    err = np.abs(_interior(out, R) - _interior(want, R)).max()
    assert err <= tol, (err, tol)


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_first_inexact_degree(oracle_mod, R, axis):
    """u = t^(2R+2) along one axis: the rule returns the exact second
    derivative plus the constant 2 * sum_k c_k k^(2R+2) (times that axis'
    weight scale), everything else vanishing by the Taylor conditions."""
    shape = (2 * R + 3, 2 * R + 4, 2 * R + 5)
    X, Y, Z = _grid(shape)
    T = (X, Y, Z)[axis].astype(np.float64)
    n = 2 * R + 2
    u = T ** n
    c = oracle_mod.second_diff_fractions(R)
    extra = float(2 * sum(c[k] * k ** n for k in range(1, R + 1)))
    w = oracle_mod.laplacian_weights(R)
    scale = [1.0, 2.0, 3.0]
    out = oracle_mod.star_apply(u, R, scale[0] * w, scale[1] * w,
                                scale[2] * w)
    want = scale[axis] * (n * (n - 1) * T ** (n - 2) + extra)
    tol = 64 * EPS * 6 * np.abs(w).sum() * np.abs(u).max()
    err = np.abs(_interior(out, R) - _interior(want, R)).max()
    assert err <= tol, (err, tol)


@pytest.mark.parametrize("R", [1, 4])
def test_constant_gives_zero(oracle_mod, R):
    w = oracle_mod.laplacian_weights(R)
    for const in (1.0, -3.75, 1e6):
        u = np.full((2 * R + 3, 2 * R + 4, 2 * R + 6), const)
        out = oracle_mod.star_apply(u, R, w)
        bound = 8 * EPS * 3 * np.abs(w).sum() * abs(const)
        assert np.abs(_interior(out, R)).max() <= bound


# --------------------------------------------------------------------------
# Plane waves: the rule's symbol
# --------------------------------------------------------------------------
@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_plane_wave_symbol(oracle_mod, R):
    """cos(k.x + phi) is an eigenfunction: the result is
    lambda * u with lambda = sum_axes (c_a0 + 2 sum_k c_ak cos(k theta_a))."""
    shape = (2 * R + 9, 2 * R + 7, 2 * R + 11)
    nz, ny, nx = shape
    Z, Y, X = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx),
                          indexing="ij")
    th = (0.37, 1.91, 2.73)  # x, y, z
    phi = 0.3
    u = np.cos(th[0] * X + th[1] * Y + th[2] * Z + phi)
    rng = np.random.default_rng(R)
    cs = [rng.uniform(-2, 2, R + 1) for _ in range(3)]
    out = oracle_mod.star_apply(u, R, cs[0], cs[1], cs[2])
    lam = sum(cs[a][0] + 2 * sum(cs[a][k] * math.cos(k * th[a])
                                 for k in range(1, R + 1)) for a in range(3))
    err = np.abs(_interior(out, R) - lam * _interior(u, R)).max()
    assert err <= 1e-13, err


# --------------------------------------------------------------------------
# Exact brute force over a dense box, and an independent library correlation
# --------------------------------------------------------------------------
def _dense_kernel(R, cx, cy, cz):
    """(2R+1)^3 correlation box, zero off the three axes; index [dz,dy,dx]."""
    K = [[[0 for _ in range(2 * R + 1)] for _ in range(2 * R + 1)]
         for _ in range(2 * R + 1)]
    K[R][R][R] = cx[0] + cy[0] + cz[0]
    for k in range(1, R + 1):
        for s in (-1, 1):
            K[R][R][R + s * k] = cx[k]
            K[R][R + s * k][R] = cy[k]
            K[R + s * k][R][R] = cz[k]
    return K


@pytest.mark.parametrize("R,shape", [(1, (8, 8, 8)), (4, (16, 16, 16)),
                                     (2, (9, 11, 13))])
def test_brute_force_rational(oracle_mod, R, shape):
    rng = np.random.default_rng(100 + R)
    u = rng.integers(-5, 6, shape).astype(np.float64)
    fr = oracle_mod.second_diff_fractions(R)
    cx = list(fr)
    cy = [2 * f for f in fr]
    cz = [Fraction(-1, 3) * f for f in fr]
    K = _dense_kernel(R, cx, cy, cz)
    nz, ny, nx = shape
    got = oracle_mod.star_apply(u, R, [float(f) for f in cx],
                                [float(f) for f in cy], [float(f) for f in cz])
    ui = u.astype(np.int64)
    offs = [(dz, dy, dx) for dz, dy, dx in
            itertools.product(range(-R, R + 1), repeat=3)
            if K[dz + R][dy + R][dx + R] != 0]
    assert len(offs) == 6 * R + 1
    worst = 0.0
    for z in range(R, nz - R):
        for y in range(R, ny - R):
            for x in range(R, nx - R):
                s = Fraction(0)
                for dz, dy, dx in offs:
                    s += K[dz + R][dy + R][dx + R] * int(ui[z + dz, y + dy,
                                                            x + dx])
                worst = max(worst, abs(float(Fraction(got[z, y, x]) - s)))
    assert worst <= 1e-13, worst


@pytest.mark.parametrize("R", [1, 3, 4])
def test_matches_scipy_correlate(oracle_mod, R):
    rng = np.random.default_rng(200 + R)
    shape = (2 * R + 11, 2 * R + 6, 2 * R + 17)
    u = rng.uniform(-1, 1, shape)
    cs = [rng.uniform(-1, 1, R + 1) for _ in range(3)]
    K = np.array(_dense_kernel(R, *cs), dtype=np.float64)
    ref = scipy.ndimage.correlate(u, K, mode="constant", cval=0.0)
    got = oracle_mod.star_apply(u, R, *cs)
    err = np.abs(_interior(got, R) - _interior(ref, R)).max()
    assert err <= 1e-14, err


# --------------------------------------------------------------------------
# Boundary modes, input widths, the Jacobi loop
# --------------------------------------------------------------------------
def test_halo_untouched_and_dirichlet(oracle_mod):
    R = 2
    rng = np.random.default_rng(7)
    u = rng.uniform(-1, 1, (9, 10, 12))
    w = oracle_mod.laplacian_weights(R)
    sentinel = np.full(u.shape, 12345.5)
    out = oracle_mod.star_apply(u, R, w, out=sentinel.copy())
    mask = np.ones(u.shape, bool)
    mask[R:-R, R:-R, R:-R] = False
    assert np.all(out[mask] == 12345.5)
    assert np.all(out[~mask] != 12345.5)
    out2 = oracle_mod.star_apply(u, R, w, boundary=oracle_mod.DIRICHLET_COPY,
                                 out=sentinel.copy())
    assert np.array_equal(out2[mask], u[mask])
    assert np.array_equal(out2[~mask], out[~mask])


def test_fp32_input_is_widened_exactly(oracle_mod):
    rng = np.random.default_rng(8)
    u32 = rng.uniform(-1, 1, (12, 11, 10)).astype(np.float32)
    w = oracle_mod.laplacian_weights(4)
    a = oracle_mod.star_apply(u32, 4, w)
    b = oracle_mod.star_apply(u32.astype(np.float64), 4, w)
    assert np.array_equal(a, b)


def test_jacobi_is_repeated_apply(oracle_mod):
    R = 1
    rng = np.random.default_rng(9)
    u = rng.uniform(-1, 1, (10, 9, 11)).astype(np.float32)
    w = oracle_mod.laplacian_weights(R)
    got = oracle_mod.jacobi(u, 3, R, w)
    ref = u.astype(np.float64)
    for _ in range(3):
        ref = oracle_mod.star_apply(ref, R, w,
                                    boundary=oracle_mod.DIRICHLET_COPY)
    assert np.array_equal(got, ref)
    mask = np.ones(u.shape, bool)
    mask[R:-R, R:-R, R:-R] = False
    assert np.array_equal(got[mask], u.astype(np.float64)[mask])


def test_planted_mistakes_fail_pins(oracle_mod):
    """A weight table with one wrong entry, or shifted offsets, must fail the
    polynomial pin -- i.e. the pins can tell a wrong stencil apart."""
    R = 4
    shape = (2 * R + 3, 2 * R + 4, 2 * R + 5)
    X, Y, Z = _grid(shape)
    u = (X.astype(np.float64) ** 4) + 0.5 * Y ** 2
    w = oracle_mod.laplacian_weights(R).copy()
    want = 12 * X.astype(np.float64) ** 2 + 1.0
    ok = oracle_mod.star_apply(u, R, w)
    assert np.abs(_interior(ok - want, R)).max() < 1e-8
    bad = w.copy()
    bad[2] = -bad[2]  # sign slip on one weight
    out = oracle_mod.star_apply(u, R, bad)
    assert np.abs(_interior(out - want, R)).max() > 1e-3
    bad = np.roll(w[1:], 1)  # weights attached to the wrong offsets
    out = oracle_mod.star_apply(u, R, np.concatenate([[w[0]], bad]))
    assert np.abs(_interior(out - want, R)).max() > 1e-3

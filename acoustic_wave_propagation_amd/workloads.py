"""Seeded synthetic workloads for the star stencil and the wave step.

This module is shared by the HIP path's callers (benchmark, tests) and by the
CPU oracle's callers.  It therefore holds only input generation -- shapes,
value distributions, the sponge field, the source time series -- and none of
the method's arithmetic: no stencil weights, no stencil sums, no update rule.

Every array is numpy, C order, shape ``(nz, ny, nx)`` (x innermost), and is
generated plane by plane: plane z of a field comes from its own generator
seeded with ``(seed, stream, z)``.  A z-range of any field can therefore be
produced without materialising the rest, which lets the 1032^3 wave grid be
streamed to the device and lets tests regenerate a small crop of it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# stream ids inside one seed
_S_VALUES, _S_NOISE, _S_POLY, _S_VEL2, _S_UPREV, _S_U = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    shape: tuple            # allocated (nz, ny, nx), halo included
    dtype: str              # "f32" | "f64"
    radius: int
    seed: int
    op: str                 # "apply" | "jacobi" | "wave"
    boundary: str = "halo_untouched"    # | "dirichlet_copy"
    sweeps: int = 1
    values: str = "uniform"             # | "cubic_noise" | "zero"
    extra: dict = field(default_factory=dict)

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float64

    @property
    def interior(self):
        R = self.radius
        return tuple(n - 2 * R for n in self.shape)

    @property
    def interior_points(self) -> int:
        nz, ny, nx = self.interior
        return nx * ny * nz


# The five workloads.  Sizes are allocated extents including the R-wide halo.
R1_64 = Workload("r1_64cube_f32", (64, 64, 64), "f32", 1, 1000, "apply")
R1_JACOBI_512 = Workload("r1_jacobi10_512cube_f32", (512, 512, 512), "f32", 1,
                         1001, "jacobi", boundary="dirichlet_copy", sweeps=10)
R4_512 = Workload("r4_512cube_f32", (520, 520, 520), "f32", 4, 1002, "apply")
R4_RAGGED_F64 = Workload("r4_ragged_1001x603x297_f64", (297, 603, 1001), "f64",
                         4, 1003, "apply", values="cubic_noise")
WAVE_1024 = Workload(
    "wave_r4_1024cube_f32_20steps", (1032, 1032, 1032), "f32", 4, 1004,
    "wave", sweeps=20, values="zero",
    extra=dict(h=10.0, dt=1.0e-3, vmin=1.5e3, vmax=4.5e3, sponge=32,
               eta_max=0.1, f0=15.0))
# Test-only: the wave update on random initial fields in a grid small enough
# that the sponge covers a large share of it (the 1024^3 run never reaches
# its sponge in 20 steps).
WAVE_128_RANDOM = Workload(
    "wave_r4_128cube_f32_random", (136, 136, 136), "f32", 4, 1005, "wave",
    sweeps=20, values="uniform",
    extra=dict(h=10.0, dt=1.0e-3, vmin=1.5e3, vmax=4.5e3, sponge=32,
               eta_max=0.1, f0=15.0))

ALL = [R1_64, R1_JACOBI_512, R4_512, R4_RAGGED_F64, WAVE_1024]
BY_NAME = {w.name: w for w in ALL + [WAVE_128_RANDOM]}


def _plane_rng(seed: int, stream: int, z: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream, z])


def uniform_planes(shape, seed, lo, hi, z0=0, z1=None, dtype=np.float32,
                   stream=_S_VALUES) -> np.ndarray:
    """Planes z0..z1-1 of a field uniform in [lo, hi): drawn in fp64, cast."""
    nz, ny, nx = shape
    z1 = nz if z1 is None else z1
    out = np.empty((z1 - z0, ny, nx), dtype=dtype)
    for z in range(z0, z1):
        out[z - z0] = _plane_rng(seed, stream, z).uniform(lo, hi, (ny, nx))
    return out


def cubic_noise_planes(shape, seed, z0=0, z1=None, noise=1e-3,
                       dtype=np.float64) -> np.ndarray:
    """Random cubic polynomial in normalised coordinates plus uniform noise.

    The 20 coefficients of the monomials xi^a eta^b zeta^c with a+b+c <= 3
    are drawn uniform in [-1, 1) from ``(seed, poly)``; xi = (x - (nx-1)/2) /
    (nx-1) and likewise eta, zeta, so the polynomial is O(1) on the grid.
    The noise is uniform in [-noise, noise), plane-seeded.  Built in fp64.
    """
    nz, ny, nx = shape
    z1 = nz if z1 is None else z1
    rng = np.random.default_rng([seed, _S_POLY])
    exps = [(a, b, c) for a in range(4) for b in range(4) for c in range(4)
            if a + b + c <= 3]
    coef = rng.uniform(-1.0, 1.0, len(exps))
    xi = (np.arange(nx) - (nx - 1) / 2.0) / (nx - 1)
    et = (np.arange(ny) - (ny - 1) / 2.0) / (ny - 1)
    out = np.empty((z1 - z0, ny, nx), dtype=dtype)
    for z in range(z0, z1):
        ze = (z - (nz - 1) / 2.0) / (nz - 1)
        plane = np.zeros((ny, nx))
        for (a, b, c), k in zip(exps, coef):
            plane += k * (ze ** c) * np.outer(et ** b, xi ** a)
        plane += _plane_rng(seed, _S_NOISE, z).uniform(-noise, noise, (ny, nx))
        out[z - z0] = plane
    return out


def cubic_poly_coefficients(seed):
    """The (exponents, coefficients) pairs used by ``cubic_noise_planes``."""
    rng = np.random.default_rng([seed, _S_POLY])
    exps = [(a, b, c) for a in range(4) for b in range(4) for c in range(4)
            if a + b + c <= 3]
    return exps, rng.uniform(-1.0, 1.0, len(exps))


def input_planes(w: Workload, z0=0, z1=None) -> np.ndarray:
    """The stencil input of an apply / jacobi workload (planes z0..z1-1)."""
    if w.values == "uniform":
        return uniform_planes(w.shape, w.seed, -1.0, 1.0, z0, z1, w.np_dtype)
    if w.values == "cubic_noise":
        return cubic_noise_planes(w.shape, w.seed, z0, z1, dtype=w.np_dtype)
    raise ValueError("workload %s has no stencil input" % w.name)


# ---------------------------------------------------------------------------
# Wave workload fields
# ---------------------------------------------------------------------------
def vel2_planes(w: Workload, z0=0, z1=None) -> np.ndarray:
    """Squared velocity in m^2/s^2: uniform in [vmin^2, vmax^2).

    1.5 and 4.5 km/s are converted to m/s so that, with h in metres and dt in
    seconds, vel2*dt^2/h^2 lies in [0.0225, 0.2025].
    """
    e = w.extra
    return uniform_planes(w.shape, w.seed, e["vmin"] ** 2, e["vmax"] ** 2,
                          z0, z1, w.np_dtype, stream=_S_VEL2)


def eta_planes(w: Workload, z0=0, z1=None) -> np.ndarray:
    """Sponge damping: a linear ramp from eta_max on the outermost interior
    layer down to 0 at depth ``sponge`` and beyond.

    With d the distance (in points) from the nearest interior face, eta =
    eta_max * (sponge - d) / sponge for d < sponge, else 0.  Halo points get
    the value of d = 0 (they are never read by the update).
    """
    e = w.extra
    R = w.radius
    nz, ny, nx = w.shape
    z1 = nz if z1 is None else z1
    W, emax = e["sponge"], e["eta_max"]

    def dist(n):  # distance from the nearest interior face along one axis
        i = np.arange(n) - R
        m = n - 2 * R
        return np.clip(np.minimum(i, m - 1 - i), 0, None)

    dx, dy = dist(nx), dist(ny)
    dz = dist(nz)
    dxy = np.minimum(dy[:, None], dx[None, :])
    out = np.empty((z1 - z0, ny, nx), dtype=w.np_dtype)
    for z in range(z0, z1):
        d = np.minimum(dxy, dz[z])
        out[z - z0] = np.where(d < W, emax * (W - d) / W, 0.0)
    return out


def initial_u_planes(w: Workload, which: str, z0=0, z1=None) -> np.ndarray:
    """Initial u_prev / u.  Zero for the point-source run; uniform [-1, 1)
    on the interior (zero halo) for the random-field test."""
    nz, ny, nx = w.shape
    z1 = nz if z1 is None else z1
    if w.values == "zero":
        return np.zeros((z1 - z0, ny, nx), dtype=w.np_dtype)
    stream = _S_UPREV if which == "u_prev" else _S_U
    a = uniform_planes(w.shape, w.seed, -1.0, 1.0, z0, z1, w.np_dtype, stream)
    R = w.radius
    a[:, :R, :] = 0
    a[:, ny - R:, :] = 0
    a[:, :, :R] = 0
    a[:, :, nx - R:] = 0
    for z in range(z0, z1):
        if z < R or z >= nz - R:
            a[z - z0] = 0
    return a


def ricker(t, f0):
    """Ricker wavelet of peak frequency f0, delayed by t0 = 1/f0, amplitude 1:
    (1 - 2 pi^2 f0^2 s^2) exp(-pi^2 f0^2 s^2) with s = t - t0."""
    s = np.asarray(t, dtype=np.float64) - 1.0 / f0
    a = (math.pi * f0 * s) ** 2
    return (1.0 - 2.0 * a) * np.exp(-a)


def source_trace(w: Workload) -> np.ndarray:
    """Values added at the source point after steps n = 0..sweeps-1
    (t = n*dt), fp64."""
    e = w.extra
    return ricker(np.arange(w.sweeps) * e["dt"], e["f0"])


def source_point(w: Workload):
    """Allocated (ix, iy, iz) of the interior centre."""
    R = w.radius
    nz, ny, nx = w.shape
    return (R + (nx - 2 * R) // 2, R + (ny - 2 * R) // 2, R + (nz - 2 * R) // 2)

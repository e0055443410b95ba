"""CPU oracle for the 3D star stencil and the acoustic wave step.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product package
(``acoustic_wave_propagation_amd``) never imports it, and the two share no
code: no kernels, headers, helpers, coefficient tables or pre/post-processing.
The only module both sides see is the seeded input generator, which holds none
of the method's arithmetic.

The arithmetic lives in ``oracle.c`` (plain fp64 loop nests, long-double
accumulation, OpenMP over z planes); this module builds it with gcc, loads it
with ctypes and adds the host loops (Jacobi ping-pong, the wave time loop with
its point source) written out step by step.

Arrays are numpy, C order, shape ``(nz, ny, nx)`` so that x is innermost, as
in "Accelerating High-Order Stencils on GPUs" (gmem kernel description: the
grid is a flat 1D array and coalescing is along the innermost axis X).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

HALO_UNTOUCHED = 0
DIRICHLET_COPY = 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or (
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or (
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64, dp = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                            ctypes.c_double)
        lib.oracle_num_threads.restype = i32
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_star_apply.restype = None
        lib.oracle_star_apply.argtypes = [vp, i32, vp, i64, i64, i64, i32,
                                          vp, vp, vp, i32]
        lib.oracle_wave_step.restype = None
        lib.oracle_wave_step.argtypes = [vp, i32, vp, i32, vp, i32, vp, i32,
                                         vp, i64, i64, i64, i32, vp, vp, vp,
                                         dp, dp]
        lib.oracle_wave_step_pml.restype = None
        lib.oracle_wave_step_pml.argtypes = lib.oracle_wave_step.argtypes
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on (OMP_NUM_THREADS or cores)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Run the oracle's loops on n threads from now on."""
    _load().oracle_set_num_threads(int(n))


# ---------------------------------------------------------------------------
# Weights.  The standard central second-difference weights of order 2R, per
# axis: index 0 is the centre, index k the weight of offsets +k and -k.  The
# pages print none of them; the 7-point rule of the register-tiling notes
# (Fig 8.10) is the R = 1 row with unit spacing.  Kept as exact fractions so
# that the tests can check the Taylor conditions exactly.
# ---------------------------------------------------------------------------
_SECOND_DIFF = {
    1: (Fraction(-2), Fraction(1)),
    2: (Fraction(-5, 2), Fraction(4, 3), Fraction(-1, 12)),
    3: (Fraction(-49, 18), Fraction(3, 2), Fraction(-3, 20), Fraction(1, 90)),
    4: (Fraction(-205, 72), Fraction(8, 5), Fraction(-1, 5), Fraction(8, 315),
        Fraction(-1, 560)),
}


def second_diff_fractions(R: int):
    """Exact per-axis weights (c0, c1, ..., cR) of the order-2R rule."""
    return _SECOND_DIFF[R]


def laplacian_weights(R: int) -> np.ndarray:
    """Per-axis fp64 weights (c0..cR), each the nearest double to the fraction."""
    return np.array([float(f) for f in _SECOND_DIFF[R]], dtype=np.float64)


def _f64flag(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("oracle takes float32 or float64 arrays, got %s" % a.dtype)


def _coef(c, R):
    c = np.ascontiguousarray(np.asarray(c, dtype=np.float64))
    if c.shape != (R + 1,):
        raise ValueError("weights must have R+1 = %d entries" % (R + 1))
    return c


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def star_apply(inp: np.ndarray, R: int, cx, cy=None, cz=None,
               boundary: int = HALO_UNTOUCHED,
               out: np.ndarray | None = None) -> np.ndarray:
    """One application of the radius-R star stencil; returns fp64 ``out``.

    Interior points (whole stencil inside the array) get the weighted sum;
    with ``boundary=DIRICHLET_COPY`` every other point gets the input value,
    with ``HALO_UNTOUCHED`` they keep ``out``'s prior contents (zeros if
    ``out`` is not given).
    """
    inp = np.ascontiguousarray(inp)
    if inp.ndim != 3:
        raise ValueError("input must be 3D (nz, ny, nx)")
    nz, ny, nx = inp.shape
    cx = _coef(cx, R)
    cy = cx if cy is None else _coef(cy, R)
    cz = cx if cz is None else _coef(cz, R)
    if out is None:
        out = np.zeros(inp.shape, dtype=np.float64)
    if out.dtype != np.float64 or not out.flags.c_contiguous or \
            out.shape != inp.shape:
        raise ValueError("out must be a C-contiguous float64 array of the "
                         "input's shape")
    _load().oracle_star_apply(_ptr(inp), _f64flag(inp), _ptr(out), nx, ny, nz,
                              R, _ptr(cx), _ptr(cy), _ptr(cz), int(boundary))
    return out


def jacobi(inp: np.ndarray, sweeps: int, R: int, cx, cy=None, cz=None):
    """Ping-pong sweeps with a fixed Dirichlet boundary.

    Buffer 0 starts as the input, buffer 1 gets the input's outer layer; sweep
    s applies the stencil from buffer s%2 into buffer (s+1)%2.  Returns the
    last written buffer (fp64).
    """
    a = np.array(inp, dtype=np.float64)
    b = np.array(inp, dtype=np.float64)  # outer layer == input's
    for _ in range(sweeps):
        star_apply(a, R, cx, cy, cz, HALO_UNTOUCHED, out=b)
        a, b = b, a
    return a


def wave_step(u_prev, u, vel2, eta, R, c, dt, h, out=None, cy=None, cz=None):
    """One wave step on the interior; returns fp64 ``u_next``.

    ``u_next = (2u - (1-eta) u_prev + vel2 dt^2 star(u)/h^2) / (1+eta)``,
    star with per-axis weights ``c`` (x), ``cy``, ``cz`` (default: ``c``).
    Non-interior points of ``out`` are left as given (zeros by default).
    """
    return _wave(_load().oracle_wave_step, u_prev, u, vel2, eta, R, c, dt, h,
                 out, cy, cz)


def _wave(fn, u_prev, u, vel2, eta, R, c, dt, h, out, cy=None, cz=None):
    arrs = [np.ascontiguousarray(a) for a in (u_prev, u, vel2, eta)]
    shape = arrs[1].shape
    if any(a.shape != shape for a in arrs) or len(shape) != 3:
        raise ValueError("all fields must share one 3D shape")
    nz, ny, nx = shape
    c = _coef(c, R)
    cy = c if cy is None else _coef(cy, R)
    cz = c if cz is None else _coef(cz, R)
    if out is None:
        out = np.zeros(shape, dtype=np.float64)
    if out.dtype != np.float64 or not out.flags.c_contiguous or \
            out.shape != shape:
        raise ValueError("out must be a C-contiguous float64 array of the "
                         "fields' shape")
    up, uu, v2, et = arrs
    fn(_ptr(up), _f64flag(up), _ptr(uu), _f64flag(uu), _ptr(v2), _f64flag(v2),
       _ptr(et), _f64flag(et), _ptr(out), nx, ny, nz, R, _ptr(c), _ptr(cy),
       _ptr(cz), float(dt), float(h))
    return out


def wave_step_pml(u_prev, u, vel2, eta, R, c, dt, h, out=None, cy=None,
                  cz=None):
    """One wave step of the PML kernel on the interior; returns fp64 ``u_next``.

    ``u_next = (2u - (1-eta) u_prev + vel2 dt^2 (star(u) + G)/h^2) / (1+eta)``
    with ``G = sum_a (eta(p+e_a) - eta(p-e_a)) (u(p+e_a) - u(p-e_a)) / 4``,
    the eta-gradient coupling (7-point stencil on eta, halo 1).  Non-interior
    points of ``out`` are left as given (zeros by default).
    """
    return _wave(_load().oracle_wave_step_pml, u_prev, u, vel2, eta, R, c,
                 dt, h, out, cy, cz)


def wave_run(u_prev, u, vel2, eta, R, c, dt, h, nsteps, src=None,
             src_trace=None, callback=None, pml=False):
    """Leapfrog time loop: ``nsteps`` wave steps with a point source.

    After step n's update, ``src_trace[n]`` is added to ``u_next`` at the
    point ``src = (ix, iy, iz)`` (allocated coordinates); then the state
    rotates (u_prev, u) <- (u, u_next).  Each new state starts as a copy of
    the old ``u_prev`` (the two-buffer leapfrog: only the interior is
    rewritten, the halo carries over).  ``callback(n, u_prev, u)`` sees the
    state after each step.  ``pml=True`` takes the PML kernel's step
    (``wave_step_pml``).  Returns the final (u_prev, u), fp64.
    """
    step = wave_step_pml if pml else wave_step
    up = np.array(u_prev, dtype=np.float64)
    uc = np.array(u, dtype=np.float64)
    for n in range(nsteps):
        un = np.array(up)
        step(up, uc, vel2, eta, R, c, dt, h, out=un)
        if src is not None:
            ix, iy, iz = src
            un[iz, iy, ix] += float(src_trace[n])
        up, uc = uc, un
        if callback is not None:
            callback(n, up, uc)
    return up, uc

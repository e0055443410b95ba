"""Analytic traffic, intensity and on-chip footprint of star-stencil kernels
(host only; no GPU, no stencil arithmetic).

Two uses:

* the algorithmic bytes the benchmark divides by (one read and one write per
  field; the star never reads the halo's edges or corners), and
* the blocking models of the pages, so that their printed worked values can
  be checked and the shipped tiles placed beside them.

Sources:

* "Thread Coarsening and Register Tiling" (PMPP chapter 8 notes): the table
  of kernel versions with their OP/B for the seven-point stencil, and the
  table of OP/B and resource formulas.  A seven-point output costs 13 flops
  (7 multiplies, 6 adds); elements are 4 bytes.  T is the input tile side,
  so an order-1 tile yields (T-2)^3 outputs.
* "Accelerating High-Order Stencils on GPUs": the points one 3D block of
  Dx x Dy x Dz fetches with its halo (smem_u description), and the on-chip
  buffers of the 2.5D kernels -- 2R+1 planes of (Dx+2R) x (Dy+2R) points for
  st_smem, one such plane for st_reg (footprint ratio 1 : 2R+1).
"""
from __future__ import annotations

SEVEN_POINT_FLOPS = 13  # 7 multiplies + 6 adds per output, as the notes count


# ---- the PMPP notes' seven-point models ---------------------------------------
def op_per_byte_basic(flops: int = SEVEN_POINT_FLOPS, reads: int = 7,
                      elem: int = 4) -> float:
    """No tiling: every output reads its 7 inputs from global memory."""
    return flops / (reads * elem)


def op_per_byte_tiled(T: int, flops: int = SEVEN_POINT_FLOPS, elem: int = 4,
                      R: int = 1) -> float:
    """Input tile T^3 loaded once, (T-2R)^3 outputs computed from it."""
    return flops * (T - 2 * R) ** 3 / (elem * T ** 3)


def op_per_byte_limit(flops: int = SEVEN_POINT_FLOPS, elem: int = 4) -> float:
    """The tiled intensity as T grows without bound."""
    return flops / elem


def halo_share(T: int, R: int = 1) -> float:
    """Share of a T^3 input tile that is halo (no output of its own)."""
    return 1.0 - ((T - 2 * R) / T) ** 3


def tile_points(T: int, R: int = 1):
    """(input points, output points, halo points) of a T^3 input tile."""
    inp, out = T ** 3, (T - 2 * R) ** 3
    return inp, out, inp - out


def coarsened_tile(T: int, coarsen: int, flops: int = SEVEN_POINT_FLOPS,
                   elem: int = 4, R: int = 1):
    """A T x T block stepping `coarsen` output planes in z: it loads a
    T x T x (coarsen + 2R) input tile and computes (T-2R)^2 x coarsen
    outputs.  Returns (input points, output points, OP/B)."""
    inp = T * T * (coarsen + 2 * R)
    out = (T - 2 * R) ** 2 * coarsen
    return inp, out, flops * out / (elem * inp)


def smem_bytes_coarsened(T: int, elem: int = 4, R: int = 1) -> int:
    """Shared memory of z coarsening: 2R+1 planes of T x T."""
    return (2 * R + 1) * T * T * elem


def smem_bytes_register_tiled(T: int, elem: int = 4) -> int:
    """Shared memory with register tiling: the current plane only."""
    return T * T * elem


def extra_registers_per_block(T: int, R: int = 1) -> int:
    """Registers that hold each thread's z column (2R+1 per thread)."""
    return (2 * R + 1) * T * T


# ---- the high-order paper's blocking models ----------------------------------
def block3d_fetch_points(Dx: int, Dy: int, Dz: int, R: int):
    """(block points, halo points) one 3D block fetches: its own Dx Dy Dz
    points and R-deep slabs on its six faces."""
    return Dx * Dy * Dz, (Dx * Dy + Dx * Dz + Dy * Dz) * R * 2


def st_smem_points(Dx: int, Dy: int, R: int) -> int:
    """On-chip points of st_smem: 2R+1 planes of the tile with its halo."""
    return (2 * R + 1) * (Dx + 2 * R) * (Dy + 2 * R)


def st_reg_points(Dx: int, Dy: int, R: int) -> int:
    """On-chip points of st_reg: the current plane with its halo (the z
    column lives in registers)."""
    return (Dx + 2 * R) * (Dy + 2 * R)


# ---- algorithmic bytes of the library's operations ---------------------------
def apply_bytes(interior, R: int, elem: int) -> int:
    """One stencil application over an interior of (nz, ny, nx) points: the
    interior and its 2R-deep face slabs read once, the interior written
    once."""
    nz, ny, nx = interior
    n = nx * ny * nz
    faces = 2 * R * (ny * nz + nx * nz + nx * ny)
    return elem * (n + faces) + elem * n


def wave_bytes(interior, R: int, elem: int) -> int:
    """One wave step: the apply's bytes for u plus u_prev, vel2 and eta read
    once on the interior."""
    nz, ny, nx = interior
    return apply_bytes(interior, R, elem) + 3 * elem * nx * ny * nz

"""The analytic traffic and footprint model (CPU only) against the values
the pages print, and against brute-force point counts where a page gives
only a formula."""
import itertools
import json
import os

import pytest

from acoustic_wave_propagation_amd import traffic as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "pmpp_seven_point_worked_values.json")


def _model(q, args):
    if q == "halo_share_percent":
        return 100.0 * M.halo_share(**args)
    if q == "coarsened_points":
        return list(M.coarsened_tile(**args)[:2])
    if q == "coarsened_op_per_byte":
        return M.coarsened_tile(**args)[2]
    if q == "tile_points":
        return list(M.tile_points(**args))
    return getattr(M, q)(**args)


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["values"]


@pytest.mark.parametrize("case", _cases(),
                         ids=lambda c: "%s%s" % (c["quantity"], c["args"]))
def test_printed_worked_values(case):
    got = _model(case["quantity"], case["args"])
    want = case["value"]
    if isinstance(want, list):
        assert got == want, case["cite"]
    else:
        assert round(got, case["digits"]) == want, (got, case["cite"])


def test_worked_values_are_consistent_with_each_other():
    # the intensity limit is the tiled intensity of an infinite tile, and
    # z coarsening approaches the same limit as the block and the depth grow
    assert abs(M.op_per_byte_tiled(10 ** 6) - M.op_per_byte_limit()) < 1e-4
    assert M.coarsened_tile(4096, 4096)[2] == pytest.approx(
        M.op_per_byte_limit(), rel=2e-3)
    # register tiling keeps 1/(2R+1) of the coarsened kernel's shared memory
    assert 3 * M.smem_bytes_register_tiled(32) == M.smem_bytes_coarsened(32)


def _brute_block_halo(Dx, Dy, Dz, R):
    """Points outside the block within distance R along one axis of a
    block point: the star's reach, counted one by one."""
    pts = set()
    for x, y, z in itertools.product(range(Dx), range(Dy), range(Dz)):
        for k in range(1, R + 1):
            for p in ((x + k, y, z), (x - k, y, z), (x, y + k, z),
                      (x, y - k, z), (x, y, z + k), (x, y, z - k)):
                if not (0 <= p[0] < Dx and 0 <= p[1] < Dy and 0 <= p[2] < Dz):
                    pts.add(p)
    return len(pts)


@pytest.mark.parametrize("dims,R", [((8, 8, 8), 4), ((8, 8, 8), 1),
                                    ((4, 6, 5), 2), ((16, 8, 4), 3)])
def test_block3d_fetch_matches_a_point_count(dims, R):
    """The smem_u fetch count (block plus R-deep slabs on its six faces,
    no edges or corners) is the set of points the star reaches outside
    the block."""
    blk, halo = M.block3d_fetch_points(*dims, R)
    assert blk == dims[0] * dims[1] * dims[2]
    assert halo == _brute_block_halo(*dims, R)


@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_st_smem_to_st_reg_ratio(R):
    """The high-order paper states the register version keeps 1 : 2R+1 of
    st_smem's on-chip buffer."""
    for Dx, Dy in ((32, 32), (64, 8), (16, 4)):
        assert M.st_smem_points(Dx, Dy, R) == (2 * R + 1) * M.st_reg_points(
            Dx, Dy, R)
        assert M.st_reg_points(Dx, Dy, R) == (Dx + 2 * R) * (Dy + 2 * R)


def test_algorithmic_bytes_match_a_point_count():
    """apply_bytes: the points the star reads (interior plus face slabs,
    counted one by one on a small grid) and the interior written, times
    the element size; wave_bytes adds three interior reads."""
    for (nz, ny, nx), R in (((3, 5, 7), 1), ((6, 5, 9), 2), ((9, 9, 9), 4)):
        read = set()
        for z, y, x in itertools.product(range(nz), range(ny), range(nx)):
            for k in range(0, R + 1):
                for p in ((z + k, y, x), (z - k, y, x), (z, y + k, x),
                          (z, y - k, x), (z, y, x + k), (z, y, x - k)):
                    read.add(p)
        n = nz * ny * nx
        assert M.apply_bytes((nz, ny, nx), R, 4) == 4 * (len(read) + n)
        assert M.wave_bytes((nz, ny, nx), R, 8) == 8 * (len(read) + 4 * n)

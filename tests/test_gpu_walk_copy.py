"""The copy kernels that measure the apply's memory walk (libwalkcopy.so,
bench.py --ceilings) copy exactly what they claim: the interior rows where
they lie, shifted to the row start, or with the rows' halo left as it was."""
import ctypes
import os

import numpy as np
import pytest

from gpu_common import log

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    L = ctypes.CDLL(os.path.join(ROOT, "acoustic_wave_propagation_amd", "libwalkcopy.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.walk_copy_zmarch.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp]
    L.walk_copy_rows.argtypes = [vp, vp, i32, i32, i32, vp]
    return L


@pytest.mark.parametrize("how", ["zmarch256", "zmarch512", "rows"])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_walk_copies(how, mode):
    import torch
    if how != "rows" and mode == 2:
        pytest.skip("the halo rewrite is a row-copy mode")
    L = _lib()
    n, R = 520, 4
    log("case walk copy %s mode %d" % (how, mode))
    g = torch.Generator(device="cuda").manual_seed(3)
    inp = torch.empty((n, n, n), device="cuda").uniform_(-1, 1, generator=g)
    out = torch.full((n, n, n), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    if how == "rows":
        rc = L.walk_copy_rows(inp.data_ptr(), out.data_ptr(), n, R, mode, s)
    else:
        rc = L.walk_copy_zmarch(inp.data_ptr(), out.data_ptr(), n, R,
                                256 if how == "zmarch256" else 512, 4, mode, s)
    assert rc == 0
    torch.cuda.synchronize()
    a, b = inp.cpu().numpy(), out.cpu().numpy()
    want = np.full_like(a, 7.0)
    src = a[R:-R, R:-R, R:-R]
    if mode == 1:
        want[R:-R, R:-R, 0:n - 2 * R] = src
    else:
        want[R:-R, R:-R, R:-R] = src
    assert np.array_equal(b, want)
    # shapes the walk does not tile are refused, nothing launched
    assert L.walk_copy_zmarch(inp.data_ptr(), out.data_ptr(), 500, R, 256, 4, 0, s) == -1

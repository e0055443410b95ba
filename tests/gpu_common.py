"""Shared helpers of the GPU parity tests: device upload of seeded planes,
sentinel fills, tolerance checks.  Imported only by tests marked ``gpu``."""
from __future__ import annotations

import sys

import numpy as np

F32_TOL = 1e-5   # max|gpu - ref| <= F32_TOL * max|ref| per sweep / step
F64_TOL = 1e-12
SENTINEL = -12345.6789


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch.device("cuda:0")


def torch_dtype(np_dtype):
    import torch
    return torch.float32 if np.dtype(np_dtype) == np.float32 else torch.float64


def upload(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def upload_planes(gen, shape, np_dtype, slab=64):
    """Device array filled slab by slab from gen(z0, z1) -> numpy planes."""
    import torch
    t = torch.empty(shape, dtype=torch_dtype(np_dtype), device=device())
    for z0 in range(0, shape[0], slab):
        z1 = min(shape[0], z0 + slab)
        t[z0:z1].copy_(torch.from_numpy(np.ascontiguousarray(gen(z0, z1))))
    return t


def sentinel_like(shape, np_dtype):
    import torch
    return torch.full(shape, SENTINEL, dtype=torch_dtype(np_dtype),
                      device=device())


def interior(a, R):
    return a[R:-R, R:-R, R:-R]


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.abs(ref).max())
    err = float(np.abs(gpu.astype(np.float64) - ref).max())
    return err / scale if scale > 0 else err


def check_close(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str):
    assert np.all(np.isfinite(gpu)), what + ": non-finite output"
    r = rel_err(gpu, ref)
    log("%s: max|err|/max|ref| = %.3e (tol %.0e)" % (what, r, tol))
    assert r <= tol, "%s: relative error %.3e > %.0e" % (what, r, tol)
    return r


def check_halo_untouched(out: np.ndarray, R: int, what: str,
                         value=SENTINEL):
    mask = np.ones(out.shape, bool)
    mask[R:-R, R:-R, R:-R] = False
    want = np.array(value, dtype=out.dtype)
    bad = np.count_nonzero(out[mask] != want)
    assert bad == 0, "%s: %d non-interior points were written" % (what, bad)

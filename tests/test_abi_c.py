"""The C ABI from plain C99 (tests/native/abi_consumer.c): no Python binding,
no torch; device memory from the HIP runtime's C API."""
import os
import runpy
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "native", "abi_consumer")


def _consumer():
    # rebuilt when missing or older than its source or the header
    srcs = [os.path.join(HERE, "native", "abi_consumer.c"),
            os.path.join(os.path.dirname(HERE), "include", "stencil3d.h")]
    if not os.path.exists(EXE) or any(os.path.getmtime(s) > os.path.getmtime(EXE)
                                      for s in srcs):
        runpy.run_path(os.path.join(HERE, "native", "build_consumer.py"),
                       run_name="build_consumer")["build"]()
    return EXE


def test_c_consumer_validation():
    r = subprocess.run([_consumer(), "cpu"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "cpu checks ok" in r.stdout


@pytest.mark.gpu
def test_c_consumer_apply(oracle_mod, tmp_path):
    out = str(tmp_path / "apply.bin")
    r = subprocess.run([_consumer(), "gpu", out], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    shape = (19, 23, 41)
    raw = np.fromfile(out, dtype=np.float32)
    n = int(np.prod(shape))
    assert raw.size == 2 * n
    inp, got = raw[:n].reshape(shape), raw[n:].reshape(shape)
    R = 2
    ref = oracle_mod.star_apply(inp, R, oracle_mod.laplacian_weights(R))
    g, f = got[R:-R, R:-R, R:-R], ref[R:-R, R:-R, R:-R]
    err = np.abs(g - f).max() / np.abs(f).max()
    assert err <= 1e-5, err
    # the halo was zero-filled by the consumer and must stay so
    mask = np.ones(shape, bool)
    mask[R:-R, R:-R, R:-R] = False
    assert not got[mask].any()


@pytest.mark.gpu
def test_c_consumer_blocked_run(oracle_mod, tmp_path):
    """Two leapfrog steps through wave_run_blocked from plain C (R = 4),
    each checked against the oracle's wave step, teacher-forced."""
    out = str(tmp_path / "blocked.bin")
    r = subprocess.run([_consumer(), "blocked", out], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    shape, R = (19, 23, 41), 4
    n = int(np.prod(shape))
    raw = np.fromfile(out, dtype=np.float32)
    assert raw.size == 6 * n
    up, uc, v2, et, l2, l3 = (raw[k * n:(k + 1) * n].reshape(shape)
                              for k in range(6))
    c = oracle_mod.laplacian_weights(R)
    src = (9, 11, 20)  # (z, y, x) of the source at allocated (20, 11, 9)
    inner = (slice(R, -R),) * 3
    for prev, cur, got, val, what in ((up, uc, l2, 0.5, "step 1"),
                                      (uc, None, l3, -0.25, "step 2")):
        if cur is None:  # teacher-forced: the GPU's level 2, zero halo
            cur = np.zeros_like(l2)
            cur[inner] = l2[inner]
        ref = oracle_mod.wave_step(prev, cur, v2, et, R, c, 1e-3, 10.0)
        ref[src] += np.float32(val)
        err = np.abs(got[inner] - ref[inner]).max() / np.abs(ref[inner]).max()
        assert err <= 1e-5, (what, err)
